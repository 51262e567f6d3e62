"""CPU tests of the HIP library's host side: exported symbols, the integer tile
schedule (bit-exact against the oracle's tile enumeration), the useful-pair
count, the config rules and the argument checks that return before any HIP
call.  No kernel runs here.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from sparse_sequence_attention_amd import _capi as C
from sparse_sequence_attention_amd import ops
from sparse_sequence_attention_amd.config import STUConfig, FULL_CAUSAL_K1

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return C.load()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b((?:sla|stu)_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert len(declared) >= 12
    assert set(declared) == set(C.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_public_header_compiles_standalone(lang, tmp_path):
    """include/sla.h is a plain C header: it compiles on its own as C and C++
    (no HIP or torch types in the boundary)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host C/C++ compiler")
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                       "sla.h")
    r = subprocess.run([cc, "-fsyntax-only", "-Wall", "-Werror", "-x", lang, hdr],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings(lib):
    for s in range(7):
        assert lib.sla_status_string(s).decode().startswith("SLA_")


def _rand_case(rng, max_len=700, max_b=5, targets=True):
    B = int(rng.integers(1, max_b + 1))
    lens = [int(x) for x in rng.integers(0, max_len, size=B)]
    tg = [int(rng.integers(0, min(L, 300) + 1)) if (targets and rng.random() < 0.5) else 0
          for L in lens]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return lens, offs, (tg if any(tg) else None)


def _fwd_pairs(rec, bn):
    out = set()
    for r in rec:
        b, r0, n = int(r[0]), int(r[1]), int(r[3])
        for i in range(n):
            lo, hi = int(r[4 + 2 * i]), int(r[5 + 2 * i])
            assert lo % bn == 0
            for c0 in range(lo, hi, bn):
                out.add((b, r0, c0))
    return out


def _bwd_pairs(rec, lens, tg, bm):
    out = set()
    for r in rec:
        b, c0 = int(r[0]), int(r[1])
        U = lens[b] - (tg[b] if tg else 0)
        ha, hb, ta, tb = (int(x) for x in r[4:8])
        if ha < hb:
            for t in range(ha // bm, -(-hb // bm)):
                out.add((b, t * bm, c0))
        if ta < tb:
            for t in range((ta - U) // bm, -(-(tb - U) // bm)):
                out.add((b, U + t * bm, c0))
    return out


@pytest.mark.parametrize("seed", range(12))
def test_schedule_matches_oracle_tiles(seed):
    rng = np.random.default_rng(seed)
    lens, offs, tg = _rand_case(rng)
    k1 = int(rng.choice([0, 1, 2, 5, 64, 130, 256, 1000, FULL_CAUSAL_K1]))
    k2 = int(rng.choice([0, 3, 64, 128, 200]))
    ctx = int(rng.choice([0, 2, 16, 150]))
    bm_f, bn_f = ops.schedule_tile(C.SLA_OP_FWD, 0), ops.schedule_tile(C.SLA_OP_FWD, 1)
    bn_b, bm_b = ops.schedule_tile(C.SLA_OP_BWD, 0), ops.schedule_tile(C.SLA_OP_BWD, 1)

    rec = ops.sla_schedule_host(offs, tg, op=C.SLA_OP_FWD, heads=1, d=128, k1=k1, k2=k2,
                                contextual_len=ctx)
    ref = oracle.tiles(offs, tg, k1, k2, ctx, bm_f, bn_f)
    assert _fwd_pairs(rec, bn_f) == {tuple(map(int, x)) for x in ref}
    # every row tile of every sequence has exactly one record
    n_rows = sum(-(-(L - t) // bm_f) + -(-t // bm_f)
                 for L, t in zip(lens, tg or [0] * len(lens)))
    assert len(rec) == n_rows

    recb = ops.sla_schedule_host(offs, tg, op=C.SLA_OP_BWD, heads=1, d=128, k1=k1, k2=k2,
                                 contextual_len=ctx)
    refb = oracle.tiles(offs, tg, k1, k2, ctx, bm_b, bn_b)
    assert _bwd_pairs(recb, lens, tg, bm_b) == {tuple(map(int, x)) for x in refb}
    # every key tile is owned by records; split tiles' chunks cover disjoint rows
    for b, L in enumerate(lens):
        mine = recb[recb[:, 0] == b]
        assert sorted(set(int(c) for c in mine[:, 1])) == list(range(0, L, bn_b))
        for c0 in set(int(c) for c in mine[:, 1]):
            ch = mine[mine[:, 1] == c0]
            n = int(ch[0, 11])
            assert len(ch) == n and sorted(int(x) for x in ch[:, 10]) == list(range(n))
            U = L - (tg[b] if tg else 0)
            rows = []
            for r in ch:
                rows += list(range(int(r[4]), int(r[5]))) + list(range(int(r[6]), int(r[7])))
            assert len(rows) == len(set(rows))


@pytest.mark.parametrize("seed", range(12))
def test_dkdv_items_cover_the_mask_tiles(seed):
    """The dK/dV items (128-key tiles walking 64-row steps) visit exactly the
    non-empty (64-row, 128-key) tiles of the mask, each once."""
    rng = np.random.default_rng(100 + seed)
    lens, offs, tg = _rand_case(rng)
    k1 = int(rng.choice([0, 1, 2, 5, 64, 130, 256, 1000]))
    k2 = int(rng.choice([0, 3, 64, 128, 200]))
    ctx = int(rng.choice([0, 2, 16, 150]))
    bn, bm = ops.schedule_tile(C.SLA_OP_BWD, 0), ops.schedule_tile(C.SLA_OP_BWD, 1)
    ref = {tuple(map(int, x)) for x in oracle.tiles(offs, tg, k1, k2, ctx, bm, bn)}
    recb = ops.sla_schedule_host(offs, tg, op=C.SLA_OP_BWD, heads=1, d=128, k1=k1, k2=k2,
                                 contextual_len=ctx)
    assert _bwd_pairs(recb, lens, tg, bm) == ref


def test_schedule_long_sequence_splits_prefix_tiles():
    offs = np.array([0, 16384], np.int64)
    rec = ops.sla_schedule_host(offs, None, op=C.SLA_OP_BWD, heads=4, d=128, k1=1024, k2=128,
                                contextual_len=16)
    first = rec[rec[:, 1] == 0]
    assert int(first[0, 11]) > 1            # the global-prefix key tile is split
    band = rec[rec[:, 1] == 8192]
    assert len(band) == 1 and int(band[0, 11]) == 1


@pytest.mark.parametrize("seed", range(8))
def test_count_pairs_host_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    lens, offs, tg = _rand_case(rng, max_len=300)
    for k1, k2, ctx in [(0, 0, 0), (1, 0, 0), (7, 3, 5), (64, 16, 0), (500, 0, 10),
                        (FULL_CAUSAL_K1, 0, 0)]:
        assert ops.count_pairs_host(offs, tg, k1, k2, ctx) == \
            oracle.count_pairs(offs, tg, k1, k2, ctx)


def test_count_pairs_host_rejects_bad_input():
    with pytest.raises(ValueError):
        ops.count_pairs_host(np.array([0, 5], np.int64), np.array([6], np.int32), 4, 0, 0)


# --------------------------------------------------------------------------
# argument checks (return before any HIP call)
# --------------------------------------------------------------------------
def _problem(**kw):
    p = C.SLAProblem()
    p.dtype = kw.get("dtype", C.SLA_BF16)
    p.batch = kw.get("batch", 2)
    p.total_tokens = kw.get("total_tokens", 100)
    p.offsets = kw.get("offsets", 0x10000)
    p.num_targets = None
    p.num_heads = kw.get("heads", 4)
    p.d_qk = kw.get("d", 128)
    p.d_v = kw.get("dv", p.d_qk)
    p.k1, p.k2, p.contextual_len = kw.get("k1", 8), kw.get("k2", 4), kw.get("ctx", 0)
    p.max_seq_len = kw.get("n", 64)
    p.alpha = kw.get("alpha", 1.0)
    return p


FAKE = ctypes.c_void_p(0x20000)  # aligned, never dereferenced on these paths


def _fwd(lib, p, ld=512, ws=FAKE, wsb=1 << 30, q=FAKE):
    return lib.sla_fwd(ctypes.byref(p), q, ld, FAKE, ld, FAKE, ld, FAKE, ld, ws, wsb, None)


def test_fwd_argument_errors(lib):
    assert _fwd(lib, _problem(), q=None) == C.SLA_ERR_NULL
    assert _fwd(lib, _problem(d=96, dv=96), ld=384) == C.SLA_ERR_UNSUPPORTED
    # any pair of widths in {32, 64, 128} is built; others are not
    for dqk, dv in ((96, 64), (64, 96), (128, 256), (16, 32)):
        assert _fwd(lib, _problem(d=dqk, dv=dv), ld=1024) == C.SLA_ERR_UNSUPPORTED, (dqk, dv)
    assert _fwd(lib, _problem(), ld=100) == C.SLA_ERR_INVALID          # ld < H*d
    assert _fwd(lib, _problem(), ld=516) == C.SLA_ERR_UNSUPPORTED      # not 16-byte rows
    assert _fwd(lib, _problem(n=0)) == C.SLA_ERR_INVALID
    assert _fwd(lib, _problem(k1=-1)) == C.SLA_ERR_INVALID
    assert _fwd(lib, _problem(batch=-1)) == C.SLA_ERR_INVALID
    assert _fwd(lib, _problem(offsets=None)) == C.SLA_ERR_NULL
    assert _fwd(lib, _problem(alpha=float("nan"))) == C.SLA_ERR_INVALID
    assert _fwd(lib, _problem(dtype=7)) == C.SLA_ERR_UNSUPPORTED
    assert _fwd(lib, _problem(), ws=None) == C.SLA_ERR_WORKSPACE
    assert _fwd(lib, _problem(), wsb=16) == C.SLA_ERR_WORKSPACE
    assert _fwd(lib, _problem(), q=ctypes.c_void_p(0x20008)) == C.SLA_ERR_UNSUPPORTED
    assert b"16-byte" in lib.sla_last_error()


def test_workspace_size_is_host_only(lib):
    p = _problem(batch=8, total_tokens=106496, k2=128, ctx=16)
    f = lib.sla_workspace_size(ctypes.byref(p), C.SLA_OP_FWD)
    b = lib.sla_workspace_size(ctypes.byref(p), C.SLA_OP_BWD)
    assert 0 < f < b
    assert lib.sla_workspace_size(ctypes.byref(_problem(d=48, dv=48)), C.SLA_OP_FWD) == 0
    assert lib.sla_workspace_size(None, C.SLA_OP_FWD) == 0


def test_backward_workspace_sizes(lib):
    """The smallest backward workspace adds to the forward's schedule only the
    fp32 partial dK|dV sums of the split global-prefix key tiles (at most 4
    tiles of 128 keys per sequence, 16 chunks each): no per-pair storage.
    The default bf16 one adds room for the stored dS: 16 KB per 64-row step
    and 128-key tile and head, bounded from the sizes (at 106,496 tokens in 8
    sequences, K1 = 1024, K2e = 128: 18 steps per key tile of the window, all
    history steps for the prefix tile), and none for fp32 inputs or where it
    would exceed 16 times the inputs' bytes."""
    big = dict(batch=8, total_tokens=106496, k1=1024, k2=128, ctx=16)
    p = _problem(**big)
    fwd = lib.sla_workspace_size(ctypes.byref(p), C.SLA_OP_FWD)
    small = lib.sla_workspace_size(ctypes.byref(p), C.SLA_OP_BWD_RECOMPUTE)
    full = lib.sla_workspace_size(ctypes.byref(p), C.SLA_OP_BWD)
    assert 0 < small - fwd <= 8 * 4 * 16 * 4 * 128 * (128 + 128) * 4 + 256
    tiles, steps = 106496 // 128 + 8, 106496 // 64 + 8
    blocks = tiles * 18 + steps
    assert full - small >= 4 * blocks * 16384
    assert full - small <= 4 * blocks * 16384 + 4 * (tiles + 9) + 1024
    p32 = _problem(dtype=C.SLA_F32, **big)
    assert lib.sla_workspace_size(ctypes.byref(p32), C.SLA_OP_BWD) == \
        lib.sla_workspace_size(ctypes.byref(p32), C.SLA_OP_BWD_RECOMPUTE)
    wide = _problem(**dict(big, k1=16384))  # 16K-key windows: dS beyond 16x the inputs
    assert lib.sla_workspace_size(ctypes.byref(wide), C.SLA_OP_BWD) == \
        lib.sla_workspace_size(ctypes.byref(wide), C.SLA_OP_BWD_RECOMPUTE)
    assert lib.sla_workspace_size(ctypes.byref(p), 3) == 0


def test_out_f32_flag(lib):
    """out_f32 is 0 or 1; with it, output token strides are counted in fp32
    elements (16-byte rows need a multiple of 4), inputs stay bf16."""
    p = _problem()
    p.out_f32 = 2
    assert lib.sla_fwd(ctypes.byref(p), FAKE, 512, FAKE, 512, FAKE, 512, FAKE, 512, FAKE,
                       1 << 30, None) == C.SLA_ERR_INVALID
    assert lib.sla_workspace_size(ctypes.byref(p), C.SLA_OP_FWD) == 0


def test_noalloc_backward_rejects_problems_beyond_its_array(lib):
    """sla_bwd_noalloc checks the smallest backward workspace its problem
    needs against its static array on the host, before any HIP call; an
    invalid problem gets sla_bwd's own error."""
    p = _problem(batch=64, total_tokens=1 << 20, k2=128)
    need = lib.sla_workspace_size(ctypes.byref(p), C.SLA_OP_BWD_RECOMPUTE)
    assert need > C.SLA_NOALLOC_SCRATCH_BYTES
    args = [FAKE, 512] * 7 + [None]
    assert lib.sla_bwd_noalloc(ctypes.byref(p), *args) == C.SLA_ERR_WORKSPACE
    msg = lib.sla_last_error()
    msg = msg.decode() if isinstance(msg, bytes) else msg
    assert "holds at most" in msg and str(need) in msg
    p.out_f32 = 2
    assert lib.sla_bwd_noalloc(ctypes.byref(p), *args) == C.SLA_ERR_INVALID


def test_bwd_and_layer_argument_errors(lib):
    p = _problem()
    st = lib.sla_bwd(ctypes.byref(p), FAKE, 512, FAKE, 512, FAKE, 512, None, 512, FAKE, 512,
                     FAKE, 512, FAKE, 512, FAKE, 1 << 30, None)
    assert st == C.SLA_ERR_NULL
    d = C.STULayerDesc()
    d.attn = _problem(dtype=C.SLA_F32)
    d.hidden, d.ln_eps = 512, 1e-5
    args = [FAKE] * 13
    assert lib.stu_layer_fwd(ctypes.byref(d), *args, 1 << 30, None) == C.SLA_ERR_UNSUPPORTED
    bargs = [FAKE] * 21  # 20 tensors and the workspace
    assert lib.stu_layer_bwd(ctypes.byref(d), *bargs, 1 << 30, None) == C.SLA_ERR_UNSUPPORTED
    d.attn = _problem()
    d.hidden = 200
    assert lib.stu_layer_fwd(ctypes.byref(d), *args, 1 << 30, None) == C.SLA_ERR_UNSUPPORTED
    assert lib.stu_layer_bwd(ctypes.byref(d), *bargs, 1 << 30, None) == C.SLA_ERR_UNSUPPORTED
    d.hidden = 512
    bargs_null_dx = [FAKE] * 11 + [None] + [FAKE] * 9
    assert lib.stu_layer_bwd(ctypes.byref(d), *bargs_null_dx, 1 << 30, None) == C.SLA_ERR_NULL
    assert lib.stu_truncate(2, 10, FAKE, None, 1, 0, FAKE, 512, 1, FAKE, None, None, None, 10,
                            None) == C.SLA_ERR_INVALID


# --------------------------------------------------------------------------
# config rules (torcheasyrec page)
# --------------------------------------------------------------------------
def test_mfma_probe_argument_errors(lib):
    import ctypes
    d = ctypes.c_double(0.0)
    assert lib.sla_probe_mfma_peak(4096, FAKE, 1 << 20, None, ctypes.byref(d),
                                   None) == C.SLA_ERR_NULL
    assert lib.sla_probe_mfma_peak(4096, None, 1 << 20, ctypes.byref(d), ctypes.byref(d),
                                   None) == C.SLA_ERR_NULL
    assert lib.sla_probe_mfma_peak(0, FAKE, 1 << 20, ctypes.byref(d), ctypes.byref(d),
                                   None) == C.SLA_ERR_INVALID
    assert lib.sla_probe_mfma_peak((1 << 20) + 1, FAKE, 1 << 20, ctypes.byref(d),
                                   ctypes.byref(d), None) == C.SLA_ERR_INVALID


def test_issue_probe_argument_errors(lib):
    import ctypes
    ms = (ctypes.c_double * 7)()
    assert lib.sla_probe_issue_rates(4096, FAKE, 1 << 20, None, 7, None) == C.SLA_ERR_NULL
    assert lib.sla_probe_issue_rates(4096, None, 1 << 20, ms, 7, None) == C.SLA_ERR_NULL
    assert lib.sla_probe_issue_rates(4096, FAKE, 1 << 20, ms, 6, None) == C.SLA_ERR_INVALID
    assert lib.sla_probe_issue_rates(0, FAKE, 1 << 20, ms, 7, None) == C.SLA_ERR_INVALID


def test_stu_config_rules():
    c = STUConfig(sla_k1=256, sla_k2=32, contextual_seq_len=64)
    assert c.sla_enabled and c.effective_k2 == 64
    off = STUConfig(sla_k1=0, sla_k2=0)
    assert not off.sla_enabled and off.kernel_k1 == FULL_CAUSAL_K1
    with pytest.raises(ValueError):
        STUConfig(attn_truncation_split_layer=2)
    with pytest.raises(ValueError):
        STUConfig(attn_truncation_tail_len=512)
    # example: 4 layers, split 2 -> layers 2..3 see the truncated sequence
    t = STUConfig(attn_num_layers=4, attn_truncation_split_layer=2, attn_truncation_tail_len=512)
    assert [t.layer_is_truncated(i) for i in range(4)] == [False, False, True, True]


def test_candidate_scoring_argument_errors(lib):
    p = _problem()
    cand = FAKE

    def call(p, cand=cand, total=64, k=FAKE, ldq=512, ws=FAKE):
        return lib.sla_fwd_candidates(ctypes.byref(p), cand, total, k, 512, FAKE, 512, FAKE, ldq,
                                      FAKE, 512, FAKE, 512, FAKE, 512, ws, 1 << 30, None)

    assert call(_problem(dtype=C.SLA_F32)) == C.SLA_ERR_UNSUPPORTED   # bf16 only
    pt = _problem()
    pt.num_targets = 0x30000
    assert call(pt) == C.SLA_ERR_INVALID                               # history has no targets
    assert call(p, total=-1) == C.SLA_ERR_INVALID
    assert call(p, cand=None) == C.SLA_ERR_NULL
    assert call(p, k=None) == C.SLA_ERR_NULL                           # history keys needed
    assert call(p, ldq=100) == C.SLA_ERR_INVALID                       # ld < H*d
    assert call(p, ws=None) == C.SLA_ERR_WORKSPACE
    assert call(p, total=0) == C.SLA_OK                                # nothing to score
    # workspace covers the larger of the history and candidate row counts
    small = lib.sla_fwd_candidates_workspace_size(ctypes.byref(p), 10)
    big = lib.sla_fwd_candidates_workspace_size(ctypes.byref(p), 100000)
    assert 0 < small <= big


def test_fp8_argument_errors(lib):
    assert lib.stu_quantize_rows_fp8(FAKE, 4, 24, FAKE, FAKE, None) == C.SLA_ERR_UNSUPPORTED
    assert lib.stu_quantize_rows_fp8(FAKE, 4, 4096, FAKE, FAKE, None) == C.SLA_ERR_UNSUPPORTED
    assert lib.stu_quantize_rows_fp8(None, 4, 512, FAKE, FAKE, None) == C.SLA_ERR_NULL
    assert lib.stu_quantize_rows_fp8(FAKE, -1, 512, FAKE, FAKE, None) == C.SLA_ERR_INVALID
    assert lib.stu_quantize_rows_fp8(None, 0, 512, None, None, None) == C.SLA_OK
    d = C.STULayerDesc()
    d.attn = _problem()
    d.hidden, d.ln_eps = 512, 1e-5
    args = [FAKE] * 15
    args[11] = ctypes.c_void_p(0x40000)                                # out (must not alias x)
    assert lib.stu_layer_fwd_fp8(ctypes.byref(d), *args, 0, None) == C.SLA_ERR_WORKSPACE
    nul = list(args)
    nul[4] = None                                                      # w_uvqk_scale
    assert lib.stu_layer_fwd_fp8(ctypes.byref(d), *nul, 1 << 30, None) == C.SLA_ERR_NULL
    d.attn = _problem(heads=1, d=64)                                   # H*d_v = 64
    assert lib.stu_layer_fwd_fp8(ctypes.byref(d), *args, 1 << 30, None) == C.SLA_ERR_UNSUPPORTED


def test_gather_targets_argument_errors(lib):
    def call(ld=1024, col=0, hidden=512, tg=FAKE, toffs=FAKE, dtype=C.SLA_BF16):
        return lib.stu_gather_targets(2, 100, FAKE, tg, FAKE, hidden, dtype, toffs, FAKE, ld, col,
                                      100, None)
    assert call(toffs=None) == C.SLA_ERR_NULL
    assert call(tg=None) == C.SLA_ERR_NULL
    assert call(col=600) == C.SLA_ERR_INVALID                          # past ld_out
    assert call(hidden=12) == C.SLA_ERR_UNSUPPORTED                    # not 16-byte rows
    assert call(col=4) == C.SLA_ERR_UNSUPPORTED                        # misaligned column block
    assert call(dtype=7) == C.SLA_ERR_UNSUPPORTED


def test_truncated_token_count_on_the_host_matches_the_oracle():
    """stu_stack_fwd's host-side count of the truncated layout (used instead
    of reading new_offsets[B] back) equals the oracle truncation's total."""
    import numpy as np
    import oracle
    from sparse_sequence_attention_amd.stack import truncated_tokens_host
    rng = np.random.default_rng(7)
    for _ in range(20):
        B = int(rng.integers(1, 12))
        lens = [int(v) for v in rng.integers(0, 400, size=B)]
        tg = [int(rng.integers(0, L + 1)) for L in lens]
        ctx, tail = int(rng.integers(0, 20)), int(rng.integers(1, 200))
        offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        new_offs, _ = oracle.truncate(offs, tg, ctx, tail)
        assert truncated_tokens_host(lens, tg, ctx, tail) == int(new_offs[-1])
        new_offs, _ = oracle.truncate(offs, None, ctx, tail)
        assert truncated_tokens_host(lens, None, ctx, tail) == int(new_offs[-1])


def test_binding_checks_every_head_width(monkeypatch):
    """Q, K (and dQ, dK) share the width d_qk, V, dO, O (and dV) the width
    d_v: the shape check rejects a tensor of another width (the library would
    read its heads at the wrong column offsets), and every entry point asks
    for the right width of each tensor.  Host tensors suffice: the calls are
    stopped before the library."""
    import torch
    bf = torch.bfloat16
    t = lambda w: torch.zeros((4, 2, w), dtype=bf)  # noqa: E731
    with pytest.raises(ValueError, match=r"k: expected shape \[T=4, H=2, 64\]"):
        ops._head_tensor("k", t(128), 4, 2, bf, 64)

    seen = {}

    class Stop(Exception):
        pass

    def record(name, x, T, H, dtype, width):
        seen[name] = (tuple(x.shape), width)
        return H * width

    def stop(*a, **k):
        raise Stop

    monkeypatch.setattr(ops, "_head_tensor", record)
    monkeypatch.setattr(ops, "make_problem", stop)
    offs = torch.tensor([0, 4], dtype=torch.int64)
    kw = dict(k1=8, k2=0, max_seq_len=4)
    calls = [
        lambda: ops.sla_fwd(t(64), t(64), t(32), offs, **kw),
        lambda: ops.sla_bwd(t(64), t(64), t(32), t(32), offs, **kw),
        lambda: ops.sla_bwd_noalloc(t(64), t(64), t(32), t(32), offs, dq=t(64), dk=t(64),
                                    dv=t(32), **kw),
        lambda: ops.sla_fwd_candidates(t(64), t(32), offs, t(64), t(64), t(32), offs, **kw),
    ]
    for call in calls:
        seen.clear()
        with pytest.raises(Stop):
            call()
        assert len(seen) >= 4
        for name, (shape, width) in seen.items():
            assert shape[2] == width, (name, shape, width)
            want = 32 if name in ("v", "v_hist", "v_c", "dout", "dv", "out") else 64
            assert width == want, (name, width)


def _ws_problem(offs, tg, heads, d, dv, k1, k2, ctx):
    p = _problem(batch=len(offs) - 1, total_tokens=int(offs[-1]), heads=heads, d=d, dv=dv, k1=k1,
                 k2=k2, ctx=ctx)
    if tg is not None:
        p.num_targets = ctypes.c_void_p(0x30000)  # only its presence counts for the size
    return p


@pytest.mark.parametrize("seed", range(16))
def test_stored_ds_blocks(seed, lib):
    """The stored-dS blocks: exactly the (64-row step, 128-key tile) pairs of
    the mask that hold a visible pair (brute force), in the order the dK/dV
    kernel numbers them (sequence, key tile, history then target steps); the
    dK/dV items' steps land on distinct blocks of their own tile; a row half
    of a dQ item that finds no block for a 64-key step sees none of its keys;
    and the workspace bound holds every block."""
    rng = np.random.default_rng(700 + seed)
    lens, offs, tg = _rand_case(rng, max_len=900 if seed % 4 else 2600)
    k1 = int(rng.choice([0, 1, 2, 5, 64, 130, 256, 1000, FULL_CAUSAL_K1]))
    k2 = int(rng.choice([0, 3, 64, 128, 200, 300]))
    ctx = int(rng.choice([0, 2, 16, 150]))
    blocks = ops.ds_blocks_host(offs, tg, k1=k1, k2=k2, contextual_len=ctx)
    triples = [tuple(map(int, x)) for x in blocks]
    assert len(set(triples)) == len(triples)
    ref = {tuple(map(int, x)) for x in oracle.tiles(offs, tg, k1, k2, ctx, 64, 128)}
    assert set(triples) == ref
    U = [L - (tg[b] if tg else 0) for b, L in enumerate(lens)]
    order = [(b, c0, m0 >= U[b], m0) for b, m0, c0 in triples]
    assert order == sorted(order)
    index = {t: i for i, t in enumerate(triples)}
    first = {}
    for i, (b, m0, c0) in enumerate(triples):
        first.setdefault((b, c0), i)

    # dK/dV items: step t of an item is block t + (history ? dh : dt) of its tile
    recb = ops.sla_schedule_host(offs, tg, op=C.SLA_OP_BWD, heads=1, d=128, k1=k1, k2=k2,
                                 contextual_len=ctx)
    written = []
    for r in recb:
        b, c0 = int(r[0]), int(r[1])
        ha, hb, ta, tb = (int(x) for x in r[4:8])
        h_first = ha // 64 if ha < hb else 0
        nh = (-(-hb // 64) - h_first) if ha < hb else 0
        t_first = (ta - U[b]) // 64 if ta < tb else 0
        nt = (-(-(tb - U[b]) // 64) - t_first) if ta < tb else 0
        tile = [t for t in triples if t[0] == b and t[2] == c0]
        th = [t for t in tile if t[1] < U[b]]
        ts_h_first = th[0][1] // 64 if th else 0
        ts_nh = len(th)
        tt = [t for t in tile if t[1] >= U[b]]
        ts_t_first = (tt[0][1] - U[b]) // 64 if tt else 0
        for t in range(nh + nt):
            m0 = (h_first + t) * 64 if t < nh else U[b] + (t_first + t - nh) * 64
            blk = t + (h_first - ts_h_first if t < nh else ts_nh + t_first - nh - ts_t_first)
            assert 0 <= blk < len(tile)
            assert index[(b, m0, c0)] == first[(b, c0)] + blk
            written.append((b, m0, c0))
    assert sorted(written) == sorted(triples)

    # dQ items: a row half without a block for a key step sees none of its keys
    recf = ops.sla_schedule_host(offs, tg, op=C.SLA_OP_FWD, heads=1, d=128, k1=k1, k2=k2,
                                 contextual_len=ctx)
    masks = {}
    for r in recf:
        b, r0, r1, n = int(r[0]), int(r[1]), int(r[2]), int(r[3])
        if b not in masks:
            masks[b] = oracle.mask_dense(lens[b], tg[b] if tg else 0, k1, k2, ctx)
        for i in range(n):
            for c0 in range(int(r[4 + 2 * i]), int(r[5 + 2 * i]), 64):
                for sg in range(2):
                    m0 = r0 + 64 * sg
                    if m0 >= r1 or (b, m0, c0 - c0 % 128) in index:
                        continue
                    assert not masks[b][m0:min(m0 + 64, r1), c0:c0 + 64].any()

    # the stored-dS workspace holds every block (one head: 16 KB each)
    for heads, d in ((1, 128), (4, 64)):
        p = _ws_problem(offs, tg, heads, d, d, k1, k2, ctx)
        full = lib.sla_workspace_size(ctypes.byref(p), C.SLA_OP_BWD)
        small = lib.sla_workspace_size(ctypes.byref(p), C.SLA_OP_BWD_RECOMPUTE)
        assert small > 0 and full >= small
        if full > small:
            assert full - small >= heads * len(triples) * 64 * 128 * 2


def test_ds_blocks_host_rejects_bad_input(lib):
    """sla_ds_blocks_host: invalid problems and layouts return -1 with a
    message; an empty batch has no blocks."""
    offs = np.array([0, 100, 50], dtype=np.int64)   # decreasing: a negative length
    with pytest.raises(ValueError):
        ops.ds_blocks_host(offs, None, k1=8, k2=0)
    with pytest.raises(ValueError):
        ops.ds_blocks_host(np.array([0, 10], np.int64), np.array([11], np.int32), k1=8, k2=0)
    with pytest.raises(ValueError):
        ops.ds_blocks_host(np.array([0, 10], np.int64), None, k1=-1, k2=0)
    assert len(ops.ds_blocks_host(np.array([0], np.int64), None, k1=8, k2=0)) == 0
    assert lib.sla_ds_blocks_host(None, None, None, None, 0) == -1
