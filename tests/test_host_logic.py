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
def test_stored_ds_rows_match_dkdv_blocks(seed):
    """The 64-row dQ items that read stored dS visit exactly the (row tile, key
    tile) blocks the dK/dV items write: both are the non-empty tiles of the
    mask at 64 rows x 128 keys, and the slot order is the record's range order."""
    rng = np.random.default_rng(100 + seed)
    lens, offs, tg = _rand_case(rng)
    k1 = int(rng.choice([0, 1, 2, 5, 64, 130, 256, 1000]))
    k2 = int(rng.choice([0, 3, 64, 128, 200]))
    ctx = int(rng.choice([0, 2, 16, 150]))
    bm, bn = ops.schedule_tile(C.SLA_OP_DQ, 0), ops.schedule_tile(C.SLA_OP_DQ, 1)
    assert (bm, bn) == (ops.schedule_tile(C.SLA_OP_BWD, 1), ops.schedule_tile(C.SLA_OP_BWD, 0))
    rec = ops.sla_schedule_host(offs, tg, op=C.SLA_OP_DQ, heads=1, d=128, k1=k1, k2=k2,
                                contextual_len=ctx)
    ref = {tuple(map(int, x)) for x in oracle.tiles(offs, tg, k1, k2, ctx, bm, bn)}
    assert _fwd_pairs(rec, bn) == ref
    recb = ops.sla_schedule_host(offs, tg, op=C.SLA_OP_BWD, heads=1, d=128, k1=k1, k2=k2,
                                 contextual_len=ctx)
    assert _bwd_pairs(recb, lens, tg, bm) == ref
    n_rows = sum(-(-(L - t) // bm) + -(-t // bm) for L, t in zip(lens, tg or [0] * len(lens)))
    assert len(rec) == n_rows


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
    assert _fwd(lib, _problem(dv=64), ld=512) == C.SLA_ERR_UNSUPPORTED
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


def test_bwd_dq_mode(lib):
    # stored dS: bf16, d in {64, 128} and at most 32 key tiles per 64-row tile
    big = dict(batch=8, total_tokens=106496, k1=1024, k2=128, ctx=16)
    assert lib.sla_bwd_dq_mode(ctypes.byref(_problem(**big))) == 1
    assert lib.sla_bwd_dq_mode(ctypes.byref(_problem(d=64, **big))) == 1
    assert lib.sla_bwd_dq_mode(ctypes.byref(_problem(d=32, **big))) == 0
    assert lib.sla_bwd_dq_mode(ctypes.byref(_problem(dtype=C.SLA_F32, **big))) == 0
    # full causal over 5000 tokens: 40 key tiles per row tile -> recompute
    full = dict(batch=1, total_tokens=5000, k1=2**31 - 1, k2=0)
    assert lib.sla_bwd_dq_mode(ctypes.byref(_problem(**full))) == 0
    assert lib.sla_bwd_dq_mode(ctypes.byref(_problem(d=48, dv=48))) == -1
    assert lib.sla_bwd_dq_mode(None) == -1
    # the stored blocks are part of the backward workspace
    p1, p0 = _problem(**big), _problem(dtype=C.SLA_F32, **big)
    extra = lib.sla_workspace_size(ctypes.byref(p1), C.SLA_OP_BWD) - \
        lib.sla_workspace_size(ctypes.byref(p1), C.SLA_OP_FWD)
    extra0 = lib.sla_workspace_size(ctypes.byref(p0), C.SLA_OP_BWD) - \
        lib.sla_workspace_size(ctypes.byref(p0), C.SLA_OP_FWD)
    assert extra - extra0 >= 106496 * 4 * 128 * 2  # at least the fp16 copy of K


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
    assert lib.sla_probe_mfma_peak(4096, None, ctypes.byref(d), None) == C.SLA_ERR_NULL
    assert lib.sla_probe_mfma_peak(0, ctypes.byref(d), ctypes.byref(d), None) == C.SLA_ERR_INVALID
    assert lib.sla_probe_mfma_peak((1 << 20) + 1, ctypes.byref(d), ctypes.byref(d),
                                   None) == C.SLA_ERR_INVALID


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
