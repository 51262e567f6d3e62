"""SLA with rectangular heads, d_qk != d_v (the boundary's separate Q / K and
V widths; the pages' STU configuration names them attention_dim and
hidden_dim): forward and backward of the bf16 path (fp32 outputs at the raw
bar, bf16 outputs at the storage-aware bar) and of the fp32 path, against
the fp64 oracle, element by element.  The cases cover targets, a global
prefix long enough to be split into chunk partials (the reduce kernel's
[dK | dV] rows of width d_qk + d_v), ragged tails and empty sequences.
Bars as in the square-head tests."""
import numpy as np
import pytest
import torch

import oracle
import sparse_sequence_attention_amd as sla
from synthetic import make_sla_workload
from tests._helpers import assert_close_bf16, assert_close_f32, assert_close_raw

pytestmark = pytest.mark.gpu
DEV = "cuda"

# lengths, targets, k1, k2, ctx, d_qk, d_v
CASES = [
    ([37, 64], None, 8, 4, 2, 64, 128),
    ([1, 700, 129, 0, 256], None, 130, 64, 8, 128, 64),
    ([513, 64, 1000], [17, 64, 200], 100, 16, 8, 64, 128),
    ([2500, 600], [0, 16], 300, 128, 16, 128, 64),   # prefix tile split into chunks
    # one width 32: the dK/dV stage of Q and dO rows is not a whole number of
    # DMA rounds and carries padding
    ([700, 129, 1], [8, 0, 0], 96, 16, 4, 32, 64),
    ([2200, 300], None, 200, 64, 8, 64, 32),         # prefix tile split into chunks
    ([450, 64], [32, 0], 64, 8, 2, 32, 128),
    ([900, 0, 77], None, 128, 32, 8, 128, 32),
]
MODES = ["bf16o32", "bf16", "f32"]


def _work(case, mode, seed):
    lens, tg, k1, k2, ctx, dqk, dv = CASES[case]
    w = make_sla_workload("jagged_2k", seed=seed, lengths=lens, num_targets=tg, heads=2, d=dqk,
                          d_v=dv, k1=k1, k2=k2, contextual_len=ctx, max_seq_len=max(lens),
                          dtype="f32" if mode == "f32" else "bf16", with_dout=True)
    print(f"[case] rect {case} {mode} lens={lens} dqk={dqk} dv={dv}", flush=True)
    dt = torch.float32 if mode == "f32" else torch.bfloat16
    t = lambda a: torch.from_numpy(a).to(DEV).to(dt)  # noqa: E731
    offs = torch.from_numpy(w.offsets).to(DEV)
    tgd = None if w.num_targets is None else torch.from_numpy(w.num_targets).to(DEV)
    kw = dict(k1=w.k1, k2=w.k2, contextual_len=w.contextual_len, max_seq_len=w.max_seq_len)
    return w, (t(w.q), t(w.k), t(w.v), t(w.dout), offs, tgd), kw


def _check(mode, got, ref, what):
    g = got.float().cpu().numpy().astype(np.float64)
    if mode == "f32":
        return assert_close_f32(g, ref, what)
    if mode == "bf16o32":
        return assert_close_raw(g, ref, what)
    return assert_close_bf16(g, ref, what)


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("mode", MODES)
def test_rect_fwd(case, mode):
    w, (q, k, v, _, offs, tgd), kw = _work(case, mode, 40 + case)
    o = sla.sla_fwd(q, k, v, offs, tgd, out_dtype=torch.float32 if mode == "bf16o32" else None,
                    **kw)
    torch.cuda.synchronize()
    assert tuple(o.shape) == tuple(w.v.shape)
    ref = oracle.sla_fwd(w.q, w.k, w.v, w.offsets, w.num_targets, w.k1, w.k2, w.contextual_len,
                         w.max_seq_len)
    _check(mode, o, ref, "O")


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("mode", MODES)
def test_rect_bwd(case, mode):
    w, (q, k, v, do, offs, tgd), kw = _work(case, mode, 50 + case)
    dq, dk, dv = sla.sla_bwd(q, k, v, do, offs, tgd,
                             grad_dtype=torch.float32 if mode == "bf16o32" else None, **kw)
    torch.cuda.synchronize()
    assert tuple(dq.shape) == tuple(w.q.shape) and tuple(dv.shape) == tuple(w.v.shape)
    rq, rk, rv = oracle.sla_bwd(w.q, w.k, w.v, w.dout, w.offsets, w.num_targets, w.k1, w.k2,
                                w.contextual_len, w.max_seq_len)
    _check(mode, dq, rq, "dQ")
    _check(mode, dk, rk, "dK")
    _check(mode, dv, rv, "dV")


def test_rect_bwd_is_deterministic():
    w, (q, k, v, do, offs, tgd), kw = _work(3, "bf16", 60)
    a = sla.sla_bwd(q, k, v, do, offs, tgd, **kw)
    b = sla.sla_bwd(q, k, v, do, offs, tgd, **kw)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _stu_rect(dqk, dv, seed=2):
    """One STU layer with attention_dim d_qk and hidden_dim d_v (H = 2,
    D = 256): Xavier-uniform projections of the rectangular widths, LayerNorm
    weights around 1, biases, a ragged batch with targets."""
    from synthetic import bf16_round_f32, make_stack_workload
    sw = make_stack_workload(seed=seed, lengths=[300, 129, 500, 1], layers=1, num_targets=8,
                             hidden=256, heads=2, contextual_len=4, k1=96, k2=16)
    H, D = 2, 256
    nw, nu = 2 * H * dv + 2 * H * dqk, H * dv
    rng = np.random.default_rng(seed + 7)
    a1, a2 = np.sqrt(6.0 / (D + nw)), np.sqrt(6.0 / (nu + D))
    host = dict(ln1_w=1.0 + 0.2 * rng.standard_normal(D),
                w_uvqk=bf16_round_f32(rng.uniform(-a1, a1, (nw, D)).astype(np.float32)),
                ln2_w=1.0 + 0.2 * rng.standard_normal(nu),
                w_out=bf16_round_f32(rng.uniform(-a2, a2, (D, nu)).astype(np.float32)),
                ln1_b=0.1 * rng.standard_normal(D), b_uvqk=0.1 * rng.standard_normal(nw),
                ln2_b=0.1 * rng.standard_normal(nu), b_out=0.1 * rng.standard_normal(D))
    host = {k: np.asarray(v, dtype=np.float32) for k, v in host.items()}
    T = int(sw.offsets[-1])
    dout = bf16_round_f32(rng.standard_normal((T, D)).astype(np.float32))
    kw = dict(heads=H, d_qk=dqk, d_v=dv, k1=sw.k1, k2=sw.k2, contextual_len=sw.contextual_len,
              max_seq_len=sw.max_seq_len)
    okw = dict(heads=H, dqk=dqk, dv=dv, k1=sw.k1, k2=sw.k2, ctx=sw.contextual_len,
               N=sw.max_seq_len, ln1_b=host["ln1_b"], b_uvqk=host["b_uvqk"],
               ln2_b=host["ln2_b"], b_out=host["b_out"])
    dev = {k: (torch.from_numpy(v).to(DEV).bfloat16() if k in ("w_uvqk", "w_out")
               else torch.from_numpy(v).to(DEV)) for k, v in host.items()}
    return sw, host, dout, kw, okw, dev


@pytest.mark.parametrize("dqk,dv", [(64, 128), (128, 64), (32, 64)])
def test_rect_stu_layer_fwd_bwd(dqk, dv):
    """The STU layer with rectangular heads, forward against the
    storage-matched oracle (the square-head layer test's bar) and backward
    against both oracle modes (the STU backward test's bars)."""
    from tests._helpers import BF16_MAX_TOL, BF16_MEAN_TOL, rel_errors
    sw, host, dout, kw, okw, dev = _stu_rect(dqk, dv)
    print(f"[case] rect stu layer dqk={dqk} dv={dv} T={int(sw.offsets[-1])}", flush=True)
    x = torch.from_numpy(sw.x).to(DEV).bfloat16()
    offs = torch.from_numpy(sw.offsets).to(DEV)
    tg = torch.from_numpy(sw.num_targets).to(DEV)
    bias = {k: dev[k] for k in ("ln1_b", "b_uvqk", "ln2_b", "b_out")}
    out = sla.stu_layer_fwd(x, offs, tg, dev["ln1_w"], dev["w_uvqk"], dev["ln2_w"], dev["w_out"],
                            **bias, **kw)
    g = sla.stu_layer_bwd(x, torch.from_numpy(dout).to(DEV).bfloat16(), offs, tg, dev["ln1_w"],
                          dev["w_uvqk"], dev["ln2_w"], dev["w_out"], **bias, **kw)
    torch.cuda.synchronize()
    ref, _ = oracle.stu_layer_fwd(sw.x, sw.offsets, sw.num_targets, host["ln1_w"],
                                  host["w_uvqk"], host["ln2_w"], host["w_out"], store_bf16=True,
                                  want_uvqk=True, **okw)
    mx, mn = assert_close_bf16(out.float().cpu().numpy().astype(np.float64), ref, "out",
                               ref_rounded=True)
    print(f"  out: max {mx:.3e} mean {mn:.3e}", flush=True)
    refs = {m: oracle.stu_layer_bwd(sw.x, sw.offsets, sw.num_targets, host["ln1_w"],
                                    host["w_uvqk"], host["ln2_w"], host["w_out"], dout,
                                    store_bf16=m, **okw) for m in (True, False)}
    for k in ("dx", "dw_uvqk", "db_uvqk", "dln2_w", "dw_out"):
        got = g[k].float().cpu().numpy().astype(np.float64)
        floor, _ = rel_errors(refs[True][k], refs[False][k])
        for what, r in (("storage-matched", refs[True][k]), ("exact", refs[False][k])):
            gm, gn = rel_errors(got, r)
            print(f"  {k:8s} vs {what}: max {gm:.3e} mean {gn:.3e} (floor {floor:.3e})",
                  flush=True)
            assert gn <= BF16_MEAN_TOL and gm <= BF16_MAX_TOL + floor, (k, what)
