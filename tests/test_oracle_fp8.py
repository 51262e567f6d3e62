"""Pins for the oracle's FP8 path (ULTRA-HSTU paper, section 4.2.2, mixed
precision: both STU projections in FP8 with row-wise scales computed where
the operand is produced).

E4M3 rounding is pinned to torch's own float32 -> float8_e4m3fn conversion;
the FP8 layer to a torch fp64 composition that quantises with that
conversion."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tests._helpers import dense_sla_torch, rel_errors


def _rne_bf16(t):
    _, e = torch.frexp(t)
    q = (e - 8).to(torch.float64)
    return torch.where(t == 0, t, torch.round(t * torch.pow(2.0, -q)) * torch.pow(2.0, q))


def test_e4m3_rounding_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 40,      # normals
        rng.standard_normal(5000).astype(np.float32) * 0.01,     # subnormals (< 2^-6)
        np.array([k / 16.0 for k in range(16, 33)], np.float32),  # ties at 1 .. 2
        np.array([448.0, -448.0, 0.0, 2.0 ** -9, 3 * 2.0 ** -10], np.float32),
    ])
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.round_e4m3(x)
    assert np.array_equal(got, ref)
    # saturation instead of NaN past the largest finite value
    assert oracle.round_e4m3([1000.0, -465.0])[0] == 448.0
    assert oracle.round_e4m3([-465.0])[0] == -448.0


def test_row_quantisation():
    """Codes decided in fp32 (the kernels' precision): a = max|x|,
    inv = 448 / a, p = x * inv, each one IEEE fp32 operation (numpy float32),
    then e4m3; scale a / 448 in fp32."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((7, 64)) * rng.uniform(0.01, 100, size=(7, 1))).astype(np.float32)
    x[3] = 0.0
    q, s = oracle.quant_rows_fp8(x)
    assert s[3] == 1.0 and not np.any(q[3])
    for r in (0, 1, 2, 4, 5, 6):
        a = np.abs(x[r]).max()
        assert s[r] == float(a / np.float32(448.0))
        assert np.abs(q[r]).max() == 448.0        # the row maximum maps to 448
        v = (x[r] * (np.float32(448.0) / a)).astype(np.float32)
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        assert np.array_equal(q[r], ref)
        # each element within half an e4m3 ulp (plus fp32 rounding) of x / s
        vv = x[r].astype(np.float64) / s[r]
        ulp = np.where(np.abs(vv) >= 2.0 ** -6,
                       2.0 ** (np.floor(np.log2(np.abs(vv) + 1e-300)) - 3), 2.0 ** -9)
        assert np.all(np.abs(q[r] - vv) <= ulp / 2 + 1e-5 * np.abs(vv) + 1e-12)


def _case(seed, lens, D=32, H=2, d=16, tg=None):
    rng = np.random.default_rng(seed)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(offs[-1])
    nw = 4 * H * d
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float32)).bfloat16().double().numpy()  # noqa
    p = dict(x=bf(rng.standard_normal((T, D))),
             ln1_w=1 + 0.1 * rng.standard_normal(D), ln1_b=0.1 * rng.standard_normal(D),
             w_uvqk=bf(rng.standard_normal((nw, D)) * 0.2), b_uvqk=0.1 * rng.standard_normal(nw),
             ln2_w=1 + 0.1 * rng.standard_normal(H * d), ln2_b=0.1 * rng.standard_normal(H * d),
             w_out=bf(rng.standard_normal((D, H * d)) * 0.2), b_out=0.1 * rng.standard_normal(D))
    return offs, p


def _torch_fp8_layer(offs, p, tg, H, d, kw):
    t = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in p.items()}
    x = t["x"]
    T, D = x.shape

    def quant(m):  # row-wise in fp32, via torch's float8 conversion
        # fp32 quotients and products rounded once: computed exactly enough in
        # fp64 and then rounded to fp32 (torch's own fp32 tensor division is
        # not correctly rounded)
        mf = m.float().double()
        a = mf.abs().amax(dim=1, keepdim=True)
        s = torch.where(a > 0, (a / 448.0).float().double(), torch.ones_like(a))
        inv = torch.where(a > 0, (448.0 / a).float().double(), torch.zeros_like(a))
        p = (mf * inv).float()
        q = p.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64)
        return q, s

    n = F.layer_norm(x, (D,), t["ln1_w"], t["ln1_b"], kw["eps"])
    nq, sn = quant(n)
    w1q, sw1 = quant(t["w_uvqk"])
    z = sn * (nq @ w1q.T) * sw1.T + t["b_uvqk"]
    s = _rne_bf16(F.silu(z))
    u, v, q, k = torch.split(s, [H * d] * 4, dim=1)
    a = dense_sla_torch(q.reshape(T, H, d), k.reshape(T, H, d), v.reshape(T, H, d), offs, tg,
                        kw["k1"], kw["k2"], kw["ctx"], kw["N"], kw["alpha"]).reshape(T, H * d)
    a = _rne_bf16(a)
    y = F.layer_norm(a, (H * d,), t["ln2_w"], t["ln2_b"], kw["eps"]) * u
    yq, sy = quant(y)
    w2q, sw2 = quant(t["w_out"])
    out = sy * (yq @ w2q.T) * sw2.T + t["b_out"] + x
    return _rne_bf16(out).numpy(), s.numpy()


@pytest.mark.parametrize("tg", [None, [2, 1, 0]])
def test_fp8_layer_matches_torch_composition(tg):
    H, d = 2, 16
    offs, p = _case(2, [9, 14, 6], H=H, d=d)
    kw = dict(k1=4, k2=2, ctx=1, N=14.0, alpha=1.0, eps=1e-5)
    out, uvqk = oracle.stu_layer_fwd_fp8(p["x"], offs, tg, p["ln1_w"], p["w_uvqk"], p["ln2_w"],
                                         p["w_out"], heads=H, dqk=d, dv=d, k1=kw["k1"],
                                         k2=kw["k2"], ctx=kw["ctx"], N=kw["N"], alpha=kw["alpha"],
                                         eps=kw["eps"], ln1_b=p["ln1_b"], b_uvqk=p["b_uvqk"],
                                         ln2_b=p["ln2_b"], b_out=p["b_out"], want_uvqk=True)
    ref, ruvqk = _torch_fp8_layer(offs, p, tg, H, d, kw)
    np.testing.assert_allclose(uvqk, ruvqk, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_fp8_layer_is_close_to_the_bf16_layer():
    """FP8 moves the layer's branch (out - x) by a few percent of its rms on
    average (e4m3 keeps 3 mantissa bits: up to 2^-4 relative per operand
    element, two quantised operands per product, two projections)."""
    H, d = 2, 16
    offs, p = _case(3, [40, 25], D=64, H=H, d=d)
    kw = dict(heads=H, dqk=d, dv=d, k1=16, k2=4, ctx=2, N=40.0, ln1_b=p["ln1_b"],
              b_uvqk=p["b_uvqk"], ln2_b=p["ln2_b"], b_out=p["b_out"])
    out8 = oracle.stu_layer_fwd_fp8(p["x"], offs, None, p["ln1_w"], p["w_uvqk"], p["ln2_w"],
                                    p["w_out"], **kw)
    out16 = oracle.stu_layer_fwd(p["x"], offs, None, p["ln1_w"], p["w_uvqk"], p["ln2_w"],
                                 p["w_out"], store_bf16=True, **kw)
    mx, mn = rel_errors(out8 - p["x"], out16 - p["x"])
    assert 0.005 < mn < 0.1 and mx < 1.0, (mx, mn)
