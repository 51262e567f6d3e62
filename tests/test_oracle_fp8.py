"""Pins for the oracle's FP8 path (ULTRA-HSTU paper, section 4.2.2, mixed
precision: both STU projections in FP8 with row-wise scales computed where
the operand is produced).

E4M3 rounding is pinned to torch's own float32 -> float8_e4m3fn conversion
and, for fp64 inputs, to a nearest-value search over the table of e4m3
values.  Row quantisation is pinned in both of its decision precisions: the
fp64 one to that search over fp64 quotients, the fp32 one (the kernels') to
the same search over numpy's IEEE fp32 quotients.  The FP8 layer is pinned to
a torch fp64 composition that quantises the fp32 way."""
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


def _e4m3_table():
    """The non-negative finite e4m3fn values in increasing order: index
    8 e + m holds mantissa m (0..7) of biased exponent e (0..15), the
    subnormals m 2^-9 for e = 0, (1 + m/8) 2^(e-7) otherwise; e = 15, m = 7
    is NaN and left out, so the largest value is 448."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def _nearest_e4m3(v):
    """Round fp64 values to the nearest e4m3 value by search over the table,
    ties to the even mantissa, saturating at 448: a brute-force definition,
    independent of the oracle's frexp arithmetic."""
    tab = _e4m3_table()
    a = np.minimum(np.abs(np.asarray(v, np.float64)), 448.0)
    hi = np.clip(np.searchsorted(tab, a), 1, len(tab) - 1)
    lo = hi - 1
    dlo, dhi = a - tab[lo], tab[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    return np.sign(v) * tab[pick]


def test_e4m3_rounding_of_fp64_values_is_nearest():
    """fp64 inputs (the quotients of the row quantisation) round once, to the
    nearest e4m3 value: values near every midpoint, at the midpoints and
    random magnitudes over the whole range."""
    rng = np.random.default_rng(4)
    tab = _e4m3_table()
    mids = (tab[1:] + tab[:-1]) / 2
    x = np.concatenate([mids, mids * (1 + 1e-12), mids * (1 - 1e-12), tab,
                        rng.uniform(-448, 448, 20000), rng.standard_normal(5000) * 0.01])
    x = np.concatenate([x, -x])
    assert np.array_equal(oracle.round_e4m3(x), _nearest_e4m3(x))


def _quant_fp32(m):
    """Row quantisation decided in fp32, by numpy's IEEE fp32 arithmetic: a
    = max|x| and 448 / a, the product and a / 448 each one fp32 operation,
    then the nearest e4m3 value of that fp32 product."""
    m32 = np.asarray(m, np.float64).astype(np.float32)
    a = np.abs(m32).max(axis=1, keepdims=True)
    nz = a > 0
    inv = np.where(nz, np.float32(448.0) / np.where(nz, a, np.float32(1.0)), np.float32(0.0))
    q = _nearest_e4m3((m32 * inv.astype(np.float32)).astype(np.float64))
    s = np.where(nz, (a / np.float32(448.0)).astype(np.float64), 1.0)
    return q, s[:, 0]


def test_row_quantisation():
    """ULTRA-HSTU paper, section 4.2.2 (a scale per row, the row maximum
    mapped to the top of the e4m3 range): a = max|x|, s = a / 448, q =
    nearest e4m3 of x * (448 / a), with that arithmetic in fp64 or in fp32."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((7, 64)) * rng.uniform(0.01, 100, size=(7, 1))).astype(np.float32)
    x[3] = 0.0
    q, s = oracle.quant_rows_fp8(x, "fp64")
    assert s[3] == 1.0 and not np.any(q[3])
    for r in (0, 1, 2, 4, 5, 6):
        xr = x[r].astype(np.float64)
        a = np.abs(xr).max()
        assert s[r] == a / 448.0
        assert np.abs(q[r]).max() == 448.0        # the row maximum maps to 448
        assert np.array_equal(q[r], _nearest_e4m3(xr * (448.0 / a)))
        # each element within half an e4m3 step of x / s
        vv = xr / s[r]
        ulp = np.where(np.abs(vv) >= 2.0 ** -6,
                       2.0 ** (np.floor(np.log2(np.abs(vv) + 1e-300)) - 3), 2.0 ** -9)
        assert np.all(np.abs(q[r] - vv) <= ulp / 2 * (1 + 1e-12))
    q32, s32 = oracle.quant_rows_fp8(x, "fp32")
    rq32, rs32 = _quant_fp32(x)
    assert np.array_equal(q32, rq32) and np.array_equal(s32, rs32)
    assert np.all(np.abs(q32).max(axis=1)[[0, 1, 2, 4, 5, 6]] == 448.0)
    with pytest.raises(ValueError):
        oracle.quant_rows_fp8(x, "fp16")


def test_fp32_decision_on_bf16_rows_with_exact_ties():
    """bf16 rows (8 significant bits) put x * 448 / a exactly on e4m3
    midpoints often; the fp32 decision still equals numpy's fp32 arithmetic
    there, code for code, and all-zero rows get scale 1."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 256)).astype(np.float32) * rng.uniform(
        0.001, 50, size=(64, 1)).astype(np.float32)
    x = torch.from_numpy(x).bfloat16().double().numpy()
    x[9] = 0.0
    q, s = oracle.quant_rows_fp8(x, "fp32")
    rq, rs = _quant_fp32(x)
    assert np.array_equal(q, rq) and np.array_equal(s, rs)
    assert s[9] == 1.0 and not np.any(q[9])
    q64, _ = oracle.quant_rows_fp8(x, "fp64")
    assert (q != q64).sum() > 0     # ties decided differently somewhere


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

    def quant(m):  # row-wise, decided in fp32 by numpy's IEEE arithmetic
        q, s = _quant_fp32(m.numpy())
        return torch.from_numpy(q), torch.from_numpy(s[:, None])

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


def test_fp32_decided_codes_differ_only_near_midpoints():
    """How often the fp32 decision (448 / a, the product and the rounding
    each one fp32 operation, as the kernels form them) differs from the fp64
    decision, on the 18-layer stack's Xavier weights
    (bf16) and on LayerNorm-like fp32 rows: only where the fp64 quotient lies
    within fp32 rounding of a point halfway between two neighbouring e4m3
    values, and then by one e4m3 step."""
    from synthetic import make_stack_workload
    sw = make_stack_workload(seed=0, lengths=[64], layers=2)
    rng = np.random.default_rng(3)
    mats = [np.asarray(w, np.float32) for w in sw.w_uvqk + sw.w_out]
    mats.append(rng.standard_normal((4096, 512)).astype(np.float32))
    tab = _e4m3_table()
    total = flips = 0
    for m in mats:
        q64, _ = oracle.quant_rows_fp8(m, "fp64")
        q32, _ = oracle.quant_rows_fp8(m, "fp32")
        a = np.abs(m).max(axis=1, keepdims=True)
        assert np.array_equal(q32, _quant_fp32(m)[0])
        diff = q32 != q64
        total += m.size
        flips += int(diff.sum())
        if diff.any():
            v64 = (m.astype(np.float64) * (448.0 / a.astype(np.float64)))[diff]
            lo = np.minimum(np.abs(q32[diff]), np.abs(q64[diff]))
            hi = np.maximum(np.abs(q32[diff]), np.abs(q64[diff]))
            idx = np.searchsorted(tab, lo)
            assert np.array_equal(tab[idx + 1], hi), "codes more than one step apart"
            mid = (lo + hi) / 2
            assert np.all(np.abs(np.abs(v64) - mid) <= 2.0 ** -22 * mid)
    print(f"fp32-decided codes differing from fp64: {flips} of {total} ({flips / total:.2e})")
    assert flips / total < 1e-4
