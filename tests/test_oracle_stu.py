"""Pins for the oracle's LayerNorm, STU layer, bf16 rounding and truncation.

STU layer: ULTRA-HSTU paper, section 3 Eq.1-5 in the order of Code Listing 1;
fused projection split U, V, Q, K (HSTU notes section 2.4 Eq.1).  Truncation:
ULTRA-HSTU section 4.3 and the torcheasyrec page's truncation bullet.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synthetic import bf16_round_f32
from tests._helpers import dense_sla_torch


def test_layernorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((17, 24)) * 3 + 1
    w = rng.standard_normal(24)
    b = rng.standard_normal(24)
    y = oracle.layernorm(x, w, b, 1e-5)
    ref = F.layer_norm(torch.from_numpy(x), (24,), torch.from_numpy(w), torch.from_numpy(b),
                       1e-5).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    y0 = oracle.layernorm(x, w, None, 1e-5)
    ref0 = F.layer_norm(torch.from_numpy(x), (24,), torch.from_numpy(w), None, 1e-5).numpy()
    np.testing.assert_allclose(y0, ref0, rtol=1e-12, atol=1e-12)


def _stu_case(seed, lens, D=16, H=2, dqk=4, dv=3, tg=None):
    rng = np.random.default_rng(seed)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(offs[-1])
    nw = 2 * H * dv + 2 * H * dqk
    p = dict(
        x=rng.standard_normal((T, D)),
        ln1_w=1 + 0.1 * rng.standard_normal(D), ln1_b=0.1 * rng.standard_normal(D),
        w_uvqk=rng.standard_normal((nw, D)) * 0.4, b_uvqk=0.1 * rng.standard_normal(nw),
        ln2_w=1 + 0.1 * rng.standard_normal(H * dv), ln2_b=0.1 * rng.standard_normal(H * dv),
        w_out=rng.standard_normal((D, H * dv)) * 0.3, b_out=0.1 * rng.standard_normal(D))
    return offs, p


def _stu_torch(offs, p, tg, H, dqk, dv, k1, k2, ctx, N, alpha, eps):
    t = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in p.items()}
    x = t["x"]
    D = x.shape[1]
    n = F.layer_norm(x, (D,), t["ln1_w"], t["ln1_b"], eps)
    z = F.silu(F.linear(n, t["w_uvqk"], t["b_uvqk"]))
    T = x.shape[0]
    u, v, q, k = torch.split(z, [H * dv, H * dv, H * dqk, H * dqk], dim=1)
    a = dense_sla_torch(q.reshape(T, H, dqk), k.reshape(T, H, dqk), v.reshape(T, H, dv), offs,
                        tg, k1, k2, ctx, N, alpha).reshape(T, H * dv)
    y = F.layer_norm(a, (H * dv,), t["ln2_w"], t["ln2_b"], eps) * u
    return (F.linear(y, t["w_out"], t["b_out"]) + x).numpy(), z.numpy()


@pytest.mark.parametrize("tg", [None, [2, 1, 0]])
def test_stu_layer_matches_torch_composition(tg):
    lens = [6, 11, 9]
    H, dqk, dv = 2, 4, 3
    offs, p = _stu_case(3, lens, H=H, dqk=dqk, dv=dv)
    out, uvqk = oracle.stu_layer_fwd(p["x"], offs, tg, p["ln1_w"], p["w_uvqk"], p["ln2_w"],
                                     p["w_out"], heads=H, dqk=dqk, dv=dv, k1=3, k2=2, ctx=1,
                                     N=11.0, alpha=0.9, eps=1e-5, ln1_b=p["ln1_b"],
                                     b_uvqk=p["b_uvqk"], ln2_b=p["ln2_b"], b_out=p["b_out"],
                                     want_uvqk=True)
    ref, zref = _stu_torch(offs, p, tg, H, dqk, dv, 3, 2, 1, 11.0, 0.9, 1e-5)
    np.testing.assert_allclose(uvqk, zref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11)


def test_stu_zero_output_projection_is_identity():
    offs, p = _stu_case(5, [7, 4])
    out = oracle.stu_layer_fwd(p["x"], offs, None, p["ln1_w"], p["w_uvqk"], p["ln2_w"],
                               np.zeros_like(p["w_out"]), heads=2, dqk=4, dv=3, k1=3, k2=1,
                               ctx=0, N=7.0)
    assert np.array_equal(out, p["x"])


def test_stu_storage_matched_mode_rounds_to_bf16():
    offs, p = _stu_case(6, [9, 5])
    kw = dict(heads=2, dqk=4, dv=3, k1=3, k2=1, ctx=0, N=9.0)
    exact = oracle.stu_layer_fwd(p["x"], offs, None, p["ln1_w"], p["w_uvqk"], p["ln2_w"],
                                 p["w_out"], **kw)
    rounded, z = oracle.stu_layer_fwd(p["x"], offs, None, p["ln1_w"], p["w_uvqk"], p["ln2_w"],
                                      p["w_out"], store_bf16=True, want_uvqk=True, **kw)
    for a in (rounded, z):
        f = a.astype(np.float32)
        assert np.array_equal(f.astype(np.float64), a)
        assert np.array_equal(bf16_round_f32(f), f)
    rel = np.abs(rounded - exact).max() / np.sqrt((exact ** 2).mean())
    assert 0 < rel < 3e-2


def test_round_bf16_ties_and_values():
    """bfloat16 keeps 8 significant bits, ties go to even."""
    r = oracle.round_bf16
    assert r(1.0) == 1.0
    assert r(1.0 + 2 ** -8) == 1.0                  # tie -> even (1.0)
    assert r(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6    # tie -> even (1 + 4*2^-8)
    assert r(1.0 + 2 ** -8 + 2 ** -20) == 1.0 + 2 ** -7
    assert r(-3.0) == -3.0
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(2000) * 10.0 ** rng.uniform(-3, 3, 2000)).astype(np.float32)
    mine = np.array([r(float(a)) for a in x])
    assert np.array_equal(mine, bf16_round_f32(x).astype(np.float64))


# --------------------------------------------------------------------------
# truncation
# --------------------------------------------------------------------------
def _truncate_by_sets(lens, tg, ctx, tail):
    gidx, new_offs = [], [0]
    base = 0
    for L, T in zip(lens, tg):
        U = L - T
        c = min(ctx, U)
        history = list(range(c, U))
        keep = set(range(c)) | set(history[-tail:] if tail > 0 else []) | set(range(U, L))
        gidx += [base + i for i in sorted(keep)]
        new_offs.append(len(gidx))
        base += L
    return np.array(new_offs, np.int64), np.array(gidx, np.int64)


def test_truncate_matches_set_construction():
    rng = np.random.default_rng(3)
    for _ in range(50):
        B = int(rng.integers(1, 6))
        lens = [int(x) for x in rng.integers(0, 60, size=B)]
        tg = [int(rng.integers(0, L + 1)) for L in lens]
        ctx, tail = int(rng.integers(0, 10)), int(rng.integers(1, 40))
        offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        no, gi = oracle.truncate(offs, tg, ctx, tail)
        rno, rgi = _truncate_by_sets(lens, tg, ctx, tail)
        assert np.array_equal(no, rno) and np.array_equal(gi, rgi)


def test_truncate_is_identity_when_tail_covers_history():
    lens = [30, 12]
    offs = np.array([0, 30, 42], np.int64)
    no, gi = oracle.truncate(offs, [4, 2], 3, 23)
    assert np.array_equal(no, offs) and np.array_equal(gi, np.arange(42))


def test_truncate_tzrec_example_lengths():
    """torcheasyrec page: after truncation a sequence holds
    contextual_seq_len + attn_truncation_tail_len + num_targets tokens."""
    lens = [16 + 3000 + 64, 16 + 1024 + 64, 16 + 700 + 64]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    no, gi = oracle.truncate(offs, [64, 64, 64], 16, 1024)
    assert list(np.diff(no)) == [16 + 1024 + 64, 16 + 1024 + 64, 16 + 700 + 64]


# ---------------------------------------------------------------------------
# STU layer backward (gradients of the layer above given dL/dout)
# ---------------------------------------------------------------------------
_GRAD_KEYS = {"x": "dx", "ln1_w": "dln1_w", "ln1_b": "dln1_b", "w_uvqk": "dw_uvqk",
              "b_uvqk": "db_uvqk", "ln2_w": "dln2_w", "ln2_b": "dln2_b", "w_out": "dw_out",
              "b_out": "db_out"}


def _stu_bwd_args(p):
    return dict(ln1_b=p["ln1_b"], b_uvqk=p["b_uvqk"], ln2_b=p["ln2_b"], b_out=p["b_out"])


@pytest.mark.parametrize("tg", [None, [2, 1, 0]])
def test_stu_layer_bwd_matches_torch_autograd(tg):
    lens = [6, 11, 9]
    H, dqk, dv = 2, 4, 3
    offs, p = _stu_case(7, lens, H=H, dqk=dqk, dv=dv)
    rng = np.random.default_rng(8)
    dout = rng.standard_normal(p["x"].shape)
    kw = dict(heads=H, dqk=dqk, dv=dv, k1=3, k2=2, ctx=1, N=11.0, alpha=0.9, eps=1e-5)
    g = oracle.stu_layer_bwd(p["x"], offs, tg, p["ln1_w"], p["w_uvqk"], p["ln2_w"], p["w_out"],
                             dout, **kw, **_stu_bwd_args(p))
    t = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True) for k, v in p.items()}
    x = t["x"]
    D, T = x.shape[1], x.shape[0]
    n = F.layer_norm(x, (D,), t["ln1_w"], t["ln1_b"], 1e-5)
    z = F.silu(F.linear(n, t["w_uvqk"], t["b_uvqk"]))
    u, v, q, k = torch.split(z, [H * dv, H * dv, H * dqk, H * dqk], dim=1)
    a = dense_sla_torch(q.reshape(T, H, dqk), k.reshape(T, H, dqk), v.reshape(T, H, dv), offs,
                        tg, 3, 2, 1, 11.0, 0.9).reshape(T, H * dv)
    y = F.layer_norm(a, (H * dv,), t["ln2_w"], t["ln2_b"], 1e-5) * u
    out = F.linear(y, t["w_out"], t["b_out"]) + x
    (out * torch.from_numpy(dout)).sum().backward()
    for name, key in _GRAD_KEYS.items():
        np.testing.assert_allclose(g[key], t[name].grad.numpy(), rtol=1e-9, atol=1e-10,
                                   err_msg=name)


def _rne_bf16_torch(t):
    """Round fp64 to the nearest bf16 value, ties to even: t = m 2^e with
    0.5 <= |m| < 1 keeps 8 significant bits, a spacing of 2^(e-8)."""
    _, e = torch.frexp(t)
    q = (e - 8).to(torch.float64)
    return torch.where(t == 0, t, torch.round(t * torch.pow(2.0, -q)) * torch.pow(2.0, q))


class _Stored(torch.autograd.Function):
    """A tensor kept in bf16 between steps: its value and the gradient that
    flows back into it are both rounded."""

    @staticmethod
    def forward(ctx, t):
        return _rne_bf16_torch(t)

    @staticmethod
    def backward(ctx, g):
        return _rne_bf16_torch(g)


class _StoredSilu(torch.autograd.Function):
    """SiLU of the projection with z kept in bf16 for the backward: the output
    is SiLU of the unrounded z, rounded; the incoming gradient is rounded, then
    multiplied by SiLU' at the rounded z (torch's own derivative of F.silu),
    and the product rounded."""

    @staticmethod
    def forward(ctx, z):
        ctx.save_for_backward(_rne_bf16_torch(z))
        return _rne_bf16_torch(F.silu(z))

    @staticmethod
    def backward(ctx, g):
        (zr,) = ctx.saved_tensors
        with torch.enable_grad():
            zz = zr.detach().requires_grad_(True)
            (ds,) = torch.autograd.grad(F.silu(zz), zz, _rne_bf16_torch(g))
        return _rne_bf16_torch(ds)


def test_bf16_rne_torch_helper_matches_torch_conversion():
    # fp32 inputs convert to bf16 with one rounding in torch itself
    x = torch.randn(4096, generator=torch.Generator().manual_seed(0)) * 7
    assert torch.equal(_rne_bf16_torch(x.double()), x.bfloat16().double())


@pytest.mark.parametrize("tg", [None, [2, 1, 0]])
def test_stu_layer_bwd_storage_mode_matches_rounded_autograd(tg):
    lens = [6, 11, 9]
    H, dqk, dv = 2, 4, 3
    offs, p = _stu_case(12, lens, H=H, dqk=dqk, dv=dv)
    rng = np.random.default_rng(13)
    dout = rng.standard_normal(p["x"].shape)
    kw = dict(heads=H, dqk=dqk, dv=dv, k1=3, k2=2, ctx=1, N=11.0, alpha=0.9, eps=1e-5)
    g = oracle.stu_layer_bwd(p["x"], offs, tg, p["ln1_w"], p["w_uvqk"], p["ln2_w"], p["w_out"],
                             dout, store_bf16=True, **kw, **_stu_bwd_args(p))
    exact = oracle.stu_layer_bwd(p["x"], offs, tg, p["ln1_w"], p["w_uvqk"], p["ln2_w"],
                                 p["w_out"], dout, **kw, **_stu_bwd_args(p))
    t = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True) for k, v in p.items()}
    x = t["x"]
    D, T = x.shape[1], x.shape[0]
    n = _Stored.apply(F.layer_norm(x, (D,), t["ln1_w"], t["ln1_b"], 1e-5))
    z = _StoredSilu.apply(F.linear(n, t["w_uvqk"], t["b_uvqk"]))
    u, v, q, k = torch.split(z, [H * dv, H * dv, H * dqk, H * dqk], dim=1)
    a = dense_sla_torch(q.reshape(T, H, dqk), k.reshape(T, H, dqk), v.reshape(T, H, dv), offs,
                        tg, 3, 2, 1, 11.0, 0.9).reshape(T, H * dv)
    a = _Stored.apply(a)
    y = _Stored.apply(F.layer_norm(a, (H * dv,), t["ln2_w"], t["ln2_b"], 1e-5) * u)
    out = F.linear(y, t["w_out"], t["b_out"]) + x
    (out * torch.from_numpy(dout)).sum().backward()
    for name, key in _GRAD_KEYS.items():
        ref = t[name].grad
        if name == "x":
            ref = _rne_bf16_torch(ref)
        np.testing.assert_allclose(g[key], ref.numpy(), rtol=1e-9, atol=1e-10, err_msg=name)
        # the rounding is really applied: storage and exact modes differ
        # (db_out, the column sums of dout, involves no stored value)
        if name != "b_out":
            assert not np.allclose(g[key], exact[key], rtol=1e-6, atol=0), name


def test_stu_layer_bwd_matches_finite_differences():
    offs, p = _stu_case(9, [5, 7], D=8, H=1, dqk=4, dv=4)
    rng = np.random.default_rng(10)
    dout = rng.standard_normal(p["x"].shape)
    kw = dict(heads=1, dqk=4, dv=4, k1=3, k2=1, ctx=0, N=7.0, alpha=1.0, eps=1e-5)

    def loss(pp):
        out = oracle.stu_layer_fwd(pp["x"], offs, None, pp["ln1_w"], pp["w_uvqk"], pp["ln2_w"],
                                   pp["w_out"], ln1_b=pp["ln1_b"], b_uvqk=pp["b_uvqk"],
                                   ln2_b=pp["ln2_b"], b_out=pp["b_out"], **kw)
        return float((out * dout).sum())

    g = oracle.stu_layer_bwd(p["x"], offs, None, p["ln1_w"], p["w_uvqk"], p["ln2_w"],
                             p["w_out"], dout, **kw, **_stu_bwd_args(p))
    h = 1e-6
    for name, idx in [("x", (3, 2)), ("x", (10, 7)), ("ln1_w", (5,)), ("ln1_b", (1,)),
                      ("w_uvqk", (0, 3)), ("w_uvqk", (9, 1)), ("b_uvqk", (13,)),
                      ("ln2_w", (2,)), ("ln2_b", (0,)), ("w_out", (4, 3)), ("b_out", (6,))]:
        pp = {k: np.array(v, dtype=np.float64, copy=True) for k, v in p.items()}
        pp[name][idx] += h
        up = loss(pp)
        pp[name][idx] -= 2 * h
        dn = loss(pp)
        fd = (up - dn) / (2 * h)
        got = g[_GRAD_KEYS[name]][idx]
        assert abs(got - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, got, fd)


def test_stu_layer_bwd_of_zero_dout_is_zero():
    offs, p = _stu_case(11, [4, 6])
    g = oracle.stu_layer_bwd(p["x"], offs, None, p["ln1_w"], p["w_uvqk"], p["ln2_w"],
                             p["w_out"], np.zeros_like(p["x"]), heads=2, dqk=4, dv=3, k1=2,
                             k2=1, ctx=0, N=6.0, **_stu_bwd_args(p))
    for key, val in g.items():
        assert not np.any(val), key


# --------------------------------------------------------------------------
# storage-matched forward mode: each rounding point on its own
# --------------------------------------------------------------------------
_FWD_POINTS = ("n", "z", "a", "y", "out")


def _stu_torch_rounded(offs, p, tg, H, dqk, dv, kw, points):
    """The STU layer as a torch fp64 composition (ULTRA-HSTU paper, section 3
    Eq.1-5 in the order of Code Listing 1), rounding to bf16 with the
    frexp-based round-to-nearest-even above at the named points only: n (the
    normalised input), z (U|V|Q|K after SiLU), a (the attention output), y
    (the gated LayerNorm output) and out (the layer output, i.e. the residual
    stream)."""
    r = lambda name, t: _rne_bf16_torch(t) if name in points else t  # noqa: E731
    t = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in p.items()}
    x = t["x"]
    T, D = x.shape
    n = r("n", F.layer_norm(x, (D,), t["ln1_w"], t["ln1_b"], kw["eps"]))
    z = r("z", F.silu(F.linear(n, t["w_uvqk"], t["b_uvqk"])))
    u, v, q, k = torch.split(z, [H * dv, H * dv, H * dqk, H * dqk], dim=1)
    a = dense_sla_torch(q.reshape(T, H, dqk), k.reshape(T, H, dqk), v.reshape(T, H, dv), offs,
                        tg, kw["k1"], kw["k2"], kw["ctx"], kw["N"], kw["alpha"]).reshape(T, H * dv)
    a = r("a", a)
    y = r("y", F.layer_norm(a, (H * dv,), t["ln2_w"], t["ln2_b"], kw["eps"]) * u)
    out = r("out", F.linear(y, t["w_out"], t["b_out"]) + x)
    return out.numpy(), z.numpy()


@pytest.mark.parametrize("mask,points", [(1, ("n", "z", "a", "y")), (2, ("out",)),
                                         (3, _FWD_POINTS)])
@pytest.mark.parametrize("tg", [None, [2, 1, 0]])
def test_stu_storage_mode_matches_rounded_composition(mask, points, tg):
    """oracle.stu_layer_fwd(store_bf16=mask) equals the torch composition that
    rounds at exactly the points of that mask (bit 1: the branch tensors n,
    U|V|Q|K, A, y; bit 2: the layer output), and differs from it as soon as
    any one of those points is left unrounded: each rounding point is
    present, and none is applied twice or in the wrong place."""
    lens = [6, 11, 9]
    H, dqk, dv = 2, 4, 3
    offs, p = _stu_case(21, lens, H=H, dqk=dqk, dv=dv)
    # inputs as a bf16 implementation receives them
    p = {k: (bf16_round_f32(np.asarray(v, np.float32)).astype(np.float64)
             if k in ("x", "w_uvqk", "w_out") else v) for k, v in p.items()}
    kw = dict(k1=3, k2=2, ctx=1, N=11.0, alpha=0.9, eps=1e-5)
    out, z = oracle.stu_layer_fwd(p["x"], offs, tg, p["ln1_w"], p["w_uvqk"], p["ln2_w"],
                                  p["w_out"], heads=H, dqk=dqk, dv=dv, ln1_b=p["ln1_b"],
                                  b_uvqk=p["b_uvqk"], ln2_b=p["ln2_b"], b_out=p["b_out"],
                                  store_bf16=mask, want_uvqk=True, **kw)
    ref, zref = _stu_torch_rounded(offs, p, tg, H, dqk, dv, kw, points)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, zref, rtol=1e-12, atol=1e-12)
    for drop in points:
        alt, _ = _stu_torch_rounded(offs, p, tg, H, dqk, dv, kw,
                                    tuple(q for q in points if q != drop))
        assert np.abs(alt - out).max() > 1e-6, f"rounding point {drop} has no effect"
    # a rounding point outside the mask is not applied either
    for extra in _FWD_POINTS:
        if extra in points:
            continue
        alt, _ = _stu_torch_rounded(offs, p, tg, H, dqk, dv, kw, points + (extra,))
        assert np.abs(alt - out).max() > 1e-6, f"rounding point {extra} applied by mask {mask}"
