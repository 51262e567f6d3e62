"""Pins for the oracle's SLA forward and backward.

Forward: a dense torch fp64 reference (library matmuls over the full mask),
textbook special cases and invariants.  Backward: central finite differences
of the oracle's own forward and torch fp64 autograd of the dense reference.
(ULTRA-HSTU paper, section 3 Eq.3 and section 4.2.1 Eq.6-7; HSTU notes,
section 2.4 Eq.2: pointwise SiLU, no softmax.)
"""
import numpy as np
import pytest
import torch

import oracle
from tests._helpers import dense_sla_torch


def _rand(rng, T, H, d, std=1.0):
    return rng.standard_normal((T, H, d)) * std


def _case(seed, lens, H=2, d=8, std=0.7):
    rng = np.random.default_rng(seed)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(offs[-1])
    return offs, _rand(rng, T, H, d, std), _rand(rng, T, H, d, std), _rand(rng, T, H, d, std), \
        _rand(rng, T, H, d)


@pytest.mark.parametrize("k1,k2,ctx,tg", [
    (8, 4, 2, None), (3, 0, 0, None), (0, 5, 0, None), (100, 0, 0, None),
    (5, 2, 3, [2, 0, 4]), (1, 1, 0, [1, 1, 1]), (0, 2, 0, [3, 0, 1]),
])
def test_fwd_matches_dense_reference(k1, k2, ctx, tg):
    lens = [13, 1, 20]
    offs, q, k, v, _ = _case(7, lens)
    N, alpha = 37.0, 0.8
    o = oracle.sla_fwd(q, k, v, offs, tg, k1, k2, ctx, N, alpha)
    ref = dense_sla_torch(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), offs,
                          tg, k1, k2, ctx, N, alpha).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_fwd_rectangular_heads():
    """d_qk != d_v: Q.K^T contracts over d_qk, P.V produces d_v columns."""
    rng = np.random.default_rng(3)
    lens = [9, 15]
    offs = np.array([0, 9, 24], np.int64)
    q, k = rng.standard_normal((24, 3, 5)), rng.standard_normal((24, 3, 5))
    v = rng.standard_normal((24, 3, 7))
    o = oracle.sla_fwd(q, k, v, offs, None, 4, 2, 0, 16.0)
    ref = dense_sla_torch(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), offs,
                          None, 4, 2, 0, 16.0).numpy()
    assert o.shape == (24, 3, 7)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_full_window_equals_full_causal_hstu():
    """K1 >= L reproduces full causal HSTU attention (Eq.6)."""
    lens = [17, 30]
    offs, q, k, v, _ = _case(11, lens)
    a = oracle.sla_fwd(q, k, v, offs, None, 30, 0, 0, 30.0)
    b = oracle.sla_fwd(q, k, v, offs, None, 10 ** 6, 7, 3, 30.0)
    assert np.array_equal(a, b)
    # hand-written causal HSTU for one row
    i, h = 40, 1
    s = q[i, h] @ k[17:41, h].T
    ref = ((s / (1 + np.exp(-s)))[:, None] * v[17:41, h]).sum(0) / 30.0
    np.testing.assert_allclose(a[i, h], ref, rtol=1e-12)


def test_perturbing_invisible_keys_leaves_rows_unchanged():
    lens = [40]
    offs, q, k, v, _ = _case(5, lens)
    k1, k2, ctx = 6, 3, 0
    base = oracle.sla_fwd(q, k, v, offs, None, k1, k2, ctx, 40.0)
    m = oracle.mask_dense(40, 0, k1, k2, ctx)
    for j in (0, 3, 10, 25, 39):
        k2_, v2_ = k.copy(), v.copy()
        k2_[j] += 3.0
        v2_[j] -= 2.0
        out = oracle.sla_fwd(q, k2_, v2_, offs, None, k1, k2, ctx, 40.0)
        unchanged = m[:, j] == 0
        assert np.array_equal(out[unchanged], base[unchanged])
        assert np.all(np.any(out[~unchanged] != base[~unchanged], axis=(1, 2)))


def test_linear_in_v_and_inverse_in_n():
    lens = [11, 23]
    offs, q, k, v, _ = _case(9, lens)
    rng = np.random.default_rng(1)
    v2 = rng.standard_normal(v.shape)
    a = oracle.sla_fwd(q, k, v, offs, None, 5, 2, 1, 8.0)
    b = oracle.sla_fwd(q, k, v2, offs, None, 5, 2, 1, 8.0)
    c = oracle.sla_fwd(q, k, 2.0 * v - 3.0 * v2, offs, None, 5, 2, 1, 8.0)
    np.testing.assert_allclose(c, 2.0 * a - 3.0 * b, rtol=1e-11, atol=1e-12)
    d = oracle.sla_fwd(q, k, v, offs, None, 5, 2, 1, 64.0)   # power-of-two ratio: exact
    assert np.array_equal(d * 8.0, a)


def test_jagged_sequences_are_independent():
    lens = [7, 19, 1, 12]
    offs, q, k, v, _ = _case(21, lens)
    tg = [2, 3, 1, 0]
    full = oracle.sla_fwd(q, k, v, offs, tg, 4, 2, 1, 20.0)
    for b, L in enumerate(lens):
        s0 = int(offs[b])
        one = oracle.sla_fwd(q[s0:s0 + L], k[s0:s0 + L], v[s0:s0 + L], [0, L], [tg[b]], 4, 2,
                             1, 20.0)
        assert np.array_equal(one, full[s0:s0 + L])


def test_target_permutation_equivariance():
    L, T = 30, 5
    offs, q, k, v, _ = _case(17, [L])
    perm = np.array([3, 0, 4, 1, 2])
    idx = np.concatenate([np.arange(L - T), L - T + perm])
    a = oracle.sla_fwd(q, k, v, offs, [T], 7, 3, 0, 30.0)
    b = oracle.sla_fwd(q[idx], k[idx], v[idx], offs, [T], 7, 3, 0, 30.0)
    assert np.array_equal(b, a[idx])


def test_one_target_equals_no_target():
    offs, q, k, v, _ = _case(2, [15, 8])
    a = oracle.sla_fwd(q, k, v, offs, [1, 1], 4, 2, 0, 15.0)
    b = oracle.sla_fwd(q, k, v, offs, None, 4, 2, 0, 15.0)
    assert np.array_equal(a, b)


def test_row_selection():
    offs, q, k, v, _ = _case(4, [10, 20])
    full = oracle.sla_fwd(q, k, v, offs, None, 4, 2, 0, 20.0)
    sel = np.zeros(30, np.uint8)
    sel[[0, 9, 10, 29]] = 1
    part = oracle.sla_fwd(q, k, v, offs, None, 4, 2, 0, 20.0, row_sel=sel)
    assert np.array_equal(part[sel == 1], full[sel == 1])
    assert np.all(part[sel == 0] == 0)


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
@pytest.mark.parametrize("k1,k2,ctx,tg,alpha", [
    (4, 2, 1, None, 1.0), (3, 0, 0, [2, 1], 0.7), (0, 3, 0, [1, 3], 1.3), (50, 0, 0, None, 1.0),
])
def test_bwd_matches_torch_autograd(k1, k2, ctx, tg, alpha):
    lens = [9, 14]
    offs, q, k, v, do = _case(31, lens, H=2, d=6)
    N = 14.0
    dq, dk, dv = oracle.sla_bwd(q, k, v, do, offs, tg, k1, k2, ctx, N, alpha)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o = dense_sla_torch(tq, tk, tv, offs, tg, k1, k2, ctx, N, alpha)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_bwd_matches_finite_differences():
    """Central differences of L(q,k,v) = sum(O * dO) through the oracle forward."""
    lens = [8, 11]
    offs, q, k, v, do = _case(41, lens, H=2, d=5)
    k1, k2, ctx, tg, N, alpha = 3, 2, 0, [0, 2], 11.0, 0.9
    dq, dk, dv = oracle.sla_bwd(q, k, v, do, offs, tg, k1, k2, ctx, N, alpha)

    def loss(qq, kk, vv):
        return float((oracle.sla_fwd(qq, kk, vv, offs, tg, k1, k2, ctx, N, alpha) * do).sum())

    eps = 1e-6
    rng = np.random.default_rng(0)
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[idx] += eps
            am[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = ap, am
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                  loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_bwd_selection():
    offs, q, k, v, do = _case(8, [12, 9])
    full = oracle.sla_bwd(q, k, v, do, offs, None, 3, 2, 0, 12.0)
    qs = np.zeros(21, np.uint8)
    qs[[1, 11, 20]] = 1
    ks = np.zeros(21, np.uint8)
    ks[[0, 5, 12]] = 1
    part = oracle.sla_bwd(q, k, v, do, offs, None, 3, 2, 0, 12.0, q_sel=qs, k_sel=ks)
    assert np.array_equal(part[0][qs == 1], full[0][qs == 1])
    assert np.array_equal(part[1][ks == 1], full[1][ks == 1])
    assert np.array_equal(part[2][ks == 1], full[2][ks == 1])
