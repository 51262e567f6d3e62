"""Pins for oracle.sla_fwd_candidates: candidate scoring against a cached
history (HSTU notes, section 2.6 M-FALCON; target rows of the ULTRA-HSTU mask).

A candidate sees the history keys that the first candidate position sees, and
itself.  Laid out as [history | candidates] per sequence with the candidates
as targets, that is exactly the target rows of the plain forward, which the
dense torch reference computes with library matmuls over the full mask."""
import numpy as np
import pytest
import torch

import oracle
from tests._helpers import dense_sla_torch


def _case(seed, hist, cands, H=2, d=8):
    rng = np.random.default_rng(seed)
    ho = np.concatenate([[0], np.cumsum(hist)]).astype(np.int64)
    co = np.concatenate([[0], np.cumsum(cands)]).astype(np.int64)
    mk = lambda n: rng.standard_normal((n, H, d)) * 0.7  # noqa: E731
    return ho, co, mk(int(ho[-1])), mk(int(ho[-1])), mk(int(co[-1])), mk(int(co[-1])), \
        mk(int(co[-1]))


def _combined(ho, co, kh, vh, qc, kc, vc, rng_q):
    """[history | candidates] per sequence; history rows get arbitrary q."""
    parts_q, parts_k, parts_v, offs, tg, rows = [], [], [], [0], [], []
    for b in range(len(ho) - 1):
        U, n = int(ho[b + 1] - ho[b]), int(co[b + 1] - co[b])
        hs, cs = slice(ho[b], ho[b + 1]), slice(co[b], co[b + 1])
        parts_q += [rng_q.standard_normal(kh[hs].shape), qc[cs]]
        parts_k += [kh[hs], kc[cs]]
        parts_v += [vh[hs], vc[cs]]
        rows += list(range(offs[-1] + U, offs[-1] + U + n))
        offs.append(offs[-1] + U + n)
        tg.append(n)
    cat = lambda p: np.concatenate(p, 0)  # noqa: E731
    return (cat(parts_q), cat(parts_k), cat(parts_v), np.asarray(offs, np.int64),
            np.asarray(tg, np.int32), np.asarray(rows, np.int64))


KW = dict(k1=5, k2=2, ctx=3, N=13.0, alpha=0.8)


@pytest.mark.parametrize("hist, cands", [([9, 14, 0, 4], [3, 5, 2, 0]), ([20], [7])])
def test_candidates_match_dense_target_rows(hist, cands):
    ho, co, kh, vh, qc, kc, vc = _case(0, hist, cands)
    o = oracle.sla_fwd_candidates(kh, vh, ho, qc, kc, vc, co, **KW)
    q, k, v, offs, tg, rows = _combined(ho, co, kh, vh, qc, kc, vc, np.random.default_rng(1))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    dense = dense_sla_torch(t(q), t(k), t(v), offs, tg, KW["k1"], KW["k2"], KW["ctx"], KW["N"],
                            KW["alpha"]).numpy()
    np.testing.assert_allclose(o, dense[rows], rtol=1e-12, atol=1e-14)
    # and the oracle's own forward on the combined layout, target rows
    full = oracle.sla_fwd(q, k, v, offs, tg, KW["k1"], KW["k2"], KW["ctx"], KW["N"], KW["alpha"])
    np.testing.assert_allclose(o, full[rows], rtol=1e-12, atol=1e-14)


def test_microbatches_give_the_same_scores():
    ho, co, kh, vh, qc, kc, vc = _case(2, [30, 17], [12, 9])
    whole = oracle.sla_fwd_candidates(kh, vh, ho, qc, kc, vc, co, **KW)
    # microbatches of at most 4 candidates per sequence, scored call by call
    got = np.zeros_like(whole)
    for m0 in range(0, 12, 4):
        sel, offs = [], [0]
        for b in range(2):
            n = int(co[b + 1] - co[b])
            idx = np.arange(co[b] + min(m0, n), co[b] + min(m0 + 4, n))
            sel.append(idx)
            offs.append(offs[-1] + len(idx))
        idx = np.concatenate(sel)
        o = oracle.sla_fwd_candidates(kh, vh, ho, qc[idx], kc[idx], vc[idx],
                                      np.asarray(offs, np.int64), **KW)
        got[idx] = o
    assert np.array_equal(got, whole)


def test_candidates_do_not_see_each_other():
    ho, co, kh, vh, qc, kc, vc = _case(3, [11], [6])
    o = oracle.sla_fwd_candidates(kh, vh, ho, qc, kc, vc, co, **KW)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[2] += 5.0
    vc2[2] -= 3.0
    o2 = oracle.sla_fwd_candidates(kh, vh, ho, qc, kc2, vc2, co, **KW)
    others = [0, 1, 3, 4, 5]
    assert np.array_equal(o[others], o2[others])
    assert not np.allclose(o[2], o2[2])


def test_candidate_without_history_sees_only_itself():
    ho, co, kh, vh, qc, kc, vc = _case(4, [0], [3], H=1, d=4)
    o = oracle.sla_fwd_candidates(kh, vh, ho, qc, kc, vc, co, **KW)
    s = KW["alpha"] * np.einsum("chd,chd->ch", qc, kc)
    silu = s / (1.0 + np.exp(-s))
    np.testing.assert_allclose(o, silu[..., None] * vc / KW["N"], rtol=1e-13)
