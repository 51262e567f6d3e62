"""Pins for the oracle's visibility predicate, pair count and tile enumeration.

The mask is the semi-local attention mask of the ULTRA-HSTU paper (section
4.2.1, Eq.7; complexity O((K1+K2) L)), with the torcheasyrec page's
effective_k2 = max(sla_k2, contextual_seq_len), and target rows as in the HSTU
notes' M-FALCON diagram (Q8).  None of these tests re-types the predicate:
they check it against printed examples, closed forms and textbook masks.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _closed_form_pairs(L, T, k1, k2e):
    """Pair count of one sequence from the closed form (summation identities).

    History part, U = L - T rows: row i sees min(i+1, K1) window keys and
    max(0, min(K2e, i-K1+1)) prefix keys outside the window, so
      P(U) = m(m+1)/2 + (U-m) K1 + S(U-K1, K2e),  m = min(U, K1),
      S(n, K) = 0 (n<0); n(n+1)/2 (n<=K); K(K+1)/2 + (n-K) K otherwise.
    Each target sees the history part of row U's view, plus itself.
    """
    def S(n, K):
        if n < 0:
            return 0
        if n <= K:
            return n * (n + 1) // 2
        return K * (K + 1) // 2 + (n - K) * K

    U = L - T
    m = min(U, k1)
    p = m * (m + 1) // 2 + (U - m) * k1 + S(U - k1, k2e)
    if T:
        window = max(0, min(U, k1 - 1))
        prefix = max(0, min(k2e, U - k1 + 1, U))
        p += T * (window + prefix + 1)
    return p


def test_closed_form_pair_count_matches_enumeration():
    rng = np.random.default_rng(1234)
    for _ in range(400):
        L = int(rng.integers(1, 60))
        T = int(rng.integers(0, L + 1)) if rng.random() < 0.5 else 0
        k1 = int(rng.integers(0, 70))
        k2 = int(rng.integers(0, 20))
        ctx = int(rng.integers(0, 20))
        got = oracle.count_pairs([0, L], [T] if T else None, k1, k2, ctx)
        assert got == _closed_form_pairs(L, T, k1, max(k2, ctx)), (L, T, k1, k2, ctx)


def test_pair_count_batch_is_sum_of_sequences():
    lens = [5, 17, 1, 40, 33]
    tg = [0, 3, 0, 7, 33]
    offs = np.concatenate([[0], np.cumsum(lens)])
    tot = oracle.count_pairs(offs, tg, 6, 3, 2)
    assert tot == sum(_closed_form_pairs(L, T, 6, 3) for L, T in zip(lens, tg))


def test_linear_complexity_rows():
    """Section 4.2.1: cost O((K1 + K2) L): far from the start every row sees
    exactly K1 + K2e keys."""
    L, k1, k2 = 300, 40, 9
    m = oracle.mask_dense(L, 0, k1, k2, 0)
    rows = m.sum(axis=1)
    assert np.all(rows[k1 + k2 - 1:] == k1 + k2)


def test_full_window_is_full_causal():
    """Eq.6: with K1 >= L the mask is the full causal (lower-triangular) mask."""
    for L in (1, 7, 33):
        for k2 in (0, 3, 50):
            m = oracle.mask_dense(L, 0, L, k2, 0)
            assert np.array_equal(m, np.tril(np.ones((L, L), np.uint8)))


def test_no_prefix_is_sliding_window():
    """K2e = 0: a causal band of width K1 (textbook sliding-window mask)."""
    L = 40
    for k1 in (1, 4, 39):
        m = oracle.mask_dense(L, 0, k1, 0, 0)
        band = np.tril(np.ones((L, L), np.uint8)) - np.tril(np.ones((L, L), np.uint8), -k1)
        assert np.array_equal(m, band)


def test_no_window_is_prefix_only():
    """K1 = 0 (global-only ablation, ULTRA-HSTU section 5.3.2): a row sees
    only prefix keys j < K2e, j <= i."""
    L, k2 = 20, 5
    m = oracle.mask_dense(L, 0, 0, k2, 0)
    ref = np.zeros((L, L), np.uint8)
    for i in range(L):
        ref[i, :min(k2, i + 1)] = 1
    assert np.array_equal(m, ref)


def test_contextual_prefix_extends_global_prefix():
    """effective_k2 = max(sla_k2, contextual_seq_len)."""
    L = 50
    a = oracle.mask_dense(L, 0, 6, 3, 11)
    b = oracle.mask_dense(L, 0, 6, 11, 0)
    c = oracle.mask_dense(L, 0, 6, 11, 4)
    assert np.array_equal(a, b) and np.array_equal(b, c)


def _read_mask_fixture(path):
    meta, rows = {}, []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        if len(parts) == 2 and parts[0].isidentifier():
            meta[parts[0]] = int(parts[1])
        else:
            rows.append([1 if ch == "1" else 0 for ch in line])
    return meta, np.array(rows, dtype=np.uint8)


def test_golden_mfalcon_mask():
    meta, expect = _read_mask_fixture(os.path.join(GOLDEN, "mfalcon_mask.txt"))
    m = oracle.mask_dense(meta["L"], meta["targets"], meta["k1"], meta["k2"], meta["ctx"])
    assert np.array_equal(m, expect)


def test_golden_tzrec_rows():
    path = os.path.join(GOLDEN, "sla_rows_tzrec_example.txt")
    n = 0
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = line.split()
        L, T, k1, k2, ctx, row = map(int, f[:6])
        expect = np.zeros(L, np.uint8)
        for iv in f[6:]:
            a, b = map(int, iv.split(","))
            expect[a:b] = 1
        got = np.array([oracle.visible(row, j, L, T, k1, k2, ctx) for j in range(L)],
                       dtype=np.uint8)
        assert np.array_equal(got, expect), line
        n += 1
    assert n == 7


def test_targets_do_not_change_history_rows():
    """Targets sit at the end; history rows never see them (causality)."""
    L, T = 30, 6
    with_t = oracle.mask_dense(L, T, 5, 3, 1)
    without = oracle.mask_dense(L, 0, 5, 3, 1)
    assert np.array_equal(with_t[:L - T], without[:L - T])
    # targets see no other target
    blk = with_t[L - T:, L - T:]
    assert np.array_equal(blk, np.eye(T, dtype=np.uint8))


def test_single_target_equals_plain_row():
    """With K1 >= 1, one target row has exactly the plain SLA view of that row."""
    for L in (1, 2, 9, 31):
        for k1 in (1, 2, 5, 40):
            a = oracle.mask_dense(L, 1, k1, 3, 0)
            b = oracle.mask_dense(L, 0, k1, 3, 0)
            assert np.array_equal(a, b)


def test_targets_share_one_history_view():
    """All candidates see the same history keys (M-FALCON: shared history)."""
    L, T = 40, 5
    m = oracle.mask_dense(L, T, 7, 2, 0)
    U = L - T
    for t in range(1, T):
        assert np.array_equal(m[U + t, :U], m[U, :U])


def _tiles_from_dense(lens, tg, k1, k2, ctx, bm, bn):
    out = []
    for b, (L, T) in enumerate(zip(lens, tg)):
        m = oracle.mask_dense(L, T, k1, k2, ctx)
        U = L - T
        starts = list(range(0, U, bm)) + list(range(U, L, bm))
        for r0 in starts:
            r1 = min(r0 + bm, U if r0 < U else L)
            for c0 in range(0, L, bn):
                if m[r0:r1, c0:c0 + bn].any():
                    out.append((b, r0, c0))
    return np.array(out, dtype=np.int64).reshape(-1, 3)


@pytest.mark.parametrize("bm,bn", [(4, 4), (8, 4), (4, 8), (16, 16)])
def test_tiles_match_block_reduction_of_dense_mask(bm, bn):
    rng = np.random.default_rng(bm * 100 + bn)
    for _ in range(20):
        B = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(1, 50, size=B)]
        tg = [int(rng.integers(0, L + 1)) if rng.random() < 0.4 else 0 for L in lens]
        k1, k2, ctx = int(rng.integers(0, 20)), int(rng.integers(0, 9)), int(rng.integers(0, 9))
        offs = np.concatenate([[0], np.cumsum(lens)])
        got = oracle.tiles(offs, tg, k1, k2, ctx, bm, bn)
        ref = _tiles_from_dense(lens, tg, k1, k2, ctx, bm, bn)
        assert np.array_equal(got, ref)
