"""Pins for the oracle's STU stack chain (ULTRA-HSTU paper, section 4.3:
attention truncation between layers) and its backward.

truncate_bwd is pinned as the adjoint of the truncation gather (the inner
product identity, exact on integer data) and by direct construction (kept rows
copy dy, dropped rows are zero).  stu_stack_bwd is pinned to central finite
differences of stu_stack_fwd, on the stack input and on weights of a layer
before and after the truncation, and to stu_layer_bwd for a one-layer stack."""
import numpy as np
import pytest

import oracle


def _layout(lens, tg):
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return offs, (None if tg is None else np.asarray(tg, np.int32))


@pytest.mark.parametrize("ctx,tail", [(2, 5), (0, 1), (3, 100)])
def test_truncate_bwd_is_the_adjoint_of_the_gather(ctx, tail):
    rng = np.random.default_rng(ctx * 10 + tail)
    lens = [20, 0, 13, 7, 40]
    tg = [3, 0, 2, 7, 0]
    offs, tgv = _layout(lens, tg)
    T, D = int(offs[-1]), 6
    new_offs, gidx = oracle.truncate(offs, tgv, ctx, tail)
    n = int(new_offs[-1])
    x = rng.integers(-50, 50, size=(T, D)).astype(np.float64)
    dy = rng.integers(-50, 50, size=(n, D)).astype(np.float64)
    dx = oracle.truncate_bwd(gidx, dy, T)
    assert dx.shape == (T, D)
    # <gather(x), dy> == <x, adjoint(dy)>, exactly (integers)
    assert float((x[gidx] * dy).sum()) == float((x * dx).sum())
    # kept rows carry their copy's gradient, dropped rows are zero
    kept = np.zeros(T, bool)
    kept[gidx] = True
    assert np.array_equal(dx[gidx], dy)
    assert not np.any(dx[~kept])
    assert len(set(gidx.tolist())) == n   # the gather is injective


def _stack_case(seed, D=16, H=2, d=4, layers=3):
    rng = np.random.default_rng(seed)
    lens, tg = [14, 9, 11], [3, 2, 0]
    offs, tgv = _layout(lens, tg)
    T = int(offs[-1])
    nw = 4 * H * d
    ws = []
    for _ in range(layers):
        ws.append(dict(
            ln1_w=1 + 0.1 * rng.standard_normal(D), ln1_b=0.1 * rng.standard_normal(D),
            w_uvqk=rng.standard_normal((nw, D)) * 0.4, b_uvqk=0.1 * rng.standard_normal(nw),
            ln2_w=1 + 0.1 * rng.standard_normal(H * d), ln2_b=0.1 * rng.standard_normal(H * d),
            w_out=rng.standard_normal((D, H * d)) * 0.3, b_out=0.1 * rng.standard_normal(D)))
    x = rng.standard_normal((T, D))
    kw = dict(heads=H, dqk=d, dv=d, k1=4, k2=2, ctx=2, N=14.0, alpha=1.0, eps=1e-5)
    return x, offs, tgv, ws, kw


def test_stack_bwd_matches_finite_differences():
    x, offs, tg, ws, kw = _stack_case(3)
    split, tail = 1, 3
    fwd = oracle.stu_stack_fwd(x, offs, tg, ws, split_layer=split, tail_len=tail, **kw)
    out = fwd["out"]
    assert out.shape[0] < x.shape[0]          # the truncation dropped rows
    rng = np.random.default_rng(4)
    dout = rng.standard_normal(out.shape)
    g = oracle.stu_stack_bwd(fwd, ws, dout, split_layer=split, **kw)
    assert g["dx"].shape == x.shape

    def loss(xx, wws):
        r = oracle.stu_stack_fwd(xx, offs, tg, wws, split_layer=split, tail_len=tail, **kw)
        return float((r["out"] * dout).sum())

    h = 1e-6
    # the input, along a random direction (rows dropped by the truncation
    # still reach the output through the layer before it)
    v = rng.standard_normal(x.shape)
    fd = (loss(x + h * v, ws) - loss(x - h * v, ws)) / (2 * h)
    got = float((g["dx"] * v).sum())
    assert abs(got - fd) <= 1e-6 * max(1.0, abs(fd)), (got, fd)
    # single weights of the layer before the truncation and of the last layer
    for li, name, key, idx in [(0, "w_out", "dw_out", (3, 2)), (0, "ln1_w", "dln1_w", (5,)),
                               (0, "w_uvqk", "dw_uvqk", (7, 1)), (2, "b_uvqk", "db_uvqk", (4,)),
                               (1, "ln2_b", "dln2_b", (1,))]:
        wp = [{k: np.array(a, copy=True) for k, a in w.items()} for w in ws]
        wp[li][name][idx] += h
        up = loss(x, wp)
        wp[li][name][idx] -= 2 * h
        dn = loss(x, wp)
        fd = (up - dn) / (2 * h)
        got = g["layers"][li][key][idx]
        assert abs(got - fd) <= 1e-6 * max(1.0, abs(fd)), (li, name, got, fd)


def test_one_layer_stack_equals_the_layer():
    x, offs, tg, ws, kw = _stack_case(5, layers=1)
    fwd = oracle.stu_stack_fwd(x, offs, tg, ws, **kw)
    w = ws[0]
    ref = oracle.stu_layer_fwd(x, offs, tg, w["ln1_w"], w["w_uvqk"], w["ln2_w"], w["w_out"],
                               ln1_b=w["ln1_b"], b_uvqk=w["b_uvqk"], ln2_b=w["ln2_b"],
                               b_out=w["b_out"], **kw)
    assert np.array_equal(fwd["out"], ref)
    dout = np.random.default_rng(6).standard_normal(ref.shape)
    g = oracle.stu_stack_bwd(fwd, ws, dout, **kw)
    gl = oracle.stu_layer_bwd(x, offs, tg, w["ln1_w"], w["w_uvqk"], w["ln2_w"], w["w_out"], dout,
                              ln1_b=w["ln1_b"], b_uvqk=w["b_uvqk"], ln2_b=w["ln2_b"],
                              b_out=w["b_out"], **kw)
    assert np.array_equal(g["dx"], gl["dx"])
    assert np.array_equal(g["layers"][0]["dw_uvqk"], gl["dw_uvqk"])


def test_truncation_at_the_first_layer_scatters_into_the_input():
    x, offs, tg, ws, kw = _stack_case(7, layers=2)
    fwd = oracle.stu_stack_fwd(x, offs, tg, ws, split_layer=0, tail_len=2, **kw)
    dout = np.random.default_rng(8).standard_normal(fwd["out"].shape)
    g = oracle.stu_stack_bwd(fwd, ws, dout, split_layer=0, **kw)
    kept = np.zeros(x.shape[0], bool)
    kept[fwd["gather_idx"]] = True
    assert not np.any(g["dx"][~kept])          # dropped input rows get no gradient
    assert np.any(g["dx"][kept])


def test_mot_is_the_concatenation_of_the_channel_candidates():
    x, offs, tg, ws, kw = _stack_case(9, layers=2)
    _, _, _, ws2, kw2 = _stack_case(10, D=8, H=1, d=4, layers=1)
    lens2 = [10, 12, 6]                       # channel 2: its own sequences,
    offs2 = np.concatenate([[0], np.cumsum(lens2)]).astype(np.int64)   # same targets
    x2 = np.random.default_rng(11).standard_normal((int(offs2[-1]), 8))
    ch1 = dict(x=x, offsets=offs, layers=ws, split_layer=1, tail_len=3, **kw)
    ch2 = dict(x=x2, offsets=offs2, layers=ws2, **kw2)
    emb = oracle.mot_fwd([ch1, ch2], tg, store_bf16=False)
    assert emb.shape == (int(tg.sum()), 16 + 8)
    r1 = oracle.stu_stack_fwd(x, offs, tg, ws, split_layer=1, tail_len=3, **kw)
    r2 = oracle.stu_stack_fwd(x2, offs2, tg, ws2, **kw2)
    # the candidates are the last num_targets rows of each sequence
    rows1 = [r for b in range(3) for r in range(int(r1["offsets"][b + 1]) - int(tg[b]),
                                                int(r1["offsets"][b + 1]))]
    rows2 = [r for b in range(3) for r in range(int(offs2[b + 1]) - int(tg[b]),
                                                int(offs2[b + 1]))]
    assert np.array_equal(emb[:, :16], r1["out"][rows1])
    assert np.array_equal(emb[:, 16:], r2["out"][rows2])
