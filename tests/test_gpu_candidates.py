"""GPU parity of candidate scoring against a cached history (sla_fwd_candidates,
M-FALCON) against the fp64 oracle, within the bf16 bar (2e-2 max, 5e-3 mean,
normalised by the reference RMS).  Bit-exact properties: scoring in
microbatches gives the same bits as one call, and with history lengths on a
64-key boundary the scores equal the target rows of sla_fwd over the
combined [history | candidates] layout (then both visit the same key tiles in
the same order)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_sequence_attention_amd as sla
from tests._helpers import assert_close_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).bfloat16()


def _case(seed, hist, cands, H=2, d=128, std=0.5, dv=None):
    """Seeded history keys/values and candidate q/k/v, bf16-exact values
    (values of width dv, d when not given)."""
    dv = d if dv is None else dv
    rng = np.random.default_rng(seed)
    ho = np.concatenate([[0], np.cumsum(hist)]).astype(np.int64)
    co = np.concatenate([[0], np.cumsum(cands)]).astype(np.int64)

    def mk(n, w=d):
        x = (rng.standard_normal((n, H, w), dtype=np.float32) * std)
        return torch.from_numpy(x).bfloat16().float().numpy()

    return ho, co, mk(int(ho[-1])), mk(int(ho[-1]), dv), mk(int(co[-1])), mk(int(co[-1])), \
        mk(int(co[-1]), dv)


def _gpu(ho, co, kh, vh, qc, kc, vc, kw, **extra):
    o = sla.sla_fwd_candidates(_bf(kh), _bf(vh), torch.from_numpy(ho).to(DEV), _bf(qc), _bf(kc),
                               _bf(vc), torch.from_numpy(co).to(DEV), **kw, **extra)
    torch.cuda.synchronize()
    return o


KW = dict(k1=128, k2=32, contextual_len=8, max_seq_len=2048)


@pytest.mark.parametrize("d", [64, 128])
def test_candidates_match_oracle(d):
    hist, cands = [300, 0, 1000, 129, 77], [70, 5, 300, 0, 129]
    ho, co, kh, vh, qc, kc, vc = _case(0, hist, cands, d=d)
    print(f"[case] candidates d={d} hist={hist} cands={cands}", flush=True)
    o = _gpu(ho, co, kh, vh, qc, kc, vc, KW)
    ref = oracle.sla_fwd_candidates(kh, vh, ho, qc, kc, vc, co, KW["k1"], KW["k2"],
                                    KW["contextual_len"], KW["max_seq_len"])
    mx, mn = assert_close_bf16(o.float().cpu().numpy(), ref, "o_c")
    print(f"  o_c max {mx:.3e} mean {mn:.3e}")


@pytest.mark.parametrize("d,dv", [(64, 128), (128, 32), (32, 64)])
def test_candidates_rect_heads_match_oracle(d, dv):
    """Query/key width d, value width dv (the forward's rectangular heads)."""
    hist, cands = [300, 0, 1000, 129], [70, 5, 300, 33]
    ho, co, kh, vh, qc, kc, vc = _case(3, hist, cands, d=d, dv=dv)
    print(f"[case] candidates d_qk={d} d_v={dv} hist={hist} cands={cands}", flush=True)
    o = _gpu(ho, co, kh, vh, qc, kc, vc, KW)
    assert tuple(o.shape) == (sum(cands), 2, dv)
    ref = oracle.sla_fwd_candidates(kh, vh, ho, qc, kc, vc, co, KW["k1"], KW["k2"],
                                    KW["contextual_len"], KW["max_seq_len"])
    mx, mn = assert_close_bf16(o.float().cpu().numpy(), ref, "o_c")
    print(f"  o_c max {mx:.3e} mean {mn:.3e}")


def test_candidates_equal_target_rows_of_the_forward_bitwise():
    hist, cands = [512, 64, 896], [200, 1, 128]
    ho, co, kh, vh, qc, kc, vc = _case(1, hist, cands)
    print(f"[case] candidates vs target rows hist={hist} cands={cands}", flush=True)
    o = _gpu(ho, co, kh, vh, qc, kc, vc, KW)
    # the combined layout: history rows (q arbitrary), then the candidates as targets
    rng = np.random.default_rng(9)
    q, k, v, offs, rows = [], [], [], [0], []
    for b in range(len(hist)):
        hs, cs = slice(ho[b], ho[b + 1]), slice(co[b], co[b + 1])
        q += [rng.standard_normal(kh[hs].shape).astype(np.float32), qc[cs]]
        k += [kh[hs], kc[cs]]
        v += [vh[hs], vc[cs]]
        rows += list(range(offs[-1] + hist[b], offs[-1] + hist[b] + cands[b]))
        offs.append(offs[-1] + hist[b] + cands[b])
    cat = lambda p: _bf(np.concatenate(p, 0))  # noqa: E731
    full = sla.sla_fwd(cat(q), cat(k), cat(v), torch.tensor(offs, dtype=torch.int64, device=DEV),
                       torch.tensor(cands, dtype=torch.int32, device=DEV), **KW)
    torch.cuda.synchronize()
    assert torch.equal(o, full[torch.tensor(rows, device=DEV)])


def test_microbatched_scoring_is_bitwise_equal():
    hist, cands = [700, 2000, 40], [300, 260, 17]
    ho, co, kh, vh, qc, kc, vc = _case(2, hist, cands)
    print(f"[case] candidates microbatches hist={hist} cands={cands}", flush=True)
    whole = _gpu(ho, co, kh, vh, qc, kc, vc, KW)
    bm = 64
    got = torch.empty_like(whole)
    for m0 in range(0, max(cands), bm):
        idx, offs = [], [0]
        for b in range(len(hist)):
            n = cands[b]
            sel = np.arange(co[b] + min(m0, n), co[b] + min(m0 + bm, n))
            idx.append(sel)
            offs.append(offs[-1] + len(sel))
        idx = np.concatenate(idx)
        o = _gpu(ho, np.asarray(offs, np.int64), kh, vh, qc[idx], kc[idx], vc[idx], KW)
        got[torch.from_numpy(idx).to(DEV)] = o
    assert torch.equal(got, whole)


def test_candidates_without_history_and_empty_calls():
    ho, co, kh, vh, qc, kc, vc = _case(3, [0, 0], [5, 130])
    print("[case] candidates without history", flush=True)
    o = _gpu(ho, co, kh, vh, qc, kc, vc, KW)
    ref = oracle.sla_fwd_candidates(kh, vh, ho, qc, kc, vc, co, KW["k1"], KW["k2"],
                                    KW["contextual_len"], KW["max_seq_len"])
    assert_close_bf16(o.float().cpu().numpy(), ref, "o_c")
    # no candidates at all: nothing is read or written
    ho2, co2, kh2, vh2, qc2, kc2, vc2 = _case(4, [50, 60], [0, 0])
    o2 = _gpu(ho2, co2, kh2, vh2, qc2, kc2, vc2, KW)
    assert o2.shape[0] == 0


def test_production_shape_candidates():
    """Contextual 16 + history U[8192, 16384], K1 = 1024, K2 = 128, H = 4, d = 128,
    512 candidates per sequence (4 sequences)."""
    rng = np.random.default_rng(5)
    hist = [16 + int(x) for x in rng.integers(8192, 16385, size=4)]
    cands = [512] * 4
    ho, co, kh, vh, qc, kc, vc = _case(6, hist, cands, H=4, d=128)
    kw = dict(k1=1024, k2=128, contextual_len=16, max_seq_len=16656)
    print(f"[case] candidates production hist={hist}", flush=True)
    o = _gpu(ho, co, kh, vh, qc, kc, vc, kw)
    ref = oracle.sla_fwd_candidates(kh, vh, ho, qc, kc, vc, co, kw["k1"], kw["k2"],
                                    kw["contextual_len"], kw["max_seq_len"])
    mx, mn = assert_close_bf16(o.float().cpu().numpy(), ref, "o_c")
    print(f"  o_c max {mx:.3e} mean {mn:.3e}")
