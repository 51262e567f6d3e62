"""Mixture of Transducers (ULTRA-HSTU paper, section 4.3 and Appendix A; the
torcheasyrec page's MoT bullet): channel stacks over their own sequences with
shared candidates, candidate embeddings concatenated along the features.

The gather of target rows is index work: bit-exact against direct indexing.
The MoT output is bit-exact against each channel's stack run alone (each
stack is checked against the oracle in test_gpu_stu.py)."""
import numpy as np
import pytest
import torch

import sparse_sequence_attention_amd as sla
from sparse_sequence_attention_amd.config import STUConfig
from sparse_sequence_attention_amd.stack import MoTChannel, STULayerWeights, stu_stack_fwd
from synthetic import make_stack_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _target_rows(offsets, tg):
    rows = []
    for b in range(len(tg)):
        rows += list(range(int(offsets[b + 1]) - int(tg[b]), int(offsets[b + 1])))
    return np.asarray(rows, np.int64)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gather_targets_is_exact(dtype):
    rng = np.random.default_rng(0)
    lens = [0, 5, 300, 17, 0, 1000, 64]
    tg = [0, 5, 20, 0, 0, 1, 64]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, D = int(offs[-1]), 256
    x = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).to(DEV).to(dtype)
    o_d = torch.from_numpy(offs).to(DEV)
    t_d = torch.tensor(tg, dtype=torch.int32, device=DEV)
    print(f"[case] gather targets {dtype}", flush=True)
    out, toffs = sla.stu_gather_targets(x, o_d, t_d)
    wide = torch.full((T, 3 * D), 7.0, dtype=dtype, device=DEV)
    sla.stu_gather_targets(x, o_d, t_d, out=wide, col_offset=D)
    torch.cuda.synchronize()
    rows = torch.from_numpy(_target_rows(offs, tg)).to(DEV)
    n = rows.numel()
    assert toffs.cpu().tolist() == [0] + list(np.cumsum(tg))
    assert torch.equal(out[:n], x[rows])
    assert torch.equal(wide[:n, D:2 * D], x[rows])
    assert torch.all(wide[:n, :D] == 7.0) and torch.all(wide[:n, 2 * D:] == 7.0)


def _channel(seed, hidden, heads, k1, k2, layers, split, tail, lens, ntg):
    sw = make_stack_workload(seed=seed, lengths=lens, layers=layers, hidden=hidden, heads=heads,
                             num_targets=ntg, contextual_len=8, k1=k1, k2=k2,
                             split_layer=split, tail_len=tail)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)  # noqa: E731
    ws = [STULayerWeights(ln1_w=f(sw.ln1_w[i]), w_uvqk=f(sw.w_uvqk[i]).bfloat16(),
                          ln2_w=f(sw.ln2_w[i]), w_out=f(sw.w_out[i]).bfloat16())
          for i in range(layers)]
    cfg = STUConfig(embedding_dim=hidden, num_heads=heads, hidden_dim=sw.d, attention_dim=sw.d,
                    sla_k1=k1, sla_k2=k2, contextual_seq_len=8, attn_num_layers=layers,
                    attn_truncation_split_layer=split, attn_truncation_tail_len=tail,
                    max_seq_len=sw.max_seq_len)
    return MoTChannel(cfg=cfg, layers=ws, x=f(sw.x).bfloat16(),
                      offsets=torch.from_numpy(sw.offsets).to(DEV))


def test_mot_concatenates_channel_candidates():
    ntg = 16
    # channel 0: the engagement-like sequence (longer, truncated); channel 1:
    # a shorter sequence with its own width and windows, no truncation
    ch0 = _channel(1, 512, 4, 128, 32, 3, 1, 256, [700, 129, 1000], ntg)
    ch1 = _channel(2, 256, 2, 64, 8, 2, 0, 0, [300, 40, 500], ntg)
    tg = torch.full((3,), ntg, dtype=torch.int32, device=DEV)
    print("[case] MoT two channels", flush=True)
    for fp8 in (False, True):
        if fp8:
            for w in ch0.layers + ch1.layers:
                w.quantize_fp8()
        emb, toffs = sla.mot_fwd([ch0, ch1], tg, fp8=fp8)
        ref = []
        for ch in (ch0, ch1):
            o = stu_stack_fwd(ch.cfg, ch.layers, ch.x, ch.offsets, tg, fp8=fp8)
            rows = torch.from_numpy(_target_rows(o.offsets.cpu().numpy(), [ntg] * 3)).to(DEV)
            ref.append(o.x[rows])
        torch.cuda.synchronize()
        assert emb.shape == (3 * ntg, 512 + 256)
        assert torch.equal(emb, torch.cat(ref, dim=1)), f"fp8={fp8}"
        assert toffs.cpu().tolist() == [0, ntg, 2 * ntg, 3 * ntg]
