"""Mixture of Transducers (ULTRA-HSTU paper, section 4.3 and Appendix A; the
torcheasyrec page's MoT bullet): channel stacks over their own sequences with
shared candidates, candidate embeddings concatenated along the features.

The gather of target rows is index work: bit-exact against direct indexing.
The MoT output is bit-exact against each channel's stack run alone, and
checked against the oracle's MoT composition (oracle.mot_fwd: the oracle's
stacks per channel, their candidate rows concatenated), bf16 and FP8
channels.  Bars: bf16 channels, the mean bar (5e-3 of the rms) and the max
bar (2e-2) widened by F, the distance between the storage-matched oracle and
the exact one.  FP8 channels: every layer of each channel's stack, applied by
the GPU to its own input, against the FP8 oracle layer with the single-layer
FP8 bars (max 5e-2 beyond one bf16 step of the stored output, mean 5e-3);
end to end, activation codes that land on the other side of an e4m3 midpoint
in the two implementations compound over the layers, so the MoT output is
reported against the FP8 oracle chain and held to the sum of its layers'
mean bars."""
import numpy as np
import pytest
import torch

import sparse_sequence_attention_amd as sla
from sparse_sequence_attention_amd.config import STUConfig
from sparse_sequence_attention_amd.stack import MoTChannel, STULayerWeights, stu_stack_fwd
import oracle
from synthetic import make_stack_workload
from tests._helpers import BF16_MAX_TOL, BF16_MEAN_TOL, bf16_ulp, rel_errors

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


def _channel(seed, hidden, heads, k1, k2, layers, split, tail, lens, ntg, host=None):
    sw = make_stack_workload(seed=seed, lengths=lens, layers=layers, hidden=hidden, heads=heads,
                             num_targets=ntg, contextual_len=8, k1=k1, k2=k2,
                             split_layer=split, tail_len=tail)
    if host is not None:   # the oracle's view of the channel
        host.update(x=sw.x, offsets=sw.offsets,
                    layers=[dict(ln1_w=sw.ln1_w[i], w_uvqk=sw.w_uvqk[i], ln2_w=sw.ln2_w[i],
                                 w_out=sw.w_out[i]) for i in range(layers)],
                    heads=heads, dqk=sw.d, dv=sw.d, k1=k1, k2=k2, ctx=8, N=sw.max_seq_len,
                    split_layer=split if split > 0 else None, tail_len=tail if split > 0 else None)
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


def _check_fp8_stack_layers(ch, host, tg, tg_host):
    o = stu_stack_fwd(ch.cfg, ch.layers, ch.x, ch.offsets, tg, keep_layers=True, fp8=True)
    torch.cuda.synchronize()
    np_ = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    for li, w in enumerate(host["layers"]):
        xin = np_(o.layer_inputs[li])
        offs = o.layer_layouts[li][0].cpu().numpy()
        ref = oracle.stu_layer_fwd_fp8(xin, offs, tg_host, w["ln1_w"], w["w_uvqk"], w["ln2_w"],
                                       w["w_out"], heads=host["heads"], dqk=host["dqk"],
                                       dv=host["dv"], k1=host["k1"], k2=host["k2"],
                                       ctx=host["ctx"], N=host["N"])
        got = np_(o.layer_outputs[li])
        rms = float(np.sqrt(np.mean(ref * ref)))
        excess = float(((np.abs(got - ref) - bf16_ulp(ref)) / rms).max())
        mx, mn = rel_errors(got, ref)
        print(f"  fp8 channel hidden {ch.cfg.embedding_dim} layer {li}: max {mx:.3e} (beyond one "
              f"bf16 step {excess:.3e}) mean {mn:.3e}", flush=True)
        assert excess <= 5e-2 and mn <= 5e-3


def test_mot_matches_oracle():
    """Two channels (hidden 512 / H = 4 with a 3-layer stack truncated before
    layer 1; hidden 256 / H = 2, 2 layers, no truncation), bf16 and FP8."""
    ntg = 16
    h0, h1 = {}, {}
    ch0 = _channel(3, 512, 4, 128, 32, 3, 1, 256, [700, 129, 1000], ntg, host=h0)
    ch1 = _channel(4, 256, 2, 64, 8, 2, 0, 0, [300, 40, 500], ntg, host=h1)
    tg_host = np.full(3, ntg, np.int32)
    tg = torch.from_numpy(tg_host).to(DEV)
    for fp8 in (False, True):
        print(f"[case] MoT vs oracle fp8={fp8}", flush=True)
        if fp8:
            for w in ch0.layers + ch1.layers:
                w.quantize_fp8()
        emb, _ = sla.mot_fwd([ch0, ch1], tg, fp8=fp8)
        torch.cuda.synchronize()
        got = emb.float().cpu().numpy().astype(np.float64)
        ref = oracle.mot_fwd([h0, h1], tg_host, fp8=fp8, store_bf16=True)
        assert got.shape == ref.shape
        if fp8:
            for ch, h in ((ch0, h0), (ch1, h1)):
                _check_fp8_stack_layers(ch, h, tg, tg_host)
            mx, mn = rel_errors(got, ref)
            n_layers = len(ch0.layers) + len(ch1.layers)
            print(f"  MoT fp8 vs FP8 oracle chain: max {mx:.3e} mean {mn:.3e}", flush=True)
            assert mn <= 5e-3 * n_layers
            continue
        exact = oracle.mot_fwd([h0, h1], tg_host, store_bf16=False)
        floor, _ = rel_errors(ref, exact)
        for what, r in (("storage-matched", ref), ("exact", exact)):
            mx, mn = rel_errors(got, r)
            print(f"  MoT bf16 vs {what} oracle: max {mx:.3e} mean {mn:.3e} (F {floor:.3e})",
                  flush=True)
            assert mn <= BF16_MEAN_TOL and mx <= BF16_MAX_TOL + floor, what
