"""STU stack forward driver: a loop over stu_layer_fwd with one stu_truncate
call before the first truncated layer (ULTRA-HSTU paper, section 4.3: after
N1 full-length layers keep the most recent UIH tokens for the remaining N2).

The driver only sequences C-ABI calls.  It reads the truncated token count
back once (one device-to-host copy of new_offsets[B]) to size the following
layers' buffers.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

from . import ops
from .config import STUConfig


@dataclass
class STULayerWeights:
    ln1_w: torch.Tensor          # [D] fp32
    w_uvqk: torch.Tensor         # [2*H*dv + 2*H*dqk, D] bf16
    ln2_w: torch.Tensor          # [H*dv] fp32
    w_out: torch.Tensor          # [D, H*dv] bf16
    ln1_b: Optional[torch.Tensor] = None
    b_uvqk: Optional[torch.Tensor] = None
    ln2_b: Optional[torch.Tensor] = None
    b_out: Optional[torch.Tensor] = None
    # FP8 copies of the projection weights (e4m3 bytes and per-row scales),
    # filled by quantize_fp8() for stu_stack_fwd(fp8=True)
    w_uvqk_q: Optional[torch.Tensor] = None
    w_uvqk_scale: Optional[torch.Tensor] = None
    w_out_q: Optional[torch.Tensor] = None
    w_out_scale: Optional[torch.Tensor] = None

    def quantize_fp8(self) -> "STULayerWeights":
        self.w_uvqk_q, self.w_uvqk_scale = ops.stu_quantize_rows_fp8(self.w_uvqk)
        self.w_out_q, self.w_out_scale = ops.stu_quantize_rows_fp8(self.w_out)
        return self


@dataclass
class StackOutput:
    x: torch.Tensor
    offsets: torch.Tensor
    num_targets: Optional[torch.Tensor]
    gather_idx: Optional[torch.Tensor] = None   # source rows of the truncated layers
    layer_tokens: List[int] = field(default_factory=list)
    layer_inputs: List[torch.Tensor] = field(default_factory=list)   # with keep_layers
    layer_outputs: List[torch.Tensor] = field(default_factory=list)


def stu_stack_fwd(cfg: STUConfig, layers: List[STULayerWeights], x: torch.Tensor,
                  offsets: torch.Tensor, num_targets: Optional[torch.Tensor],
                  keep_layers: bool = False, fp8: bool = False) -> StackOutput:
    """fp8: both projections of every layer in FP8 (stu_layer_fwd_fp8), with
    the weights' FP8 copies from STULayerWeights.quantize_fp8()."""
    if len(layers) != cfg.attn_num_layers:
        raise ValueError(f"{len(layers)} layer weights for {cfg.attn_num_layers} layers")
    out = StackOutput(x=x, offsets=offsets, num_targets=num_targets)
    cur, offs, tg = x, offsets, num_targets
    for li, w in enumerate(layers):
        if cfg.truncation_enabled and li == cfg.attn_truncation_split_layer:
            xt, offs, tg, gidx = ops.stu_truncate(cur, offs, tg,
                                                  contextual_len=cfg.contextual_seq_len,
                                                  tail_len=cfg.attn_truncation_tail_len)
            n = int(offs[-1].item())
            cur = xt[:n]
            out.gather_idx = gidx[:n]
        out.layer_tokens.append(int(cur.shape[0]))
        if keep_layers:
            out.layer_inputs.append(cur)
        kw = dict(heads=cfg.num_heads, d_qk=cfg.attention_dim, d_v=cfg.hidden_dim,
                  k1=cfg.kernel_k1, k2=cfg.kernel_k2, contextual_len=cfg.contextual_seq_len,
                  max_seq_len=cfg.max_seq_len, alpha=cfg.alpha, ln_eps=cfg.ln_eps,
                  ln1_b=w.ln1_b, b_uvqk=w.b_uvqk, ln2_b=w.ln2_b, b_out=w.b_out)
        if fp8:
            if w.w_uvqk_q is None or w.w_out_q is None:
                raise ValueError(f"layer {li}: FP8 weights missing (call quantize_fp8())")
            cur = ops.stu_layer_fwd_fp8(cur, offs, tg, w.ln1_w, w.w_uvqk_q, w.w_uvqk_scale,
                                        w.ln2_w, w.w_out_q, w.w_out_scale, **kw)
        else:
            cur = ops.stu_layer_fwd(cur, offs, tg, w.ln1_w, w.w_uvqk, w.ln2_w, w.w_out, **kw)
        if keep_layers:
            out.layer_outputs.append(cur)
    out.x, out.offsets, out.num_targets = cur, offs, tg
    return out


@dataclass
class MoTChannel:
    """One channel of a Mixture of Transducers: its own STU stack (config,
    layer weights) over its own jagged sequences [contextual | UIH of this
    channel | the shared candidates]."""
    cfg: STUConfig
    layers: List[STULayerWeights]
    x: torch.Tensor
    offsets: torch.Tensor


def mot_fwd(channels: List[MoTChannel], num_targets: torch.Tensor, fp8: bool = False):
    """Mixture of Transducers (ULTRA-HSTU paper, section 4.3 and Appendix A;
    the torcheasyrec page's MoT bullet): every channel runs its own stack,
    and the channels' candidate (target) embeddings are concatenated along
    the feature dimension, channel by channel.  All channels carry the same
    candidates: num_targets [B] is shared.  Returns (emb [sum of targets,
    sum of D_c], target_offsets [B+1])."""
    if not channels:
        raise ValueError("no channels")
    outs = [stu_stack_fwd(ch.cfg, ch.layers, ch.x, ch.offsets, num_targets, fp8=fp8)
            for ch in channels]
    widths = [int(o.x.shape[1]) for o in outs]
    cap = int(channels[0].x.shape[0])
    emb = torch.empty((cap, sum(widths)), dtype=outs[0].x.dtype, device=outs[0].x.device)
    col, toffs = 0, None
    for o, w in zip(outs, widths):
        _, toffs = ops.stu_gather_targets(o.x, o.offsets, o.num_targets, out=emb, col_offset=col)
        col += w
    n = int(toffs[-1].item())
    return emb[:n], toffs
