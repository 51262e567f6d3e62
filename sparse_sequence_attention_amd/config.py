"""STU stack configuration, with the field names of the torcheasyrec
"ULTRA HSTU" model page (stu { embedding_dim num_heads hidden_dim
attention_dim sla_k1 sla_k2 } attn_num_layers attn_truncation_split_layer
attn_truncation_tail_len max_seq_len) and its validity rules:

* SLA is on when sla_k1 > 0 or sla_k2 > 0; with both 0 the layers use the full
  causal mask (here: a local window wider than any sequence);
* effective_k2 = max(sla_k2, contextual_seq_len);
* truncation is on only when both attn_truncation_split_layer and
  attn_truncation_tail_len are > 0; setting only one of them is rejected.  The
  page's example (split layer 2 of 4 keeps the tail for layers 2..3) fixes the
  indexing: layers [0, split) run on full sequences, layers [split, n) on the
  truncated ones.
"""
from __future__ import annotations

from dataclasses import dataclass

FULL_CAUSAL_K1 = 2 ** 31 - 1


@dataclass(frozen=True)
class STUConfig:
    embedding_dim: int = 512
    num_heads: int = 4
    hidden_dim: int = 128          # d_v per head
    attention_dim: int = 128       # d_qk per head
    sla_k1: int = 0
    sla_k2: int = 0
    contextual_seq_len: int = 0
    attn_num_layers: int = 1
    attn_truncation_split_layer: int = 0
    attn_truncation_tail_len: int = 0
    max_seq_len: int = 4096        # N of the 1/N attention scaling
    alpha: float = 1.0
    ln_eps: float = 1e-5

    def __post_init__(self):
        if self.sla_k1 < 0 or self.sla_k2 < 0 or self.contextual_seq_len < 0:
            raise ValueError("sla_k1, sla_k2 and contextual_seq_len must be >= 0")
        s, t = self.attn_truncation_split_layer, self.attn_truncation_tail_len
        if (s > 0) != (t > 0):
            raise ValueError("attention truncation needs both attn_truncation_split_layer and "
                             "attn_truncation_tail_len > 0")
        if s < 0 or t < 0:
            raise ValueError("truncation fields must be >= 0")
        if s > 0 and s >= self.attn_num_layers:
            raise ValueError("attn_truncation_split_layer must be < attn_num_layers")
        if self.attn_num_layers < 1 or self.max_seq_len < 1:
            raise ValueError("attn_num_layers and max_seq_len must be >= 1")

    @property
    def sla_enabled(self) -> bool:
        return self.sla_k1 > 0 or self.sla_k2 > 0

    @property
    def truncation_enabled(self) -> bool:
        return self.attn_truncation_split_layer > 0 and self.attn_truncation_tail_len > 0

    @property
    def kernel_k1(self) -> int:
        """K1 passed to the kernels (a window wider than any sequence when SLA is off)."""
        return self.sla_k1 if self.sla_enabled else FULL_CAUSAL_K1

    @property
    def kernel_k2(self) -> int:
        return self.sla_k2 if self.sla_enabled else 0

    @property
    def effective_k2(self) -> int:
        return max(self.kernel_k2, self.contextual_seq_len)

    def layer_is_truncated(self, layer: int) -> bool:
        return self.truncation_enabled and layer >= self.attn_truncation_split_layer
