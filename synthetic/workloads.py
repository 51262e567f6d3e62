"""Seeded synthetic workloads for Semi-Local Attention (SLA) and the STU stack.

The shapes follow the workloads of the ULTRA-HSTU paper page ("4.2.1 Semi-local
attention design", "Appendix E.2 attention operator benchmark"; user histories
of thousands to 16K events) and the torcheasyrec UltraHSTU page (STU config
fields: embedding_dim 512, num_heads 4, hidden_dim/attention_dim 128).  Real
user histories are not available; these draws stand in for them:

* lengths: uniform integers in the stated range (numpy PCG64, one generator per
  seed, drawn first);
* Q, K, V (and dO): independent normal draws in float32, in the order
  lengths -> Q -> K -> V -> dO -> weights, then rounded to bfloat16 with
  round-to-nearest-even when the workload is bf16; the very same bits go to
  the oracle (converted exactly to fp64) and to the GPU;
* STU weights: Xavier-uniform, a = sqrt(6 / (fan_in + fan_out)); LayerNorm
  weights 1, no biases.

Nothing here computes attention, LayerNorm or masks.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional

import numpy as np


# ----------------------------------------------------------------------------
# bfloat16 storage helpers (rounding of inputs, not method arithmetic)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (round-to-nearest-even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round_f32(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class SLAConfig:
    name: str
    dtype: str                 # "f32" or "bf16"
    heads: int
    d: int
    k1: int
    k2: int
    contextual_len: int
    max_seq_len: int           # N of the 1/N scaling
    std: float                 # std of Q, K, V
    lengths: Callable[[np.random.Generator], List[int]]
    targets: Callable[[List[int]], List[int]] = lambda ls: [0] * len(ls)
    backward: bool = True
    description: str = ""


def _fixed(vals):
    return lambda rng: list(vals)


def _uniform(b, lo, hi):
    return lambda rng: [int(x) for x in rng.integers(lo, hi + 1, size=b)]


def _long_mix(rng):
    return [16384] * 4 + [int(x) for x in rng.integers(4096, 16384 + 1, size=4)]


def _targets_lengths(rng):
    uih = rng.integers(8192, 16384 + 1, size=16)
    return [int(16 + u + 256) for u in uih]


CONFIGS: Dict[str, SLAConfig] = {
    "tiny_f32": SLAConfig(
        name="tiny_f32", dtype="f32", heads=2, d=32, k1=8, k2=4, contextual_len=2,
        max_seq_len=64, std=1.0, lengths=_fixed([37, 64]), backward=False,
        description="SLA forward, fp32, B=2 lengths {37,64}, H=2, d=32, K1=8, K2=4, ctx=2"),
    "jagged_2k": SLAConfig(
        name="jagged_2k", dtype="bf16", heads=4, d=128, k1=256, k2=64, contextual_len=8,
        max_seq_len=2048, std=0.5, lengths=_uniform(32, 512, 2048),
        description="SLA fwd+bwd, bf16, B=32 lengths U[512,2048], H=4, d=128, K1=256, K2=64, ctx=8"),
    "long_16k": SLAConfig(
        name="long_16k", dtype="bf16", heads=4, d=128, k1=1024, k2=128, contextual_len=16,
        max_seq_len=16384, std=0.5, lengths=_long_mix,
        description="SLA fwd+bwd, bf16, B=8 lengths 16384x4 + U[4096,16384]x4, H=4, d=128, "
                    "K1=1024, K2=128, ctx=16"),
    "targets_16k": SLAConfig(
        name="targets_16k", dtype="bf16", heads=4, d=128, k1=1024, k2=128, contextual_len=16,
        max_seq_len=16 + 16384 + 256, std=0.5, lengths=_targets_lengths,
        targets=lambda ls: [256] * len(ls), backward=False,
        description="target-aware SLA forward, bf16, B=16, 16 ctx + UIH U[8192,16384] + 256 "
                    "targets, K1=1024, K2=128, H=4, d=128"),
}


def config_by_name(name: str) -> SLAConfig:
    return CONFIGS[name]


@dataclass
class Workload:
    cfg: SLAConfig
    seed: int
    lengths: List[int]
    num_targets: Optional[np.ndarray]   # int32 [B] or None
    offsets: np.ndarray                 # int64 [B+1]
    q: np.ndarray                       # float32 [T, H, d] (bf16-representable if bf16)
    k: np.ndarray
    v: np.ndarray
    dout: Optional[np.ndarray]
    k1: int = 0
    k2: int = 0
    contextual_len: int = 0
    max_seq_len: int = 1
    alpha: float = 1.0
    dtype: str = "bf16"          # storage type of q, k, v, dout

    @property
    def total_tokens(self) -> int:
        return int(self.offsets[-1])

    @property
    def batch(self) -> int:
        return len(self.lengths)


def _normal(rng, shape, std, dtype):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == "bf16":
        a = bf16_round_f32(a)
    return a


def make_sla_workload(cfg: SLAConfig | str, seed: int = 0, *, lengths: Optional[List[int]] = None,
                      num_targets: Optional[List[int]] = None, with_dout: Optional[bool] = None,
                      k1: Optional[int] = None, k2: Optional[int] = None,
                      contextual_len: Optional[int] = None, heads: Optional[int] = None,
                      d: Optional[int] = None, max_seq_len: Optional[int] = None,
                      dtype: Optional[str] = None, d_v: Optional[int] = None) -> Workload:
    """Draw one workload.  Keyword overrides let tests build small variants
    (d: the Q / K head width; d_v: the V and dO width, d when not given)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = np.random.default_rng(seed)
    lens = list(lengths) if lengths is not None else cfg.lengths(rng)
    tg = list(num_targets) if num_targets is not None else cfg.targets(lens)
    H = heads if heads is not None else cfg.heads
    dd = d if d is not None else cfg.d
    dt = dtype if dtype is not None else cfg.dtype
    offsets = np.zeros(len(lens) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    T = int(offsets[-1])
    q = _normal(rng, (T, H, dd), cfg.std, dt)
    k = _normal(rng, (T, H, dd), cfg.std, dt)
    dw = dd if d_v is None else d_v
    v = _normal(rng, (T, H, dw), cfg.std, dt)
    want_do = cfg.backward if with_dout is None else with_dout
    dout = _normal(rng, (T, H, dw), 1.0, dt) if want_do else None
    nt = np.asarray(tg, dtype=np.int32) if any(t != 0 for t in tg) else None
    return Workload(cfg=cfg, seed=seed, lengths=lens, num_targets=nt, offsets=offsets,
                    q=q, k=k, v=v, dout=dout,
                    k1=cfg.k1 if k1 is None else k1, k2=cfg.k2 if k2 is None else k2,
                    contextual_len=cfg.contextual_len if contextual_len is None else contextual_len,
                    max_seq_len=cfg.max_seq_len if max_seq_len is None else max_seq_len,
                    dtype=dt)


# ----------------------------------------------------------------------------
# STU stack (18 layers, hidden 512) workload
# ----------------------------------------------------------------------------
@dataclass
class StackWorkload:
    seed: int
    lengths: List[int]
    offsets: np.ndarray
    num_targets: np.ndarray
    x: np.ndarray                      # [T, D] float32, bf16-representable
    ln1_w: List[np.ndarray]
    w_uvqk: List[np.ndarray]           # [2*H*dv + 2*H*dqk, D] (out-features major)
    ln2_w: List[np.ndarray]
    w_out: List[np.ndarray]            # [D, H*dv]
    layers: int = 18
    hidden: int = 512
    heads: int = 4
    d: int = 128
    k1: int = 512
    k2: int = 64
    contextual_len: int = 16
    max_seq_len: int = 4096
    split_layer: int = 9
    tail_len: int = 1024
    ln_eps: float = 1e-5
    alpha: float = 1.0


def _xavier(rng, out_f, in_f):
    a = np.float32(np.sqrt(6.0 / (in_f + out_f)))
    w = rng.uniform(-1.0, 1.0, size=(out_f, in_f)).astype(np.float32) * a
    return bf16_round_f32(w)


def make_stack_workload(seed: int = 0, *, batch: int = 8, min_len: int = 2048,
                        max_len: int = 4096, layers: int = 18, hidden: int = 512,
                        heads: int = 4, d: int = 128, num_targets: int = 64,
                        contextual_len: int = 16, k1: int = 512, k2: int = 64,
                        split_layer: int = 9, tail_len: int = 1024,
                        lengths: Optional[List[int]] = None) -> StackWorkload:
    """18-layer STU stack, bf16 storage: x ~ N(0,1), Xavier-uniform weights."""
    rng = np.random.default_rng(seed)
    lens = list(lengths) if lengths is not None else \
        [int(x) for x in rng.integers(min_len, max_len + 1, size=batch)]
    offsets = np.zeros(len(lens) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    T = int(offsets[-1])
    x = bf16_round_f32(rng.standard_normal(size=(T, hidden), dtype=np.float32))
    n_uvqk = 2 * heads * d + 2 * heads * d
    ln1, w1, ln2, w2 = [], [], [], []
    for _ in range(layers):
        ln1.append(np.ones(hidden, dtype=np.float32))
        w1.append(_xavier(rng, n_uvqk, hidden))
        ln2.append(np.ones(heads * d, dtype=np.float32))
        w2.append(_xavier(rng, hidden, heads * d))
    return StackWorkload(seed=seed, lengths=lens, offsets=offsets,
                         num_targets=np.full(len(lens), num_targets, dtype=np.int32),
                         x=x, ln1_w=ln1, w_uvqk=w1, ln2_w=ln2, w_out=w2, layers=layers,
                         hidden=hidden, heads=heads, d=d, k1=k1, k2=k2,
                         contextual_len=contextual_len, max_seq_len=max_len,
                         split_layer=split_layer, tail_len=tail_len)
