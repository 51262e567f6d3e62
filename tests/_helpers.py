"""Shared test utilities: error metrics and a dense fp64 torch reference.

The dense reference is a second, independent formulation of the attention
(library matmuls over a full L x L mask) used only to pin the oracle.
"""
import numpy as np
import torch

import oracle


def rel_errors(got, ref):
    """(max|got-ref| / rms(ref), mean|got-ref| / rms(ref)) over the whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        rms = 1.0
    d = np.abs(got - ref)
    return float(d.max() / rms) if d.size else 0.0, float(d.mean() / rms) if d.size else 0.0


BF16_MAX_TOL = 2e-2
BF16_MEAN_TOL = 5e-3
F32_MAX_TOL = 1e-5


def assert_close_bf16(got, ref, what=""):
    mx, mn = rel_errors(got, ref)
    assert mx <= BF16_MAX_TOL and mn <= BF16_MEAN_TOL, f"{what}: max {mx:.3e} mean {mn:.3e}"
    return mx, mn


def assert_close_f32(got, ref, what=""):
    mx, mn = rel_errors(got, ref)
    assert mx <= F32_MAX_TOL, f"{what}: max {mx:.3e} mean {mn:.3e}"
    return mx, mn


def dense_sla_torch(q, k, v, offsets, num_targets, k1, k2, ctx, N, alpha=1.0):
    """O = (SiLU(alpha Q K^T) * M) V / N per sequence and head, float64 torch.

    q, k, v are torch float64 tensors [T, H, d] (requires_grad allowed)."""
    outs = []
    B = len(offsets) - 1
    for b in range(B):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        L = s1 - s0
        if L == 0:
            continue
        T = 0 if num_targets is None else int(num_targets[b])
        m = torch.from_numpy(oracle.mask_dense(L, T, k1, k2, ctx).astype(np.float64))
        qb = q[s0:s1].transpose(0, 1)          # [H, L, d]
        kb = k[s0:s1].transpose(0, 1)
        vb = v[s0:s1].transpose(0, 1)
        s = torch.matmul(qb, kb.transpose(1, 2).contiguous())
        p = torch.nn.functional.silu(alpha * s) * m / N
        outs.append(torch.matmul(p, vb).transpose(0, 1))
    return torch.cat(outs, 0) if outs else q.new_zeros((0,) + tuple(v.shape[1:]))
