"""Thin torch-facing wrappers over the C ABI (argument marshalling only).

Torch provides device memory and the current stream; every arithmetic step
runs in the HIP kernels of libsla_mi355x.so.  Names follow the C entry points.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _capi as C

_DT = {torch.bfloat16: C.SLA_BF16, torch.float32: C.SLA_F32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _head_tensor(name: str, t: torch.Tensor, T: int, H: int, dtype, width: int) -> int:
    """Check a [T, H, width] view with unit inner stride; returns the token
    stride.  The library finds head h at column h * width of a row, so a
    tensor of another width would be read at the wrong offsets."""
    if t.dim() != 3 or t.shape[0] != T or t.shape[1] != H or t.shape[2] != width:
        raise ValueError(f"{name}: expected shape [T={T}, H={H}, {width}], got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if T == 0:
        return H * t.shape[2]  # no rows: nothing is read or written
    if t.stride(2) != 1 or (H > 1 and t.stride(1) != t.shape[2]):
        raise ValueError(f"{name}: heads must be packed ([T][H][d] with token stride >= H*d)")
    return t.stride(0)


def make_problem(dtype, offsets: torch.Tensor, num_targets: Optional[torch.Tensor], T: int, H: int,
                 d_qk: int, d_v: int, k1: int, k2: int, contextual_len: int, max_seq_len: int,
                 alpha: float = 1.0, out_f32: bool = False) -> C.SLAProblem:
    if offsets.dtype != torch.int64 or offsets.dim() != 1:
        raise TypeError("offsets must be a 1-D int64 tensor [B+1]")
    if num_targets is not None and (num_targets.dtype != torch.int32 or
                                    num_targets.numel() != offsets.numel() - 1):
        raise TypeError("num_targets must be an int32 tensor [B]")
    p = C.SLAProblem()
    p.dtype = _DT[dtype] if not isinstance(dtype, int) else dtype
    p.batch = offsets.numel() - 1
    p.total_tokens = T
    p.offsets = offsets.data_ptr()
    p.num_targets = None if num_targets is None else num_targets.data_ptr()
    p.num_heads, p.d_qk, p.d_v = H, d_qk, d_v
    p.k1, p.k2, p.contextual_len = int(k1), int(k2), int(contextual_len)
    p.max_seq_len = int(max_seq_len)
    p.alpha = float(alpha)
    p.out_f32 = int(bool(out_f32))
    return p


def _out_f32(in_dtype, out_dtype) -> bool:
    """Whether a bf16 problem writes its outputs in fp32."""
    if out_dtype is None or out_dtype == in_dtype:
        return False
    if in_dtype == torch.bfloat16 and out_dtype == torch.float32:
        return True
    raise TypeError(f"outputs of a {in_dtype} problem can be {in_dtype} or float32, not {out_dtype}")


def workspace_size(p: C.SLAProblem, op: int) -> int:
    return int(C.load().sla_workspace_size(ctypes.byref(p), op))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _reused_workspace(nbytes: int, ws: Optional[torch.Tensor]) -> torch.Tensor:
    """The caller's workspace, which must already hold a schedule: never
    replaced by a fresh one."""
    if ws is None or ws.numel() * ws.element_size() < nbytes:
        raise ValueError("reuse_schedule needs the workspace of the call that built the schedule")
    return ws


def sla_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, offsets: torch.Tensor,
            num_targets: Optional[torch.Tensor] = None, *, k1: int, k2: int,
            contextual_len: int = 0, max_seq_len: int, alpha: float = 1.0,
            out: Optional[torch.Tensor] = None, out_dtype=None,
            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """O[T, H, d_v] = (1/N) (SiLU(alpha Q K^T) * M_SLA) V over jagged sequences.
    out_dtype: torch.float32 writes O in fp32 from bf16 inputs (the dtype of a
    given `out` decides when out_dtype is None)."""
    T, H, dqk = q.shape
    dv = v.shape[2]
    ldq = _head_tensor("q", q, T, H, q.dtype, dqk)
    ldk = _head_tensor("k", k, T, H, q.dtype, dqk)
    ldv = _head_tensor("v", v, T, H, q.dtype, dv)
    odt = out_dtype if out_dtype is not None else (out.dtype if out is not None else q.dtype)
    f32o = _out_f32(q.dtype, odt)
    if out is None:
        out = torch.empty((T, H, dv), dtype=odt, device=q.device)
    ldo = _head_tensor("out", out, T, H, odt, dv)
    p = make_problem(q.dtype, offsets, num_targets, T, H, dqk, dv, k1, k2, contextual_len,
                     max_seq_len, alpha, f32o)
    nbytes = workspace_size(p, C.SLA_OP_FWD)
    ws = _workspace(nbytes, q.device, workspace)
    C.check(C.load().sla_fwd(ctypes.byref(p), _ptr(q), ldq, _ptr(k), ldk, _ptr(v), ldv, _ptr(out),
                             ldo, _ptr(ws), ws.numel(), _stream(q.device)))
    return out


def sla_fwd_candidates(k_hist: torch.Tensor, v_hist: torch.Tensor, hist_offsets: torch.Tensor,
                       q_c: torch.Tensor, k_c: torch.Tensor, v_c: torch.Tensor,
                       cand_offsets: torch.Tensor, *, k1: int, k2: int, contextual_len: int = 0,
                       max_seq_len: int, alpha: float = 1.0, out: Optional[torch.Tensor] = None,
                       out_dtype=None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """O_c[C, H, d_v]: candidates scored against the cached history keys/values
    (each sees the history window of the first candidate slot and itself)."""
    Th, H, dqk = k_hist.shape
    Cn = q_c.shape[0]
    dv = v_c.shape[2]
    dt = q_c.dtype
    ldk = _head_tensor("k_hist", k_hist, Th, H, dt, dqk)
    ldv = _head_tensor("v_hist", v_hist, Th, H, dt, dv)
    ldq = _head_tensor("q_c", q_c, Cn, H, dt, dqk)
    ldkc = _head_tensor("k_c", k_c, Cn, H, dt, dqk)
    ldvc = _head_tensor("v_c", v_c, Cn, H, dt, dv)
    odt = out_dtype if out_dtype is not None else (out.dtype if out is not None else dt)
    f32o = _out_f32(dt, odt)
    if out is None:
        out = torch.empty((Cn, H, dv), dtype=odt, device=q_c.device)
    ldo = _head_tensor("out", out, Cn, H, odt, dv)
    if cand_offsets.dtype != torch.int64 or cand_offsets.numel() != hist_offsets.numel():
        raise TypeError("cand_offsets must be an int64 tensor [B+1] like hist_offsets")
    p = make_problem(dt, hist_offsets, None, Th, H, dqk, dv, k1, k2, contextual_len, max_seq_len,
                     alpha, f32o)
    lib = C.load()
    nbytes = int(lib.sla_fwd_candidates_workspace_size(ctypes.byref(p), Cn))
    ws = _workspace(nbytes, q_c.device, workspace)
    C.check(lib.sla_fwd_candidates(ctypes.byref(p), _ptr(cand_offsets), Cn, _ptr(k_hist), ldk,
                                   _ptr(v_hist), ldv, _ptr(q_c), ldq, _ptr(k_c), ldkc, _ptr(v_c),
                                   ldvc, _ptr(out), ldo, _ptr(ws), ws.numel(),
                                   _stream(q_c.device)))
    return out


def sla_bwd(q, k, v, dout, offsets, num_targets=None, *, k1: int, k2: int,
            contextual_len: int = 0, max_seq_len: int, alpha: float = 1.0, dq=None, dk=None,
            dv=None, grad_dtype=None, workspace: Optional[torch.Tensor] = None,
            stage: int = C.SLA_BWD_ALL, recompute_dq: bool = False):
    """(dQ, dK, dV) of sla_fwd given dO (stage: see sla_bwd_stage in sla.h).
    grad_dtype: torch.float32 writes the gradients in fp32 from bf16 inputs
    (the dtype of given output tensors decides when grad_dtype is None).
    The library stores dS for the dQ kernel when the workspace holds it
    (sla_workspace_size(SLA_OP_BWD), allocated here by default);
    recompute_dq=True hands it only the smallest workspace, so dQ recomputes
    S and dO.V^T instead.  A given workspace is used as it is when it holds
    at least the smallest one (its size then decides)."""
    T, H, dqk = q.shape
    dvd = v.shape[2]
    ldq = _head_tensor("q", q, T, H, q.dtype, dqk)
    ldk = _head_tensor("k", k, T, H, q.dtype, dqk)
    ldv = _head_tensor("v", v, T, H, q.dtype, dvd)
    lddo = _head_tensor("dout", dout, T, H, q.dtype, dvd)
    given = [t for t in (dq, dk, dv) if t is not None]
    gdt = grad_dtype if grad_dtype is not None else (given[0].dtype if given else q.dtype)
    f32o = _out_f32(q.dtype, gdt)
    dq = torch.empty((T, H, dqk), dtype=gdt, device=q.device) if dq is None else dq
    dk = torch.empty((T, H, dqk), dtype=gdt, device=q.device) if dk is None else dk
    dv = torch.empty((T, H, dvd), dtype=gdt, device=q.device) if dv is None else dv
    lddq = _head_tensor("dq", dq, T, H, gdt, dqk)
    lddk = _head_tensor("dk", dk, T, H, gdt, dqk)
    lddv = _head_tensor("dv", dv, T, H, gdt, dvd)
    p = make_problem(q.dtype, offsets, num_targets, T, H, dqk, dvd, k1, k2, contextual_len,
                     max_seq_len, alpha, f32o)
    small = workspace_size(p, C.SLA_OP_BWD_RECOMPUTE)
    nbytes = small if recompute_dq else workspace_size(p, C.SLA_OP_BWD)
    if workspace is not None and workspace.numel() * workspace.element_size() >= small:
        ws = workspace
    else:
        ws = _workspace(nbytes, q.device, None)
    ws_bytes = ws.numel() * ws.element_size()
    if recompute_dq:
        ws_bytes = min(ws_bytes, small)
    C.check(C.load().sla_bwd_stage(ctypes.byref(p), stage, _ptr(q), ldq, _ptr(k), ldk, _ptr(v),
                                   ldv, _ptr(dout), lddo, _ptr(dq), lddq, _ptr(dk), lddk,
                                   _ptr(dv), lddv, _ptr(ws), ws_bytes, _stream(q.device)))
    return dq, dk, dv


def sla_bwd_noalloc(q, k, v, dout, offsets, num_targets=None, *, k1: int, k2: int,
                    contextual_len: int = 0, max_seq_len: int, alpha: float = 1.0, dq, dk, dv):
    """sla_bwd for callers that cannot allocate device memory: the caller
    passes the output tensors (bf16 or fp32 from bf16 inputs), and the
    workspace is the library's static per-device array (see sla_bwd_noalloc in
    sla.h: at most SLA_NOALLOC_SCRATCH_BYTES; overlapping calls on one device
    race).  Neither this wrapper nor the call allocates device memory."""
    T, H, dqk = q.shape
    dvd = v.shape[2]
    ldq = _head_tensor("q", q, T, H, q.dtype, dqk)
    ldk = _head_tensor("k", k, T, H, q.dtype, dqk)
    ldv = _head_tensor("v", v, T, H, q.dtype, dvd)
    lddo = _head_tensor("dout", dout, T, H, q.dtype, dvd)
    gdt = dq.dtype
    lddq = _head_tensor("dq", dq, T, H, gdt, dqk)
    lddk = _head_tensor("dk", dk, T, H, gdt, dqk)
    lddv = _head_tensor("dv", dv, T, H, gdt, dvd)
    p = make_problem(q.dtype, offsets, num_targets, T, H, dqk, dvd, k1, k2, contextual_len,
                     max_seq_len, alpha, _out_f32(q.dtype, gdt))
    C.check(C.load().sla_bwd_noalloc(ctypes.byref(p), _ptr(q), ldq, _ptr(k), ldk, _ptr(v), ldv,
                                     _ptr(dout), lddo, _ptr(dq), lddq, _ptr(dk), lddk, _ptr(dv),
                                     lddv, _stream(q.device)))
    return dq, dk, dv


def sla_schedule(offsets, num_targets, *, op: int, heads: int, d: int, k1: int, k2: int,
                 contextual_len: int = 0, total_tokens: int, dtype=torch.bfloat16) -> torch.Tensor:
    """The kernels' work list as an int32 tensor [n, SLA_SCHED_RECORD_INTS] (on the device)."""
    p = make_problem(dtype, offsets, num_targets, total_tokens, heads, d, d, k1, k2,
                     contextual_len, 1)
    lib = C.load()
    cap = int(lib.sla_schedule_capacity(ctypes.byref(p), op))
    if cap < 0:
        C.check(C.SLA_ERR_INVALID)
    rec = torch.zeros((max(cap, 1), C.SLA_SCHED_RECORD_INTS), dtype=torch.int32,
                      device=offsets.device)
    cnt = torch.zeros(1, dtype=torch.int32, device=offsets.device)
    nbytes = workspace_size(p, C.SLA_OP_FWD)
    ws = _workspace(nbytes, offsets.device, None)
    C.check(lib.sla_schedule(ctypes.byref(p), op, _ptr(rec), cap, _ptr(cnt), _ptr(ws), ws.numel(),
                             _stream(offsets.device)))
    n = int(cnt.item())
    return rec[:n]


def sla_schedule_host(offsets, num_targets, *, op: int, heads: int, d: int, k1: int, k2: int,
                      contextual_len: int = 0, dtype=torch.bfloat16):
    """The work list computed on the host from host offsets (numpy int32 [n, 12])."""
    import numpy as np
    o = np.ascontiguousarray(offsets, dtype=np.int64)
    t = None if num_targets is None else np.ascontiguousarray(num_targets, dtype=np.int32)
    p = C.SLAProblem()
    p.dtype = _DT[dtype]
    p.batch = len(o) - 1
    p.total_tokens = int(o[-1])
    p.num_heads, p.d_qk, p.d_v = heads, d, d
    p.k1, p.k2, p.contextual_len, p.max_seq_len, p.alpha = int(k1), int(k2), int(contextual_len), 1, 1.0
    lib = C.load()
    tp = None if t is None else t.ctypes.data_as(ctypes.c_void_p)
    n = lib.sla_schedule_host(ctypes.byref(p), op, o.ctypes.data_as(ctypes.c_void_p), tp, None, 0)
    if n < 0:
        raise ValueError(lib.sla_last_error().decode())
    rec = np.zeros((max(n, 1), C.SLA_SCHED_RECORD_INTS), dtype=np.int32)
    lib.sla_schedule_host(ctypes.byref(p), op, o.ctypes.data_as(ctypes.c_void_p), tp,
                          rec.ctypes.data_as(ctypes.c_void_p), n)
    return rec[:n]


def ds_blocks_host(offsets, num_targets, *, k1: int, k2: int, contextual_len: int = 0):
    """The stored-dS blocks of one head in block order, from host offsets
    (numpy int64 [n, 3]: sequence, first row of the 64-row step, first key of
    the 128-key tile)."""
    import numpy as np
    o = np.ascontiguousarray(offsets, dtype=np.int64)
    t = None if num_targets is None else np.ascontiguousarray(num_targets, dtype=np.int32)
    p = C.SLAProblem()
    p.dtype = C.SLA_BF16
    p.batch = len(o) - 1
    p.total_tokens = int(o[-1])
    p.num_heads, p.d_qk, p.d_v = 1, 128, 128
    p.k1, p.k2, p.contextual_len, p.max_seq_len, p.alpha = int(k1), int(k2), int(contextual_len), 1, 1.0
    lib = C.load()
    tp = None if t is None else t.ctypes.data_as(ctypes.c_void_p)
    n = lib.sla_ds_blocks_host(ctypes.byref(p), o.ctypes.data_as(ctypes.c_void_p), tp, None, 0)
    if n < 0:
        raise ValueError(lib.sla_last_error().decode())
    out = np.zeros((max(n, 1), 3), dtype=np.int64)
    lib.sla_ds_blocks_host(ctypes.byref(p), o.ctypes.data_as(ctypes.c_void_p), tp,
                           out.ctypes.data_as(ctypes.c_void_p), n)
    return out[:n]


def schedule_tile(op: int, which: int) -> int:
    return int(C.load().sla_schedule_tile(op, which))


def count_pairs_host(offsets, num_targets, k1: int, k2: int, contextual_len: int) -> int:
    """Visible (row, key) pairs per head from host copies of offsets / num_targets."""
    import numpy as np
    o = np.ascontiguousarray(offsets, dtype=np.int64)
    t = None if num_targets is None else np.ascontiguousarray(num_targets, dtype=np.int32)
    n = C.load().sla_count_pairs_host(len(o) - 1, o.ctypes.data_as(ctypes.c_void_p),
                                      None if t is None else t.ctypes.data_as(ctypes.c_void_p),
                                      int(k1), int(k2), int(contextual_len))
    if n < 0:
        raise ValueError("invalid offsets / num_targets / window sizes")
    return int(n)


def probe_mfma_peak(iters: int = 4096, device=None) -> dict:
    """bf16 dense MFMA rate measured on the current device with an MFMA-only
    kernel, and the shader clock during it (sla_probe_mfma_peak)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    tf, ghz = ctypes.c_double(0.0), ctypes.c_double(0.0)
    lib = C.load()
    with torch.cuda.device(dev):
        nbytes = int(lib.sla_probe_scratch_size())
    if nbytes <= 0:
        C.check(C.SLA_ERR_DEVICE)
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    C.check(lib.sla_probe_mfma_peak(int(iters), _ptr(scratch), nbytes, ctypes.byref(tf),
                                    ctypes.byref(ghz), _stream(dev)))
    return {"tflops": tf.value, "sclk_ghz": ghz.value}


ISSUE_PROBE_MODES = ("mfma_only", "fma_only", "split_waves", "mixed_waves", "split_waves_agpr",
                     "exp_only", "rcp_only")


def probe_issue_rates(iters: int = 4096, device=None) -> dict:
    """Durations (ms) of the issue-rate probe's arrangements on the current
    device (sla_probe_issue_rates), and two ratios derived from them: the
    share of the shorter of MFMA-only and FMA-only that a SIMD hides when one
    wave issues the MFMAs and the other the FMAs (1 = full overlap, 0 = none),
    and the time of a transcendental relative to an FMA."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    lib = C.load()
    with torch.cuda.device(dev):
        nbytes = int(lib.sla_probe_scratch_size())
    if nbytes <= 0:
        C.check(C.SLA_ERR_DEVICE)
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ms = (ctypes.c_double * len(ISSUE_PROBE_MODES))()
    C.check(lib.sla_probe_issue_rates(int(iters), _ptr(scratch), nbytes, ms, len(ms), _stream(dev)))
    r = {k: ms[i] for i, k in enumerate(ISSUE_PROBE_MODES)}
    tm, tv = r["mfma_only"], r["fma_only"]
    for k in ("split_waves", "mixed_waves", "split_waves_agpr"):
        r["hidden_" + k] = (tm + tv - r[k]) / min(tm, tv)
    r["exp_per_fma"] = r["exp_only"] / tv
    r["rcp_per_fma"] = r["rcp_only"] / tv
    return r


class SLAFunction(torch.autograd.Function):
    """Autograd wrapper: forward sla_fwd, backward sla_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, offsets, num_targets, k1, k2, contextual_len, max_seq_len, alpha):
        ctx.save_for_backward(q, k, v, offsets, num_targets)
        ctx.args = (k1, k2, contextual_len, max_seq_len, alpha)
        return sla_fwd(q, k, v, offsets, num_targets, k1=k1, k2=k2, contextual_len=contextual_len,
                       max_seq_len=max_seq_len, alpha=alpha)

    @staticmethod
    def backward(ctx, dout):
        q, k, v, offsets, num_targets = ctx.saved_tensors
        k1, k2, cl, n, alpha = ctx.args
        dq, dk, dv = sla_bwd(q, k, v, dout.contiguous(), offsets, num_targets, k1=k1, k2=k2,
                             contextual_len=cl, max_seq_len=n, alpha=alpha)
        return dq, dk, dv, None, None, None, None, None, None, None


def sla_attention(q, k, v, offsets, num_targets=None, *, k1, k2, contextual_len=0, max_seq_len,
                  alpha=1.0):
    return SLAFunction.apply(q, k, v, offsets, num_targets, k1, k2, contextual_len, max_seq_len,
                             alpha)


# ---------------------------------------------------------------------------
# STU layer and truncation
# ---------------------------------------------------------------------------
def stu_layer_fwd(x: torch.Tensor, offsets: torch.Tensor, num_targets: Optional[torch.Tensor],
                  ln1_w: torch.Tensor, w_uvqk: torch.Tensor, ln2_w: torch.Tensor,
                  w_out: torch.Tensor, *, heads: int, d_qk: int, d_v: int, k1: int, k2: int,
                  contextual_len: int, max_seq_len: int, alpha: float = 1.0,
                  ln_eps: float = 1e-5, ln1_b=None, b_uvqk=None, ln2_b=None, b_out=None,
                  out: Optional[torch.Tensor] = None, want_uvqk: bool = False,
                  want_attn: bool = False, workspace: Optional[torch.Tensor] = None,
                  reuse_schedule: bool = False):
    """One STU layer forward (bf16): LN -> UVQK GEMM + SiLU -> SLA -> LN(A)*U -> GEMM + x.

    Returns out, then uvqk [T, NW] if want_uvqk, then the attention output
    A [T, H*d_v] if want_attn (what stu_layer_bwd keeps from the forward).
    reuse_schedule: the given workspace holds this layout's attention
    schedule from an earlier layer call (STU_REUSE_SCHEDULE in sla.h)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise TypeError("x must be a contiguous bf16 [T, D] tensor")
    T, D = x.shape
    nw = 2 * heads * d_v + 2 * heads * d_qk
    for name, w, shape in (("w_uvqk", w_uvqk, (nw, D)), ("w_out", w_out, (D, heads * d_v))):
        if tuple(w.shape) != shape or w.dtype != torch.bfloat16 or not w.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bf16 tensor of shape {shape}")
    vecs = [ln1_w, ln1_b, b_uvqk, ln2_w, ln2_b, b_out]
    for v_ in vecs:
        if v_ is not None and (v_.dtype != torch.float32 or not v_.is_contiguous()):
            raise TypeError("LayerNorm weights and biases must be contiguous float32 tensors")
    d = C.STULayerDesc()
    d.attn = make_problem(torch.bfloat16, offsets, num_targets, T, heads, d_qk, d_v, k1, k2,
                          contextual_len, max_seq_len, alpha)
    d.hidden = D
    d.ln_eps = float(ln_eps)
    d.flags = C.STU_REUSE_SCHEDULE if reuse_schedule else 0
    lib = C.load()
    nbytes = int(lib.stu_layer_workspace_size(ctypes.byref(d)))
    ws = _reused_workspace(nbytes, workspace) if reuse_schedule else \
        _workspace(nbytes, x.device, workspace)
    out = torch.empty_like(x) if out is None else out
    uvqk = torch.empty((T, nw), dtype=torch.bfloat16, device=x.device) if want_uvqk else None
    attn = torch.empty((T, heads * d_v), dtype=torch.bfloat16, device=x.device) if want_attn else None
    C.check(lib.stu_layer_fwd(ctypes.byref(d), _ptr(x), _ptr(ln1_w), _ptr(ln1_b), _ptr(w_uvqk),
                              _ptr(b_uvqk), _ptr(ln2_w), _ptr(ln2_b), _ptr(w_out), _ptr(b_out),
                              _ptr(out), _ptr(uvqk), _ptr(attn), _ptr(ws), ws.numel(),
                              _stream(x.device)))
    extra = tuple(t for t, want in ((uvqk, want_uvqk), (attn, want_attn)) if want)
    return (out,) + extra if extra else out


def stu_quantize_rows_fp8(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Row-wise e4m3 quantisation of a contiguous bf16 [R, C] matrix:
    (q uint8 [R, C] holding e4m3 bytes, scale float32 [R]), x ~ q * scale."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous() or not x.is_cuda:
        raise TypeError("x must be a contiguous bf16 [R, C] GPU tensor")
    R, Cn = x.shape
    q = torch.empty((R, Cn), dtype=torch.uint8, device=x.device)
    sc = torch.empty(R, dtype=torch.float32, device=x.device)
    C.check(C.load().stu_quantize_rows_fp8(_ptr(x), R, Cn, _ptr(q), _ptr(sc), _stream(x.device)))
    return q, sc


def stu_layer_fwd_fp8(x: torch.Tensor, offsets: torch.Tensor, num_targets: Optional[torch.Tensor],
                      ln1_w: torch.Tensor, w_uvqk_q: torch.Tensor, w_uvqk_scale: torch.Tensor,
                      ln2_w: torch.Tensor, w_out_q: torch.Tensor, w_out_scale: torch.Tensor, *,
                      heads: int, d_qk: int, d_v: int, k1: int, k2: int, contextual_len: int,
                      max_seq_len: int, alpha: float = 1.0, ln_eps: float = 1e-5, ln1_b=None,
                      b_uvqk=None, ln2_b=None, b_out=None, out: Optional[torch.Tensor] = None,
                      want_uvqk: bool = False, want_attn: bool = False,
                      workspace: Optional[torch.Tensor] = None,
                      reuse_schedule: bool = False):
    """stu_layer_fwd with both projections in FP8 (weights from
    stu_quantize_rows_fp8).  Returns out (then uvqk, attn if asked)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise TypeError("x must be a contiguous bf16 [T, D] tensor")
    T, D = x.shape
    nu = heads * d_v
    nw = 2 * nu + 2 * heads * d_qk
    for name, w, shape in (("w_uvqk_q", w_uvqk_q, (nw, D)), ("w_out_q", w_out_q, (D, nu))):
        if tuple(w.shape) != shape or w.dtype != torch.uint8 or not w.is_contiguous():
            raise TypeError(f"{name} must be a contiguous uint8 (e4m3) tensor of shape {shape}")
    for name, sc, n in (("w_uvqk_scale", w_uvqk_scale, nw), ("w_out_scale", w_out_scale, D)):
        if sc.dtype != torch.float32 or sc.numel() != n or not sc.is_contiguous():
            raise TypeError(f"{name} must be a contiguous float32 tensor of {n} scales")
    for v_ in (ln1_w, ln1_b, b_uvqk, ln2_w, ln2_b, b_out):
        if v_ is not None and (v_.dtype != torch.float32 or not v_.is_contiguous()):
            raise TypeError("LayerNorm weights and biases must be contiguous float32 tensors")
    d = C.STULayerDesc()
    d.attn = make_problem(torch.bfloat16, offsets, num_targets, T, heads, d_qk, d_v, k1, k2,
                          contextual_len, max_seq_len, alpha)
    d.hidden = D
    d.ln_eps = float(ln_eps)
    d.flags = C.STU_REUSE_SCHEDULE if reuse_schedule else 0
    lib = C.load()
    nbytes = int(lib.stu_layer_fp8_workspace_size(ctypes.byref(d)))
    ws = _reused_workspace(nbytes, workspace) if reuse_schedule else \
        _workspace(nbytes, x.device, workspace)
    out = torch.empty_like(x) if out is None else out
    uvqk = torch.empty((T, nw), dtype=torch.bfloat16, device=x.device) if want_uvqk else None
    attn = torch.empty((T, nu), dtype=torch.bfloat16, device=x.device) if want_attn else None
    C.check(lib.stu_layer_fwd_fp8(ctypes.byref(d), _ptr(x), _ptr(ln1_w), _ptr(ln1_b),
                                  _ptr(w_uvqk_q), _ptr(w_uvqk_scale), _ptr(b_uvqk), _ptr(ln2_w),
                                  _ptr(ln2_b), _ptr(w_out_q), _ptr(w_out_scale), _ptr(b_out),
                                  _ptr(out), _ptr(uvqk), _ptr(attn), _ptr(ws), ws.numel(),
                                  _stream(x.device)))
    extra = tuple(t for t, want in ((uvqk, want_uvqk), (attn, want_attn)) if want)
    return (out,) + extra if extra else out


def stu_layer_workspace_bytes(T: int, D: int, offsets: torch.Tensor,
                              num_targets: Optional[torch.Tensor], *, heads: int, d_qk: int,
                              d_v: int, k1: int, k2: int, contextual_len: int, max_seq_len: int,
                              alpha: float = 1.0, backward: bool = False,
                              fp8: bool = False) -> int:
    """Workspace bytes of stu_layer_fwd (stu_layer_bwd, stu_layer_fwd_fp8) for T
    tokens of width D."""
    d = C.STULayerDesc()
    d.attn = make_problem(torch.bfloat16, offsets, num_targets, T, heads, d_qk, d_v, k1, k2,
                          contextual_len, max_seq_len, alpha)
    d.hidden = D
    d.ln_eps = 1e-5
    lib = C.load()
    fn = lib.stu_layer_bwd_workspace_size if backward else \
        lib.stu_layer_fp8_workspace_size if fp8 else lib.stu_layer_workspace_size
    return int(fn(ctypes.byref(d)))


def stu_layer_bwd(x: torch.Tensor, dout: torch.Tensor, offsets: torch.Tensor,
                  num_targets: Optional[torch.Tensor], ln1_w: torch.Tensor, w_uvqk: torch.Tensor,
                  ln2_w: torch.Tensor, w_out: torch.Tensor, *, heads: int, d_qk: int, d_v: int,
                  k1: int, k2: int, contextual_len: int, max_seq_len: int, alpha: float = 1.0,
                  ln_eps: float = 1e-5, ln1_b=None, b_uvqk=None, ln2_b=None, b_out=None,
                  attn: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Gradients of stu_layer_fwd given dout, as a dict: dx (bf16 [T, D]) and the
    fp32 parameter gradients dln1_w, dw_uvqk, dln2_w, dw_out, plus dln1_b,
    db_uvqk, dln2_b, db_out for the biases that are given.  attn: the saved
    attention output (stu_layer_fwd(want_attn=True)); recomputed when None."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise TypeError("x must be a contiguous bf16 [T, D] tensor")
    if dout.shape != x.shape or dout.dtype != torch.bfloat16 or not dout.is_contiguous():
        raise TypeError("dout must be a contiguous bf16 tensor shaped like x")
    T, D = x.shape
    nu = heads * d_v
    nw = 2 * nu + 2 * heads * d_qk
    for name, w, shape in (("w_uvqk", w_uvqk, (nw, D)), ("w_out", w_out, (D, nu))):
        if tuple(w.shape) != shape or w.dtype != torch.bfloat16 or not w.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bf16 tensor of shape {shape}")
    if attn is not None and (tuple(attn.shape) != (T, nu) or attn.dtype != torch.bfloat16 or
                             not attn.is_contiguous()):
        raise TypeError(f"attn must be a contiguous bf16 tensor of shape {(T, nu)}")
    for v_ in (ln1_w, ln1_b, b_uvqk, ln2_w, ln2_b, b_out):
        if v_ is not None and (v_.dtype != torch.float32 or not v_.is_contiguous()):
            raise TypeError("LayerNorm weights and biases must be contiguous float32 tensors")
    d = C.STULayerDesc()
    d.attn = make_problem(torch.bfloat16, offsets, num_targets, T, heads, d_qk, d_v, k1, k2,
                          contextual_len, max_seq_len, alpha)
    d.hidden = D
    d.ln_eps = float(ln_eps)
    lib = C.load()
    nbytes = int(lib.stu_layer_bwd_workspace_size(ctypes.byref(d)))
    ws = _workspace(nbytes, x.device, workspace)
    f32 = dict(dtype=torch.float32, device=x.device)
    g = {"dx": torch.empty_like(x), "dln1_w": torch.empty(D, **f32),
         "dw_uvqk": torch.empty((nw, D), **f32), "dln2_w": torch.empty(nu, **f32),
         "dw_out": torch.empty((D, nu), **f32)}
    for name, bias, n in (("dln1_b", ln1_b, D), ("db_uvqk", b_uvqk, nw), ("dln2_b", ln2_b, nu),
                          ("db_out", b_out, D)):
        if bias is not None:
            g[name] = torch.empty(n, **f32)
    C.check(lib.stu_layer_bwd(
        ctypes.byref(d), _ptr(x), _ptr(attn), _ptr(ln1_w), _ptr(ln1_b), _ptr(w_uvqk), _ptr(b_uvqk),
        _ptr(ln2_w), _ptr(ln2_b), _ptr(w_out), _ptr(b_out), _ptr(dout), _ptr(g["dx"]),
        _ptr(g["dln1_w"]), _ptr(g.get("dln1_b")), _ptr(g["dw_uvqk"]), _ptr(g.get("db_uvqk")),
        _ptr(g["dln2_w"]), _ptr(g.get("dln2_b")), _ptr(g["dw_out"]), _ptr(g.get("db_out")),
        _ptr(ws), ws.numel(), _stream(x.device)))
    return g


def stu_gather_targets(x: torch.Tensor, offsets: torch.Tensor, num_targets: torch.Tensor,
                       out: Optional[torch.Tensor] = None, col_offset: int = 0,
                       capacity: Optional[int] = None):
    """(out, target_offsets): the last num_targets[b] rows of every sequence of
    x [T, D], in order, written to columns [col_offset, col_offset + D) of out
    [capacity, W] (allocated [capacity, D] when None; capacity defaults to T)."""
    if x.dim() != 2 or not x.is_contiguous() or x.dtype not in _DT:
        raise TypeError("x must be a contiguous bf16 or float32 [T, D] tensor")
    T, D = x.shape
    if num_targets is None or num_targets.dtype != torch.int32:
        raise TypeError("num_targets must be an int32 tensor [B]")
    B = offsets.numel() - 1
    cap = T if capacity is None else int(capacity)
    if out is None:
        out = torch.empty((cap, D), dtype=x.dtype, device=x.device)
    if out.dtype != x.dtype or out.dim() != 2 or out.stride(1) != 1:
        raise TypeError("out must be a row-major [rows, W] tensor of x's dtype")
    toffs = torch.empty(B + 1, dtype=torch.int64, device=x.device)
    C.check(C.load().stu_gather_targets(B, T, _ptr(offsets), _ptr(num_targets), _ptr(x), D,
                                        _DT[x.dtype], _ptr(toffs), _ptr(out), out.stride(0),
                                        int(col_offset), min(cap, out.shape[0]),
                                        _stream(x.device)))
    return out, toffs


def stu_truncate(x: Optional[torch.Tensor], offsets: torch.Tensor,
                 num_targets: Optional[torch.Tensor], *, contextual_len: int, tail_len: int,
                 capacity: Optional[int] = None, want_gather: bool = True):
    """(x_out [capacity, D] or None, new_offsets [B+1], new_num_targets [B], gather_idx).

    Rows past the new total (new_offsets[-1], on the device) are left unwritten."""
    B = offsets.numel() - 1
    T = int(x.shape[0]) if x is not None else None
    if capacity is None:
        if x is None:
            raise ValueError("capacity is required without x")
        capacity = T
    total = T if T is not None else capacity
    dev = offsets.device
    new_offsets = torch.empty(B + 1, dtype=torch.int64, device=dev)
    new_nt = torch.empty(max(B, 1), dtype=torch.int32, device=dev)
    gidx = torch.empty(max(capacity, 1), dtype=torch.int64, device=dev) if want_gather else None
    x_out = None
    dtype_code, hidden = C.SLA_BF16, 0
    if x is not None:
        if x.dim() != 2 or not x.is_contiguous():
            raise TypeError("x must be a contiguous [T, D] tensor")
        dtype_code = _DT[x.dtype]
        hidden = x.shape[1]
        x_out = torch.empty((capacity, hidden), dtype=x.dtype, device=dev)
    C.check(C.load().stu_truncate(B, total, _ptr(offsets), _ptr(num_targets), int(contextual_len),
                                  int(tail_len), _ptr(x), hidden, dtype_code, _ptr(new_offsets),
                                  _ptr(new_nt), _ptr(gidx), _ptr(x_out), int(capacity),
                                  _stream(dev)))
    return x_out, new_offsets, new_nt[:B], gidx


def stu_truncate_bwd(dy: torch.Tensor, offsets: torch.Tensor, num_targets: Optional[torch.Tensor],
                     new_offsets: torch.Tensor, *, contextual_len: int, tail_len: int,
                     total_tokens: int, dx: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gradient of stu_truncate's input rows given dy, the gradient of its kept
    rows (rows of dy past new_offsets[-1] are not read): dx [total_tokens, D],
    each kept row's gradient at its source row, zeros for dropped rows."""
    if dy.dim() != 2 or not dy.is_contiguous():
        raise TypeError("dy must be a contiguous [rows, D] tensor")
    B = offsets.numel() - 1
    hidden = dy.shape[1]
    if dx is None:
        dx = torch.empty((total_tokens, hidden), dtype=dy.dtype, device=dy.device)
    if tuple(dx.shape) != (total_tokens, hidden) or dx.dtype != dy.dtype or not dx.is_contiguous():
        raise TypeError("dx must be a contiguous [total_tokens, D] tensor of dy's dtype")
    C.check(C.load().stu_truncate_bwd(B, int(total_tokens), _ptr(offsets), _ptr(num_targets),
                                      int(contextual_len), int(tail_len), _ptr(new_offsets),
                                      _ptr(dy), hidden, _DT[dy.dtype], _ptr(dx),
                                      _stream(dy.device)))
    return dx
