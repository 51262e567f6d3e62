"""fp64 CPU oracle for Semi-Local Attention and the STU layer (ctypes binding).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg are the only code that may import this package.  The product
library never loads it; it shares no code with the HIP path.

The arithmetic lives in ``sla_oracle.c`` (plain C, fp64); this module builds it
with gcc and converts numpy arrays to fp64 before each call.

Functions whose results are "parity pinned" and the pins (tests/test_oracle_*):
  visible / mask_dense / count_pairs / tiles  -- closed-form pair count, golden
      masks, textbook special cases (full causal, sliding window, prefix only).
  sla_fwd   -- dense numpy/torch fp64 reference, invariants (perturbation,
      linearity, 1/N scaling, jagged independence, target permutation).
  sla_bwd   -- central finite differences of sla_fwd, torch fp64 autograd.
  layernorm / stu_layer_fwd -- torch fp64 functional composition, W2 = 0.
  stu_layer_bwd -- torch fp64 autograd of that composition; central finite
      differences of stu_layer_fwd; dout = 0 gives zero gradients.
  stu_layer_bwd(store_bf16=True) -- torch fp64 autograd of the composition
      with bf16 rounding of every stored value and of its gradient.
  sla_fwd_candidates -- dense fp64 torch reference and sla_fwd's target rows
      on the combined [history | candidates] layout; microbatch invariance;
      candidates do not see each other.
  round_e4m3 / quant_rows_fp8 -- torch's float32 -> float8_e4m3fn conversion;
      a nearest-value search over the e4m3 table (fp64 decision) and over
      numpy's fp32 quotients (fp32 decision); the row maximum maps to 448.
  stu_layer_fwd_fp8 -- a torch fp64 composition that quantises with torch's
      float8_e4m3fn conversion; FP8 error against the bf16 layer.
  truncate  -- direct set construction, identity when tail >= history.
  truncate_bwd -- the adjoint identity of the gather (exact on integers);
      kept rows copy dy, dropped rows are zero.
  stu_stack_fwd / stu_stack_bwd -- central finite differences of the stack
      (input and weights before and after the truncation); a one-layer
      stack equals stu_layer_fwd / stu_layer_bwd.
  target_rows / mot_fwd -- composition of the pinned stacks: one channel
      gives that stack's candidate rows; channels concatenate in order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile sla_oracle.c into liboracle.so with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_visible.argtypes = [i64] * 7
        lib.oracle_visible.restype = ctypes.c_int
        lib.oracle_mask_dense.argtypes = [i64, i64, i64, i64, i64, P]
        lib.oracle_mask_dense.restype = None
        lib.oracle_count_pairs.argtypes = [i32, P, P, i64, i64, i64]
        lib.oracle_count_pairs.restype = i64
        lib.oracle_tiles.argtypes = [i32, P, P, i64, i64, i64, i64, i64, P, i64]
        lib.oracle_tiles.restype = i64
        lib.oracle_sla_fwd.argtypes = [i32, P, P, i32, i32, i32, i64, i64, i64, dbl, dbl,
                                       P, P, P, P, P]
        lib.oracle_sla_fwd.restype = None
        lib.oracle_sla_bwd.argtypes = [i32, P, P, i32, i32, i32, i64, i64, i64, dbl, dbl,
                                       P, P, P, P, P, P, P, P, P]
        lib.oracle_sla_bwd.restype = None
        lib.oracle_sla_fwd_candidates.argtypes = [i32, P, P, i32, i32, i32, i64, i64, i64,
                                                  dbl, dbl, P, P, P, P, P, P]
        lib.oracle_sla_fwd_candidates.restype = None
        lib.oracle_round_bf16.argtypes = [dbl]
        lib.oracle_round_bf16.restype = dbl
        lib.oracle_layernorm.argtypes = [i64, i64, P, P, P, dbl, P]
        lib.oracle_layernorm.restype = None
        lib.oracle_stu_layer_fwd.argtypes = [i32, P, P, i32, i32, i32, i32, i64, i64, i64,
                                             dbl, dbl, dbl, P, P, P, P, P, P, P, P, P,
                                             i32, P, P]
        lib.oracle_stu_layer_fwd.restype = None
        lib.oracle_stu_layer_bwd.argtypes = [i32, P, P, i32, i32, i32, i32, i64, i64, i64,
                                             dbl, dbl, dbl] + [P] * 10 + [i32] + [P] * 9
        lib.oracle_stu_layer_bwd.restype = None
        lib.oracle_round_e4m3.argtypes = [dbl]
        lib.oracle_round_e4m3.restype = dbl
        lib.oracle_quant_rows_fp8.argtypes = [i64, i64, P, P, P, i32]
        lib.oracle_quant_rows_fp8.restype = None
        lib.oracle_stu_layer_fwd_fp8.argtypes = [i32, P, P, i32, i32, i32, i32, i64, i64, i64,
                                                 dbl, dbl, dbl] + [P] * 11
        lib.oracle_stu_layer_fwd_fp8.restype = None
        lib.oracle_truncate.argtypes = [i32, P, P, i64, i64, P, P]
        lib.oracle_truncate.restype = i64
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _offs(offsets):
    return np.ascontiguousarray(offsets, dtype=np.int64)


def _tg(num_targets):
    return None if num_targets is None else np.ascontiguousarray(num_targets, dtype=np.int32)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def visible(i, j, L, num_targets, k1, k2, ctx) -> bool:
    return bool(_load().oracle_visible(i, j, L, num_targets, k1, k2, ctx))


def mask_dense(L, num_targets, k1, k2, ctx) -> np.ndarray:
    out = np.zeros((L, L), dtype=np.uint8)
    _load().oracle_mask_dense(L, num_targets, k1, k2, ctx, _ptr(out))
    return out


def count_pairs(offsets, num_targets, k1, k2, ctx) -> int:
    o = _offs(offsets)
    t = _tg(num_targets)
    return int(_load().oracle_count_pairs(len(o) - 1, _ptr(o), _ptr(t), k1, k2, ctx))


def tiles(offsets, num_targets, k1, k2, ctx, bm, bn) -> np.ndarray:
    """Non-empty (b, row_tile_start, key_tile_start) triples, int64 [n, 3]."""
    o = _offs(offsets)
    t = _tg(num_targets)
    lib = _load()
    n = lib.oracle_tiles(len(o) - 1, _ptr(o), _ptr(t), k1, k2, ctx, bm, bn, None, 0)
    out = np.zeros((max(n, 1), 3), dtype=np.int64)
    lib.oracle_tiles(len(o) - 1, _ptr(o), _ptr(t), k1, k2, ctx, bm, bn, _ptr(out), n)
    return out[:n]


def sla_fwd_candidates(k_hist, v_hist, hist_offsets, q_c, k_c, v_c, cand_offsets, k1, k2, ctx,
                       N, alpha=1.0) -> np.ndarray:
    """O_c [C, H, dv] in fp64: each candidate scored against the history keys
    the first candidate position sees, plus itself (M-FALCON)."""
    k_hist, v_hist = _f64(k_hist), _f64(v_hist)
    q_c, k_c, v_c = _f64(q_c), _f64(k_c), _f64(v_c)
    C, H, dqk = q_c.shape
    dv = v_c.shape[2]
    o = np.zeros((C, H, dv), dtype=np.float64)
    ho, co = _offs(hist_offsets), _offs(cand_offsets)
    assert len(ho) == len(co)
    _load().oracle_sla_fwd_candidates(len(ho) - 1, _ptr(ho), _ptr(co), H, dqk, dv, k1, k2, ctx,
                                      float(N), float(alpha), _ptr(k_hist), _ptr(v_hist),
                                      _ptr(q_c), _ptr(k_c), _ptr(v_c), _ptr(o))
    return o


def sla_fwd(q, k, v, offsets, num_targets, k1, k2, ctx, N, alpha=1.0,
            row_sel: Optional[np.ndarray] = None) -> np.ndarray:
    """O [T, H, dv] in fp64.  q, k: [T, H, dqk]; v: [T, H, dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, dqk = q.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv), dtype=np.float64)
    offs, tg = _offs(offsets), _tg(num_targets)
    sel = None if row_sel is None else np.ascontiguousarray(row_sel, dtype=np.uint8)
    _load().oracle_sla_fwd(len(offs) - 1, _ptr(offs), _ptr(tg), H, dqk, dv, k1, k2, ctx,
                           float(N), float(alpha), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                           _ptr(sel))
    return o


def sla_bwd(q, k, v, dout, offsets, num_targets, k1, k2, ctx, N, alpha=1.0,
            q_sel=None, k_sel=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dQ, dK, dV) in fp64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    T, H, dqk = q.shape
    dv = v.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    offs, tg = _offs(offsets), _tg(num_targets)
    qs = None if q_sel is None else np.ascontiguousarray(q_sel, dtype=np.uint8)
    ks = None if k_sel is None else np.ascontiguousarray(k_sel, dtype=np.uint8)
    _load().oracle_sla_bwd(len(offs) - 1, _ptr(offs), _ptr(tg), H, dqk, dv, k1, k2, ctx,
                           float(N), float(alpha), _ptr(q), _ptr(k), _ptr(v), _ptr(do),
                           _ptr(dq), _ptr(dk), _ptr(dvv), _ptr(qs), _ptr(ks))
    return dq, dk, dvv


def round_bf16(x: float) -> float:
    return float(_load().oracle_round_bf16(float(x)))


def layernorm(x, w, b=None, eps=1e-5) -> np.ndarray:
    x = _f64(x)
    rows, cols = x.shape
    y = np.zeros_like(x)
    _load().oracle_layernorm(rows, cols, _ptr(x), _ptr(_f64(w)),
                             None if b is None else _ptr(_f64(b)), float(eps), _ptr(y))
    return y


def stu_layer_fwd(x, offsets, num_targets, ln1_w, w_uvqk, ln2_w, w_out, *, heads, dqk, dv,
                  k1, k2, ctx, N, alpha=1.0, eps=1e-5, ln1_b=None, b_uvqk=None, ln2_b=None,
                  b_out=None, store_bf16=False, want_uvqk=False):
    x = _f64(x)
    T, D = x.shape
    out = np.zeros_like(x)
    nw = 2 * heads * dv + 2 * heads * dqk
    uvqk = np.zeros((T, nw), dtype=np.float64) if want_uvqk else None
    offs, tg = _offs(offsets), _tg(num_targets)
    keep = [_f64(a) if a is not None else None
            for a in (ln1_w, ln1_b, w_uvqk, b_uvqk, ln2_w, ln2_b, w_out, b_out)]
    _load().oracle_stu_layer_fwd(len(offs) - 1, _ptr(offs), _ptr(tg), D, heads, dqk, dv, k1,
                                 k2, ctx, float(N), float(alpha), float(eps), _ptr(x),
                                 *[_ptr(a) for a in keep], _store_mask(store_bf16), _ptr(out),
                                 _ptr(uvqk))
    return (out, uvqk) if want_uvqk else out


def stu_layer_bwd(x, offsets, num_targets, ln1_w, w_uvqk, ln2_w, w_out, dout, *, heads, dqk,
                  dv, k1, k2, ctx, N, alpha=1.0, eps=1e-5, ln1_b=None, b_uvqk=None, ln2_b=None,
                  b_out=None, store_bf16=False):
    """Gradients of stu_layer_fwd's output given dout, as a dict: dx [T, D],
    dln1_w / dln1_b [D], dw_uvqk [NW, D], db_uvqk [NW], dln2_w / dln2_b [H*dv],
    dw_out [D, H*dv], db_out [D] (fp64; the forward is recomputed in fp64).
    store_bf16: round to bf16 every activation and gradient a bf16
    implementation stores between steps (n, z, U/V/Q/K, A, y, dy, dU, dA, dQ,
    dK, dV, dz, dn, dx); the exact chain otherwise."""
    x = _f64(x)
    T, D = x.shape
    nu = heads * dv
    nw = 2 * nu + 2 * heads * dqk
    g = dict(dx=np.zeros_like(x), dln1_w=np.zeros(D), dln1_b=np.zeros(D),
             dw_uvqk=np.zeros((nw, D)), db_uvqk=np.zeros(nw), dln2_w=np.zeros(nu),
             dln2_b=np.zeros(nu), dw_out=np.zeros((D, nu)), db_out=np.zeros(D))
    offs, tg = _offs(offsets), _tg(num_targets)
    keep = [_f64(a) if a is not None else None
            for a in (ln1_w, ln1_b, w_uvqk, b_uvqk, ln2_w, ln2_b, w_out, b_out)]
    do = _f64(dout)
    _load().oracle_stu_layer_bwd(len(offs) - 1, _ptr(offs), _ptr(tg), D, heads, dqk, dv, k1,
                                 k2, ctx, float(N), float(alpha), float(eps), _ptr(x),
                                 *[_ptr(a) for a in keep], _ptr(do), int(bool(store_bf16)),
                                 *[_ptr(g[k]) for k in ("dx", "dln1_w", "dln1_b", "dw_uvqk",
                                                         "db_uvqk", "dln2_w", "dln2_b",
                                                         "dw_out", "db_out")])
    return g


def round_e4m3(x) -> np.ndarray:
    """Nearest FP8 E4M3 (e4m3fn) values, ties to even, saturating at +-448."""
    f = _load().oracle_round_e4m3
    return np.vectorize(lambda v: f(float(v)), otypes=[np.float64])(np.asarray(x, np.float64))


def quant_rows_fp8(x, decision: str = "fp32") -> Tuple[np.ndarray, np.ndarray]:
    """(q [R, C] e4m3 values, scale [R]) with x ~ q * scale[:, None].

    decision: "fp32" takes 448 / max|x|, the product and the scale as fp32
    operations (the kernels' precision, used for every comparison with them);
    "fp64" gives the nearest e4m3 value of the fp64 quotient."""
    if decision not in ("fp32", "fp64"):
        raise ValueError("decision must be 'fp32' or 'fp64'")
    x = _f64(x)
    R, Cn = x.shape
    q = np.zeros_like(x)
    sc = np.zeros(R)
    _load().oracle_quant_rows_fp8(R, Cn, _ptr(x), _ptr(q), _ptr(sc), int(decision == "fp32"))
    return q, sc


def stu_layer_fwd_fp8(x, offsets, num_targets, ln1_w, w_uvqk, ln2_w, w_out, *, heads, dqk, dv,
                      k1, k2, ctx, N, alpha=1.0, eps=1e-5, ln1_b=None, b_uvqk=None, ln2_b=None,
                      b_out=None, want_uvqk=False):
    """The STU layer with both projections in FP8 (row-wise quantised n, y and
    weights; bf16 storage elsewhere).  Returns out [T, D] (and uvqk)."""
    x = _f64(x)
    T, D = x.shape
    nw = 2 * heads * dv + 2 * heads * dqk
    out = np.zeros_like(x)
    uvqk = np.zeros((T, nw)) if want_uvqk else None
    offs, tg = _offs(offsets), _tg(num_targets)
    keep = [_f64(a) if a is not None else None
            for a in (ln1_w, ln1_b, w_uvqk, b_uvqk, ln2_w, ln2_b, w_out, b_out)]
    _load().oracle_stu_layer_fwd_fp8(len(offs) - 1, _ptr(offs), _ptr(tg), D, heads, dqk, dv, k1,
                                     k2, ctx, float(N), float(alpha), float(eps), _ptr(x),
                                     *[_ptr(a) for a in keep], _ptr(out), _ptr(uvqk))
    return (out, uvqk) if want_uvqk else out


def _store_mask(store_bf16) -> int:
    """True -> 3 (every storage point bf16); an int is passed through as the mask
    (1 = branch tensors n, U/V/Q/K, A, y; 2 = layer output)."""
    if isinstance(store_bf16, bool) or store_bf16 is None:
        return 3 if store_bf16 else 0
    return int(store_bf16)


def truncate(offsets, num_targets, ctx, tail_len):
    """(new_offsets [B+1], gather_idx [T']) as int64."""
    offs, tg = _offs(offsets), _tg(num_targets)
    B = len(offs) - 1
    new_offs = np.zeros(B + 1, dtype=np.int64)
    gidx = np.zeros(max(int(offs[-1]), 1), dtype=np.int64)
    n = _load().oracle_truncate(B, _ptr(offs), _ptr(tg), ctx, tail_len, _ptr(new_offs),
                                _ptr(gidx))
    return new_offs, gidx[:n].copy()


def truncate_bwd(gather_idx, dy, total_tokens):
    """Adjoint of the truncation gather (ULTRA-HSTU paper, section 4.3: the
    truncated layers see a subset of the rows, in order).  The forward copies
    source row gather_idx[r] to row r, so the gradient of each kept source row
    is the gradient of its copy and every dropped row gets zero:
    dx [total_tokens, ...] with dx[gather_idx[r]] = dy[r]."""
    gidx = np.asarray(gather_idx, dtype=np.int64)
    dy = _f64(dy)
    dx = np.zeros((int(total_tokens),) + dy.shape[1:])
    np.add.at(dx, gidx, dy)
    return dx


def stu_stack_fwd(x, offsets, num_targets, layers, *, heads, dqk, dv, k1, k2, ctx, N,
                  split_layer=None, tail_len=None, alpha=1.0, eps=1e-5, store_bf16=False,
                  fp8=False):
    """The STU stack (ULTRA-HSTU paper, section 4.3): len(layers) layers of
    stu_layer_fwd, with the attention truncation (keep the contextual prefix,
    the last tail_len history tokens and the targets) applied to the input of
    layer split_layer when it is given.  layers: dicts of the stu_layer_fwd
    weights (ln1_w, w_uvqk, ln2_w, w_out and optional biases).  Returns a dict:
    out (the last layer's output), offsets (the final layout), gather_idx and
    source_rows (the truncation's source row of each kept row, and the row
    count before it; absent without truncation), and per layer its input and
    its layout (inputs, layouts: lists of (offsets, num_targets))."""
    cur, offs = _f64(x), _offs(offsets)
    tg = None if num_targets is None else _tg(num_targets)
    res = dict(inputs=[], layouts=[])
    for li, w in enumerate(layers):
        if split_layer is not None and li == split_layer:
            res["source_rows"] = cur.shape[0]
            offs, gidx = truncate(offs, tg, ctx, tail_len)
            cur = cur[gidx]
            res["gather_idx"] = gidx
        res["inputs"].append(cur)
        res["layouts"].append((offs, tg))
        layer = stu_layer_fwd_fp8 if fp8 else stu_layer_fwd
        extra = {} if fp8 else dict(store_bf16=store_bf16)
        cur = layer(cur, offs, tg, w["ln1_w"], w["w_uvqk"], w["ln2_w"], w["w_out"],
                    heads=heads, dqk=dqk, dv=dv, k1=k1, k2=k2, ctx=ctx, N=N, alpha=alpha,
                    eps=eps, ln1_b=w.get("ln1_b"), b_uvqk=w.get("b_uvqk"),
                    ln2_b=w.get("ln2_b"), b_out=w.get("b_out"), **extra)
    res["out"], res["offsets"] = cur, offs
    return res


def target_rows(x, offsets, num_targets):
    """The last num_targets[b] rows of every sequence b, in order (the
    candidate tokens): [sum of num_targets, ...]."""
    offs = _offs(offsets)
    rows = [r for b in range(len(offs) - 1)
            for r in range(int(offs[b + 1]) - int(num_targets[b]), int(offs[b + 1]))]
    return _f64(x)[np.asarray(rows, dtype=np.int64)]


def mot_fwd(channels, num_targets, *, fp8=False, store_bf16=True):
    """Mixture of Transducers (ULTRA-HSTU paper, section 4.3 and Appendix A;
    the torcheasyrec page's MoT bullet): each channel runs its own stack over
    its own sequences (which all end in the same candidates), and the
    channels' candidate rows are concatenated along the features, channel by
    channel.  channels: dicts with x, offsets, layers and the stu_stack_fwd
    keywords (heads, dqk, dv, k1, k2, ctx, N, split_layer, tail_len).
    Returns [sum of num_targets, sum of the channel widths]."""
    outs = []
    for ch in channels:
        kw = {k: v for k, v in ch.items() if k not in ("x", "offsets", "layers")}
        r = stu_stack_fwd(ch["x"], ch["offsets"], num_targets, ch["layers"], fp8=fp8,
                          store_bf16=store_bf16, **kw)
        outs.append(target_rows(r["out"], r["offsets"], num_targets))
    return np.concatenate(outs, axis=1)


def stu_stack_bwd(fwd, layers, dout, *, heads, dqk, dv, k1, k2, ctx, N, split_layer=None,
                  alpha=1.0, eps=1e-5, store_bf16=False):
    """Gradients of stu_stack_fwd's output given dout, by the chain rule over
    the layers in reverse: each layer's stu_layer_bwd at its saved input and
    layout, and at the truncation the adjoint of its gather (truncate_bwd).
    fwd: the dict stu_stack_fwd returned.  Returns dict(dx [rows of the stack
    input, D], layers=[per-layer gradient dicts])."""
    g = _f64(dout)
    grads = [None] * len(layers)
    for li in reversed(range(len(layers))):
        w = layers[li]
        offs, tg = fwd["layouts"][li]
        r = stu_layer_bwd(fwd["inputs"][li], offs, tg, w["ln1_w"], w["w_uvqk"], w["ln2_w"],
                          w["w_out"], g, heads=heads, dqk=dqk, dv=dv, k1=k1, k2=k2, ctx=ctx, N=N,
                          alpha=alpha, eps=eps, ln1_b=w.get("ln1_b"), b_uvqk=w.get("b_uvqk"),
                          ln2_b=w.get("ln2_b"), b_out=w.get("b_out"), store_bf16=store_bf16)
        grads[li] = r
        g = r["dx"]
        if split_layer is not None and li == split_layer:
            # copies and zeros only: nothing to round
            g = truncate_bwd(fwd["gather_idx"], g, fwd["source_rows"])
    return dict(dx=g, layers=grads)
