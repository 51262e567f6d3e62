/*
 * sla.h -- C ABI of the MI355X (gfx950) Semi-Local Attention library.
 *
 * The library computes, on one GPU, the hot path of ULTRA-HSTU's sequence
 * encoder:
 *   - HSTU pointwise attention A = (SiLU(alpha Q K^T) (.) M) V / N over jagged
 *     sequences (ULTRA-HSTU paper, section 3 Eq.3; HSTU notes, section 2.4
 *     Eq.2: pointwise SiLU, no softmax), under the semi-local mask M of
 *     section 4.2.1 Eq.7: row i sees key j iff
 *        j <= i  and  (i - j < K1  or  j < K2e),   K2e = max(K2, contextual_len)
 *     (effective_k2 rule of the torcheasyrec "ULTRA HSTU" page), and target
 *     (candidate) rows see only the history and themselves (HSTU notes, Q8,
 *     M-FALCON mask): a target row i >= U sees j == i, or a history key j < U
 *     with (U - j < K1 or j < K2e), where U = L - num_targets is the first
 *     target slot;
 *   - its backward (dQ, dK, dV);
 *   - one STU layer forward around it (ULTRA-HSTU paper, section 3 Eq.1-5,
 *     operation order of Code Listing 1);
 *   - attention truncation between layers (ULTRA-HSTU paper, section 4.3;
 *     torcheasyrec page, truncation bullet).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers are DEVICE pointers unless marked "host".  The caller allocates and
 * owns every buffer, workspace included; the library never allocates or frees
 * device memory and keeps no device state between calls (one exception:
 * sla_bwd_noalloc's static workspace array).  All work is enqueued
 * on the caller's stream (hipStream_t passed as void*; NULL = default stream)
 * without any host synchronisation; outputs are valid once the stream reaches
 * that point.  Calls are thread-safe.
 *
 * Jagged layout: sequence b owns tokens [offsets[b], offsets[b+1]) of every
 * [T, ...] tensor.  offsets is int64 [B+1], offsets[0] = 0, non-decreasing,
 * offsets[B] = total_tokens.  num_targets is int32 [B] (or NULL = no targets),
 * 0 <= num_targets[b] <= L_b; targets are the last num_targets[b] tokens.
 * These device-resident facts are trusted (checking them needs a sync),
 * unless the environment variable SLA_VALIDATE is set to a value other than
 * "0": then sla_fwd, sla_fwd_candidates (both layouts), sla_bwd,
 * sla_bwd_stage, sla_schedule, stu_layer_fwd, stu_layer_fwd_fp8, stu_layer_bwd
 * and stu_truncate first run a check kernel on the caller's stream, synchronise
 * it, and return SLA_ERR_INVALID (message: which fact, which sequence) before
 * any other kernel when offsets[0] != 0, offsets decrease, offsets[B] !=
 * total_tokens, a num_targets[b] lies outside [0, L_b], or (stu_truncate)
 * contextual_len + num_targets[b] > L_b for a sequence that keeps history.
 * The check borrows the first 8 bytes of the workspace (of new_offsets for
 * stu_truncate) and is a debugging aid: it costs a synchronisation per call
 * and cannot be captured in a graph.
 *
 * Per-head tensors are [T][H][d] row-major with a token stride ld (elements)
 * >= H*d, so Q/K/V/U may be strided column blocks of one fused projection
 * buffer; head h of token t starts at element t*ld + h*d.
 *
 * Errors: every call returns sla_status_t and never throws.  Host-checkable
 * problems are rejected before any HIP call; the message of the last failure
 * on the calling thread is available from sla_last_error().
 */
#ifndef SLA_MI355X_H
#define SLA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SLA_OK = 0,
    SLA_ERR_NULL = 1,        /* a required pointer is NULL                        */
    SLA_ERR_INVALID = 2,     /* negative size, ld < H*d, max_seq_len < 1, ...     */
    SLA_ERR_UNSUPPORTED = 3, /* head dim / dtype / alignment the kernels lack     */
    SLA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than *_workspace_size   */
    SLA_ERR_HIP = 5,         /* a HIP runtime call or kernel launch failed        */
    SLA_ERR_DEVICE = 6       /* the current device is not gfx950                  */
} sla_status_t;

typedef enum { SLA_F32 = 0, SLA_BF16 = 1 } sla_dtype_t;

/* One SLA problem.  Host struct, read during the call only. */
typedef struct {
    int32_t dtype;               /* sla_dtype_t of Q, K, V, O, dO, dQ, dK, dV       */
    int32_t batch;               /* B >= 0                                          */
    int64_t total_tokens;        /* T = offsets[B] (host-known: the tensor shape)   */
    const int64_t *offsets;      /* device int64 [B+1]                              */
    const int32_t *num_targets;  /* device int32 [B], or NULL                       */
    int32_t num_heads;           /* H >= 1                                          */
    int32_t d_qk;                /* head dim of Q and K: 32, 64 or 128              */
    int32_t d_v;                 /* head dim of V and O: 32, 64 or 128 (any pair    */
                                 /* with d_qk)                                      */
    int32_t k1;                  /* local window K1 >= 0 (keys, the row included)   */
    int32_t k2;                  /* global prefix K2 >= 0                           */
    int32_t contextual_len;      /* contextual prefix >= 0; K2e = max(k2, this)     */
    int32_t max_seq_len;         /* N of the 1/N output scaling, >= 1               */
    float alpha;                 /* pre-activation factor: SiLU(alpha * q.k)        */
    int32_t out_f32;             /* 0 or 1.  With dtype SLA_BF16 and 1, the outputs */
                                 /* O (sla_fwd, sla_fwd_candidates) and dQ, dK, dV  */
                                 /* (sla_bwd) are written as fp32 (their token      */
                                 /* strides in fp32 elements); inputs stay bf16.    */
                                 /* Ignored for SLA_F32.  The STU layer entry       */
                                 /* points require 0.                               */
} sla_problem_t;

/* Operation selector for sla_workspace_size and the schedule inspection
 * calls: FWD = row tiles (forward and dQ), BWD = key tiles (dK/dV).
 * BWD_RECOMPUTE (sla_workspace_size only): the smallest backward workspace. */
enum { SLA_OP_FWD = 0, SLA_OP_BWD = 1, SLA_OP_BWD_RECOMPUTE = 2 };

/* Bytes of device workspace sla_fwd (op = SLA_OP_FWD) or sla_bwd
 * (op = SLA_OP_BWD) needs for problem p: the on-device tile schedule (about
 * 20 bytes per sequence) and, for the backward, the fp32 partial dK|dV sums
 * of the split global-prefix key tiles (at most 4 key tiles of 128 keys per
 * sequence, each cut into at most 16 row chunks: up to
 * 64 * 128 * H * (d_qk + d_v) * 4 bytes per sequence, about 17 MB for 8
 * sequences, 4 heads, d = 128).  On the bf16 path with d_qk >= 64,
 * SLA_OP_BWD adds room for dS: the dK/dV kernel stores the bf16 dS of every
 * visited 64-row x 128-key tile (16 KB each, per head) and the dQ kernel
 * reads it back instead of recomputing S and dO.V^T (an upper bound from
 * the sizes: 1.19 GB for 110K tokens in 8 sequences, 4 heads, K1 = 1024,
 * K2 = 128, of which 1.08 GB are written).  That room is only requested
 * where it stays within 16 times the bytes of Q, K, V and dO (windows K1
 * up to about 8K at d = 128); otherwise, and with SLA_OP_BWD_RECOMPUTE,
 * the size is the schedule and partials only, with which sla_bwd
 * recomputes in the dQ kernel.  Depends only on host-known fields.
 * Returns 0 if p is invalid. */
size_t sla_workspace_size(const sla_problem_t *p, int op);

/* SLA forward (ULTRA-HSTU paper, section 4.2.1 Eq.6-7 with Eq.3):
 *   O[i] = (1/N) * sum_{j visible from i} SiLU(alpha * q_i . k_j) * v_j
 * q, k: [T][H][d_qk] with token strides ldq, ldk; v: [T][H][d_v] (ldv);
 * o: [T][H][d_v] (ldo), fully written for every token (rows of empty
 * sequences do not exist).  bf16 path: bf16 inputs, bf16 MFMA products with
 * fp32 accumulation, SiLU in fp32, P rounded to bf16 for the P.V product; O
 * in bf16, or fp32 with p->out_f32 (bf16 shares fp32's exponent range, so no
 * range limit beyond fp32's applies).  f32 path: fp32 throughout.  Only the non-empty tiles of the local band, the global prefix
 * and (for targets) the diagonal are visited.
 * Errors: NULL -> SLA_ERR_NULL; bad sizes/strides -> SLA_ERR_INVALID; head dims
 * not in {32,64,128}, ld or pointer not 16-byte aligned ->
 * SLA_ERR_UNSUPPORTED; ws_bytes < sla_workspace_size(p, SLA_OP_FWD) ->
 * SLA_ERR_WORKSPACE. */
sla_status_t sla_fwd(const sla_problem_t *p, const void *q, int64_t ldq, const void *k,
                     int64_t ldk, const void *v, int64_t ldv, void *o, int64_t ldo,
                     void *workspace, size_t ws_bytes, void *stream);

/* SLA backward: given dO, the gradients of the forward above,
 *   dV_j = (1/N) sum_i a_ij dO_i,            a_ij = SiLU(alpha s_ij), s_ij = q_i.k_j
 *   dS_ij = (1/N) (dO_i . v_j) alpha SiLU'(alpha s_ij)
 *   dQ_i = sum_j dS_ij k_j,   dK_j = sum_i dS_ij q_i
 * over visible pairs only.  dq/dk/dv may be strided column blocks of one
 * buffer (no concatenation needed, ULTRA-HSTU paper section 4.2.2).  Every
 * output row is written (zero where a token sees / is seen by nothing).  No
 * atomics: dK/dV are owned by key tiles, dQ by row tiles; the global-prefix
 * key tiles are split over row chunks whose fp32 partial sums are added in a
 * fixed order, so results are bitwise reproducible run to run.  dQ reads the
 * bf16 dS the dK/dV kernel stored when ws_bytes >= sla_workspace_size(p,
 * SLA_OP_BWD) includes room for it, and recomputes S and dO.V^T for its
 * rows when ws_bytes is smaller (at least SLA_OP_BWD_RECOMPUTE's size); the
 * dS it uses is the same bf16 rounding either way.  bf16 path: bf16 MFMA products with fp32
 * accumulation; P and dS enter the dV, dK and dQ products rounded to bf16,
 * except on key tiles that hold global-prefix keys (j < K2e), whose dV and dK
 * sums run over every later row: there P and dS enter as the sum of two bf16
 * numbers (16 significant bits).  Outputs bf16, or fp32 with p->out_f32.
 * Errors as sla_fwd, with ws_bytes checked against SLA_OP_BWD. */
sla_status_t sla_bwd(const sla_problem_t *p, const void *q, int64_t ldq, const void *k,
                     int64_t ldk, const void *v, int64_t ldv, const void *dout, int64_t lddo,
                     void *dq, int64_t lddq, void *dk, int64_t lddk, void *dv, int64_t lddv,
                     void *workspace, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid allocation): sla_bwd with
 * the same arguments, kernels and results as sla_bwd given a workspace of
 * SLA_NOALLOC_SCRATCH_BYTES, minus the workspace argument (so dS is stored
 * where its room fits in that size, and recomputed by dQ otherwise).  Its
 * workspace is a static device array of SLA_NOALLOC_SCRATCH_BYTES (64 MiB)
 * that the library holds on each device it runs on until the process ends
 * (its address is looked up on the first call on each device).  The call
 * allocates and frees nothing.  A problem whose sla_workspace_size(p,
 * SLA_OP_BWD_RECOMPUTE) exceeds the array -> SLA_ERR_WORKSPACE (about 117K
 * tokens with a one-tile global prefix at H = 4, d = 128).  Every call on one device shares
 * that device's array and leaves its contents behind; nothing in it needs to
 * start at zero, but calls that overlap on one device (two streams, two
 * threads) race on it and must be serialised by the caller.  Other errors as
 * sla_bwd. */
#define SLA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
sla_status_t sla_bwd_noalloc(const sla_problem_t *p, const void *q, int64_t ldq, const void *k,
                             int64_t ldk, const void *v, int64_t ldv, const void *dout,
                             int64_t lddo, void *dq, int64_t lddq, void *dk, int64_t lddk,
                             void *dv, int64_t lddv, void *stream);

/* The backward in stages: sla_bwd(...) equals, on one stream,
 *   sla_bwd_stage(SLA_BWD_PREPARE)  tile schedule (workspace)
 *   sla_bwd_stage(SLA_BWD_DKDV)     dK, dV (key-tile kernel + prefix reduce)
 *   sla_bwd_stage(SLA_BWD_DQ)       dQ (row-tile kernel)
 * with identical arguments and workspace; PREPARE first, then DKDV, then DQ
 * (with the stored-dS workspace DQ reads the dS that DKDV wrote; with the
 * recompute workspace the two only read the schedule and may run in either
 * order).  A stage ignores the output pointers it does not write (they may
 * be NULL).  SLA_BWD_ALL runs all three. */
enum { SLA_BWD_ALL = 0, SLA_BWD_PREPARE = 1, SLA_BWD_DKDV = 2, SLA_BWD_DQ = 3 };
sla_status_t sla_bwd_stage(const sla_problem_t *p, int stage, const void *q, int64_t ldq,
                           const void *k, int64_t ldk, const void *v, int64_t ldv,
                           const void *dout, int64_t lddo, void *dq, int64_t lddq, void *dk,
                           int64_t lddk, void *dv, int64_t lddv, void *workspace,
                           size_t ws_bytes, void *stream);

/* Schedule inspection (the integer part of the hot path, exposed so that it
 * can be checked bit for bit).  Writes the work list the kernels of `op` run:
 *   op = SLA_OP_FWD: row-tile items (forward and dQ kernels)
 *   op = SLA_OP_BWD: key-tile items (dK/dV kernel)
 * as int32 records of SLA_SCHED_RECORD_INTS fields into `records` (device,
 * capacity `capacity` records) and the record count into `*count` (device
 * int32).  Record fields:
 *   [0] b  [1] tile_lo  [2] tile_hi    (rows for FWD, keys for BWD; tokens
 *                                       within sequence b, [lo, hi))
 *   [3] n_ranges (0..3)
 *   [4..9] up to 3 half-open ranges of the other operand, in tokens within b:
 *        FWD: key ranges visited, each a union of whole key tiles of
 *             sla_schedule_tile(op, 1) keys (last tile clipped at L_b);
 *        BWD: row ranges visited (history rows, target rows), split into the
 *             chunk this record covers;
 *   [10] chunk index, [11] number of chunks of this key tile (1 = unsplit).
 * Returns SLA_ERR_INVALID if capacity is below sla_schedule_capacity(p, op). */
#define SLA_SCHED_RECORD_INTS 12
int64_t sla_schedule_capacity(const sla_problem_t *p, int op);
int32_t sla_schedule_tile(int op, int which /*0 = stationary tile, 1 = moving tile*/);
sla_status_t sla_schedule(const sla_problem_t *p, int op, int32_t *records, int64_t capacity,
                          int32_t *count, void *workspace, size_t ws_bytes, void *stream);

/* The same work list computed on the host from HOST copies of offsets [B+1]
 * and num_targets [B] (nullable); p->offsets / p->num_targets are ignored.
 * Writes at most `capacity` records (records may be NULL to count only) and
 * returns the number of records, or -1 on invalid input. */
int64_t sla_schedule_host(const sla_problem_t *p, int op, const int64_t *offsets_host,
                          const int32_t *num_targets_host, int32_t *records, int64_t capacity);

/* The dS blocks the backward stores with the stored-dS workspace (one head's
 * worth; the same for every head), from HOST copies of offsets [B+1] and
 * num_targets [B] (nullable): for each sequence b and each 128-key tile in
 * key order, the 64-row steps of the rows that see the tile (history steps
 * from row 0, then target steps from the first target row), as int64 triples
 * (b, first row of the step, first key of the tile) in block order.  These
 * are exactly the (64-row step, 128-key tile) pairs holding a visible pair.
 * Writes at most `capacity` triples (blocks may be NULL to count only) and
 * returns the number of blocks, or -1 on invalid input. */
int64_t sla_ds_blocks_host(const sla_problem_t *p, const int64_t *offsets_host,
                           const int32_t *num_targets_host, int64_t *blocks, int64_t capacity);

/* Useful work: number of visible (row, key) pairs per head, summed over the
 * batch, from HOST copies of offsets [B+1] and num_targets [B] (nullable).
 * Useful FLOPs are this count times H times 2*(d_qk+d_v) (forward) and
 * 2*(3*d_qk+2*d_v) (backward).  Returns -1 on invalid input. */
int64_t sla_count_pairs_host(int32_t batch, const int64_t *offsets_host,
                             const int32_t *num_targets_host, int32_t k1, int32_t k2,
                             int32_t contextual_len);

/* Candidate scoring against a cached history (M-FALCON; HSTU notes, section
 * 2.6; the target rows of the ULTRA-HSTU mask): the history's keys and values
 * are computed once, and any number of candidates, in microbatches of the
 * caller's choosing, are scored against them.  p describes the history:
 * batch B, total_tokens = T_hist, offsets [B+1] of the history tokens, heads,
 * d, k1, k2, contextual_len, max_seq_len N, alpha; p->num_targets must be
 * NULL and p->dtype SLA_BF16.  cand_offsets (device int64 [B+1], offsets[0]
 * = 0, non-decreasing, offsets[B] = total_candidates) lays out the
 * candidates of each sequence.  Candidate c of sequence b (history length
 * U_b) gets
 *   o_c = (1/N) ( sum over history keys j with U_b - j < K1 or j < K2eff of
 *                 SiLU(alpha q_c . k_j) v_j  +  SiLU(alpha q_c . k_c) v_c ),
 * i.e. the row of a target placed right after the history.  Candidates never
 * see each other, and each candidate's sum runs over the same key tiles in
 * the same order whichever candidates share the call, so scoring them in one
 * call or in several microbatches gives the same values bit for bit.  k_hist, v_hist: [T_hist][H][d] with
 * token strides ldk, ldv (not read when T_hist = 0); q_c, k_c, v_c, o_c:
 * [total_candidates][H][d] with their own strides.  Workspace:
 * sla_fwd_candidates_workspace_size(p, total_candidates) bytes, 16-byte
 * aligned.  Conventions and errors as sla_fwd. */
size_t sla_fwd_candidates_workspace_size(const sla_problem_t *p, int64_t total_candidates);
sla_status_t sla_fwd_candidates(const sla_problem_t *p, const int64_t *cand_offsets,
                                int64_t total_candidates, const void *k_hist, int64_t ldk,
                                const void *v_hist, int64_t ldv, const void *q_c, int64_t ldq,
                                const void *k_c, int64_t ldkc, const void *v_c, int64_t ldvc,
                                void *o_c, int64_t ldo, void *workspace, size_t ws_bytes,
                                void *stream);

/* One STU layer forward, bf16 storage, fp32 accumulation and statistics
 * (ULTRA-HSTU paper, section 3 Eq.1-5; Code Listing 1 order):
 *   n    = LayerNorm(x) * ln1_w (+ ln1_b)                 row of D = hidden
 *   uvqk = SiLU(n W1^T (+ b_uvqk)), split U | V | Q | K     (each [H][d], head-major)
 *   A    = SLA(Q, K, V)                                   as sla_fwd
 *   y    = (LayerNorm(A) * ln2_w (+ ln2_b)) (.) U           LayerNorm over the H*d_v row
 *   out  = y W2^T (+ b_out) + x                           residual fused in the epilogue
 * x, out: [T][D] bf16 contiguous (out may not alias x); w_uvqk: [2*H*d_v +
 * 2*H*d_qk][D] bf16 (out-features major, as a Linear weight); w_out:
 * [D][H*d_v] bf16; ln*_w, ln*_b, b_*: fp32 vectors (ln*_w and ln*_b
 * 16-byte aligned, as every bf16 buffer); biases nullable.
 * uvqk_out (nullable): [T][2*H*d_v + 2*H*d_qk] bf16 copy of U|V|Q|K; the
 * layer keeps it in the workspace otherwise.  attn_out (nullable): [T][H*d_v]
 * bf16 copy of A, the activation stu_layer_bwd takes instead of recomputing
 * the attention.  attn.dtype must be SLA_BF16, D a multiple of 128 and at
 * most 2048, H*d_v a multiple of 64 and at most 2048. */
typedef struct {
    sla_problem_t attn;
    int32_t hidden;  /* D */
    float ln_eps;    /* LayerNorm epsilon (e.g. 1e-5) */
    int32_t flags;   /* 0, or STU_REUSE_SCHEDULE (forward calls only)        */
} stu_layer_desc_t;

/* flags: the workspace already holds the attention tile schedule of this
 * layout, written by an earlier stu_layer_fwd or stu_layer_fwd_fp8 call on the
 * same stream with the same workspace, offsets, num_targets, total_tokens,
 * num_heads, k1, k2 and contextual_len (a stack's layers between two
 * truncations); the call skips rebuilding it.  stu_layer_bwd requires 0. */
#define STU_REUSE_SCHEDULE 1

size_t stu_layer_workspace_size(const stu_layer_desc_t *d);
sla_status_t stu_layer_fwd(const stu_layer_desc_t *d, const void *x, const float *ln1_w,
                           const float *ln1_b, const void *w_uvqk, const float *b_uvqk,
                           const float *ln2_w, const float *ln2_b, const void *w_out,
                           const float *b_out, void *out, void *uvqk_out, void *attn_out,
                           void *workspace, size_t ws_bytes, void *stream);

/* Gradients of one STU layer (the stu_layer_fwd chain differentiated in
 * reverse; ULTRA-HSTU paper, section 4.2.2 selective rematerialisation: the
 * normalised input and the fused projection are recomputed from x, the
 * attention output A is taken from the forward when given, and y is formed
 * inside the gated LayerNorm backward):
 *   dy = dout W2
 *   gated LayerNorm backward -> dU, dA, dln2_w, dln2_b and y
 *   dW2 = dout^T y, db_out = column sums of dout
 *   sla_bwd(Q, K, V; dA) -> dQ, dK, dV
 *   dz = d[U|V|Q|K] (.) SiLU'(z), z the projection before SiLU
 *   dW1 = dz^T n, db_uvqk = column sums of dz, dn = dz W1
 *   LayerNorm backward -> dx (+ dout, the residual), dln1_w, dln1_b
 * Inputs as stu_layer_fwd (same descriptor, weights and x); attn (nullable):
 * A from stu_layer_fwd's attn_out, recomputed with the attention forward when
 * NULL; dout: [T][D] bf16.  Outputs: dx [T][D] bf16 (required, may not alias
 * an input); the parameter gradients are fp32 of the parameters' shapes
 * (dw_uvqk [2*H*d_v + 2*H*d_qk][D], dw_out [D][H*d_v]) and each is nullable
 * (not computed).  Gradients are written, not accumulated.  Weight gradients
 * are fp32 sums over tokens of bf16 products, split over token ranges and
 * added in a fixed order: results are deterministic.  Limits as the forward,
 * plus H*d_v and 2*H*d_qk multiples of 128 (the weight-gradient tiles).
 * Workspace: stu_layer_bwd_workspace_size(d) bytes, 16-byte aligned. */
size_t stu_layer_bwd_workspace_size(const stu_layer_desc_t *d);
sla_status_t stu_layer_bwd(const stu_layer_desc_t *d, const void *x, const void *attn,
                           const float *ln1_w, const float *ln1_b, const void *w_uvqk,
                           const float *b_uvqk, const float *ln2_w, const float *ln2_b,
                           const void *w_out, const float *b_out, const void *dout, void *dx,
                           float *dln1_w, float *dln1_b, float *dw_uvqk, float *db_uvqk,
                           float *dln2_w, float *dln2_b, float *dw_out, float *db_out,
                           void *workspace, size_t ws_bytes, void *stream);

/* FP8 projections (ULTRA-HSTU paper, section 4.2.2, mixed precision: both
 * STU GEMMs in FP8, everything else bf16; row-wise scaling and quantisation
 * fused into the LayerNorm in front of each GEMM; the post-attention GEMM
 * adds the 2-D residual in its epilogue).  Format FP8 E4M3 (OCP e4m3fn,
 * largest finite 448), one scale per row: row x is stored as
 * q = e4m3(x * 448 / max|x|) (round to nearest even) with scale
 * max|x| / 448, so x ~ q * scale; an all-zero row has q = 0, scale = 1.
 *
 * stu_quantize_rows_fp8: x bf16 [rows][cols] (contiguous; cols a multiple of
 * 16, at most 2048) -> q [rows][cols] e4m3 bytes, scale fp32 [rows].  Used
 * once per weight matrix (rows = output features): w_uvqk [NW][D] and
 * w_out [D][H*d_v] as stu_layer_fwd takes them.
 *
 * stu_layer_fwd_fp8: stu_layer_fwd with the quantised weights (w_*_q e4m3,
 * w_*_scale fp32 per output feature):
 *   n  = LayerNorm(x) quantised row-wise (never stored in bf16)
 *   uvqk = SiLU(sn[t] sw1[o] (nq . w1q[o]) (+ b_uvqk[o]))      bf16
 *   A  = SLA(Q, K, V)                                          bf16
 *   y  = (LayerNorm(A) * ln2_w (+ ln2_b)) (.) U quantised row-wise
 *   out = sy[t] sw2[o] (yq . w2q[o]) (+ b_out[o]) + x          bf16
 * Other arguments, outputs and limits as stu_layer_fwd, plus H*d_v a multiple
 * of 128.  Workspace: stu_layer_fp8_workspace_size(d) bytes. */
sla_status_t stu_quantize_rows_fp8(const void *x, int64_t rows, int32_t cols, void *q,
                                   float *scale, void *stream);
size_t stu_layer_fp8_workspace_size(const stu_layer_desc_t *d);
sla_status_t stu_layer_fwd_fp8(const stu_layer_desc_t *d, const void *x, const float *ln1_w,
                               const float *ln1_b, const void *w_uvqk_q,
                               const float *w_uvqk_scale, const float *b_uvqk,
                               const float *ln2_w, const float *ln2_b, const void *w_out_q,
                               const float *w_out_scale, const float *b_out, void *out,
                               void *uvqk_out, void *attn_out, void *workspace, size_t ws_bytes,
                               void *stream);

/* Target (candidate) rows of a jagged batch gathered into a column block of a
 * dense output (Mixture of Transducers, ULTRA-HSTU paper section 4.3 and
 * Appendix A, and the torcheasyrec page's MoT bullet: every channel runs its own STU stack over
 * its own UIH sequence with the shared contextual and candidate tokens, and
 * the channels' candidate embeddings are concatenated along the feature
 * dimension).  Writes target_offsets [B+1] (int64, device: sequence b's
 * targets are rows target_offsets[b] .. target_offsets[b+1] of out) and, when
 * out is non-NULL, copies the last num_targets[b] rows of each sequence of
 * x [total_tokens][hidden] into out rows in order, columns [col_offset,
 * col_offset + hidden) of rows of ld_out elements.  dtype as x (bf16 or
 * f32); hidden, ld_out and col_offset multiples of 16 bytes; capacity >= the
 * total number of targets (rows past capacity are not written). */
sla_status_t stu_gather_targets(int32_t batch, int64_t total_tokens, const int64_t *offsets,
                                const int32_t *num_targets, const void *x, int32_t hidden,
                                int32_t dtype, int64_t *target_offsets, void *out, int64_t ld_out,
                                int64_t col_offset, int64_t capacity, void *stream);

/* Attention truncation (ULTRA-HSTU paper, section 4.3; torcheasyrec page,
 * truncation bullet): per sequence keep, in order, the contextual prefix
 * [0, c), the most recent tail_len history tokens and the num_targets[b]
 * targets, where U = L_b - num_targets[b], c = min(contextual_len, U), and
 * the history is [c, U).  Writes new_offsets [B+1] (int64),
 * new_num_targets [B] (int32, = num_targets, nullable), gather_idx
 * [capacity] (int64 source token of each kept row, nullable) and x_out
 * [capacity][hidden] (nullable; dtype element size 2 for bf16, 4 for f32).
 * capacity >= min(total_tokens, B * (contextual_len + tail_len) + sum of
 * targets) must hold; pass total_tokens when in doubt.  tail_len >= 1. */
sla_status_t stu_truncate(int32_t batch, int64_t total_tokens, const int64_t *offsets,
                          const int32_t *num_targets, int32_t contextual_len,
                          int32_t tail_len, const void *x, int32_t hidden, int32_t dtype,
                          int64_t *new_offsets, int32_t *new_num_targets, int64_t *gather_idx,
                          void *x_out, int64_t capacity, void *stream);

/* Backward of stu_truncate, its adjoint (ULTRA-HSTU paper, section 4.3: the
 * layers after the truncation see only the kept rows): given dy, the gradient
 * of the truncated rows [new_offsets[B]][hidden], writes dx [total_tokens]
 * [hidden] with dx[s] = dy[r] for every source token s that the truncation
 * kept as row r and dx[s] = 0 for every token it dropped.  offsets,
 * num_targets, contextual_len and tail_len are those of the stu_truncate call,
 * new_offsets its output.  Every row of dx is written once: no atomics, no
 * host synchronisation.  dtype SLA_BF16 or SLA_F32 for dy and dx; hidden rows
 * a multiple of 16 bytes; dy and dx 16-byte aligned.  B = 0 or T = 0: no-op.
 * Errors as stu_truncate. */
sla_status_t stu_truncate_bwd(int32_t batch, int64_t total_tokens, const int64_t *offsets,
                              const int32_t *num_targets, int32_t contextual_len,
                              int32_t tail_len, const int64_t *new_offsets, const void *dy,
                              int32_t hidden, int32_t dtype, void *dx, void *stream);

/* Measurement aid, not part of the attention path: the bf16 dense MFMA rate
 * the current device sustains, measured with an MFMA-only kernel (four
 * workgroups of four waves per CU, each wave `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 chains; one warm-up launch, then one
 * launch timed with HIP events on `stream`, which is synchronised).  Writes
 * the rate in TFLOP/s to *tflops and the shader clock observed during the
 * timed launch (shader-clock counter over the 100 MHz constant clock) in GHz
 * to *sclk_ghz.  scratch: caller-owned device memory of at least
 * sla_probe_scratch_size() bytes (16-byte aligned; about 1 MB on a 256-CU
 * device), overwritten; a smaller one -> SLA_ERR_WORKSPACE.  Allocates
 * nothing.  1 <= iters <= 1048576 (4096: about 1 ms).
 * sla_probe_scratch_size returns 0 when no device is current. */
size_t sla_probe_scratch_size(void);
sla_status_t sla_probe_mfma_peak(int32_t iters, void *scratch, size_t scratch_bytes, double *tflops,
                                 double *sclk_ghz, void *stream);

/* Measurement aid, not part of the attention path: how far one SIMD of the
 * current device runs MFMA and VALU instructions concurrently, and the rate
 * of the SiLU's transcendentals.  One workgroup of eight waves per CU (two
 * per SIMD); per SIMD every MFMA arrangement issues 2 * iters * 4
 * v_mfma_f32_32x32x16_bf16 (four independent chains) and every VALU one
 * 2 * iters * 32 v_fma_f32 (eight independent chains).  ms[0..6] receive the
 * duration of one launch (after a warm-up, HIP events on `stream`, which is
 * synchronised) of: 0 MFMA only, 1 FMA only, 2 one wave per SIMD with all the
 * MFMAs and the other with all the FMAs, 3 both waves half of each,
 * interleaved, 4 as 2 with the accumulators in AGPRs, 5 v_exp_f32 only and
 * 6 v_rcp_f32 only (32 per round, in place of the FMAs of 1).  n_ms >= 7.
 * scratch: caller-owned device memory of at least sla_probe_scratch_size()
 * bytes (16-byte aligned), overwritten; a smaller one -> SLA_ERR_WORKSPACE.
 * Allocates nothing.  1 <= iters <= 1048576 (4096: about 0.5 ms per mode). */
sla_status_t sla_probe_issue_rates(int32_t iters, void *scratch, size_t scratch_bytes, double *ms,
                                   int32_t n_ms, void *stream);

const char *sla_status_string(sla_status_t s);
const char *sla_last_error(void); /* thread-local message of the last failure */

#ifdef __cplusplus
}
#endif
#endif /* SLA_MI355X_H */
