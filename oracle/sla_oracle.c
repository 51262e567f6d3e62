/*
 * sla_oracle.c -- plain fp64 CPU oracle for Semi-Local Attention (SLA) and the
 * STU layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code, header,
 * table or helper with the HIP library; the two meet only through the seeded
 * arrays that the synthetic-input package produces.
 *
 * Everything here is the definition written out, loop by loop, in double
 * precision, in the order the pages state it:
 *
 *  - visibility: ULTRA-HSTU paper, section 4.2.1, Eq.7 (semi-local mask: a
 *    local window of K1 keys plus a global prefix of K2 keys, intersected with
 *    causality, Eq.6), read 0-based as  j <= i && (i - j < K1 || j < K2e);
 *    torcheasyrec "ULTRA HSTU" page, SLA bullet: K2e = max(sla_k2,
 *    contextual_seq_len).  Target rows: HSTU notes page, Q8 (M-FALCON mask
 *    diagram): a candidate sees the history and itself, never another
 *    candidate; the history part is the view of the first target slot.
 *  - attention: ULTRA-HSTU paper, section 3, Eq.3 / section 4.2.1, Eq.6:
 *    A = (SiLU(Q K^T) (.) M) V, pointwise SiLU and no softmax (HSTU notes,
 *    section 2.4, Eq.2), scaled by 1/N and with a pre-activation factor alpha.
 *  - backward: the chain rule of that forward, written per visible pair.
 *  - STU layer: ULTRA-HSTU paper, section 3, Eq.1-5, in the operation order
 *    of the paper's Code Listing 1 (norm -> fused projection + SiLU split
 *    U,V,Q,K -> attention -> gated norm -> projection with the input as
 *    residual).
 *  - truncation: ULTRA-HSTU paper, section 4.3 ("attention truncation") and
 *    the torcheasyrec page's truncation bullet: keep the contextual prefix,
 *    the most recent tail_len history tokens and all targets.
 *
 * Precision: inputs arrive as fp64 copies of the exact values the GPU gets;
 * all arithmetic is fp64.  The STU layer has an optional "storage-matched"
 * mode that rounds the tensors the GPU keeps in bfloat16 (round to nearest
 * even) at the same points.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* visibility                                                                */
/* ------------------------------------------------------------------------ */

/* Row i (0-based, within one sequence) may attend key j.
 * U = first target index (= L when there are no targets), K2e = effective
 * global prefix.  History rows: causal and (local window or global prefix).
 * Target rows: self, or a history key inside the view of row U restricted to
 * history keys. */
static int visible(int64_t i, int64_t j, int64_t U, int64_t K1, int64_t K2e)
{
    if (i < U)
        return (j <= i) && ((i - j < K1) || (j < K2e));
    if (j == i)
        return 1;
    return (j < U) && ((U - j < K1) || (j < K2e));
}

static int64_t k2_effective(int64_t k2, int64_t ctx) { return k2 > ctx ? k2 : ctx; }

EXPORT int oracle_visible(int64_t i, int64_t j, int64_t L, int64_t num_targets,
                          int64_t k1, int64_t k2, int64_t ctx)
{
    if (i < 0 || j < 0 || i >= L || j >= L) return 0;
    return visible(i, j, L - num_targets, k1, k2_effective(k2, ctx));
}

/* Dense L x L 0/1 mask of one sequence, row-major. */
EXPORT void oracle_mask_dense(int64_t L, int64_t num_targets, int64_t k1, int64_t k2,
                              int64_t ctx, uint8_t *out)
{
    int64_t U = L - num_targets, K2e = k2_effective(k2, ctx);
    for (int64_t i = 0; i < L; ++i)
        for (int64_t j = 0; j < L; ++j)
            out[i * L + j] = (uint8_t)visible(i, j, U, k1, K2e);
}

static int64_t seq_targets(const int32_t *num_targets, int b)
{
    return num_targets ? (int64_t)num_targets[b] : 0;
}

/* Number of visible (row, key) pairs per head, summed over the batch,
 * counted by visiting every (i, j). */
EXPORT int64_t oracle_count_pairs(int B, const int64_t *offsets, const int32_t *num_targets,
                                  int64_t k1, int64_t k2, int64_t ctx)
{
    int64_t K2e = k2_effective(k2, ctx), total = 0;
    for (int b = 0; b < B; ++b) {
        int64_t L = offsets[b + 1] - offsets[b];
        int64_t U = L - seq_targets(num_targets, b);
        int64_t cnt = 0;
#pragma omp parallel for reduction(+ : cnt) schedule(dynamic, 64)
        for (int64_t i = 0; i < L; ++i)
            for (int64_t j = 0; j < L; ++j)
                cnt += visible(i, j, U, k1, K2e);
        total += cnt;
    }
    return total;
}

/* Enumerate the non-empty (row-tile, key-tile) pairs.
 * Row tiles: the history [0, U) cut into BM-row tiles starting at row 0, then
 * the targets [U, L) cut into BM-row tiles starting at row U, so that no tile
 * mixes history and target rows.  Key tiles: [0, L) cut into BN-key tiles
 * starting at key 0.  A pair is non-empty when at least one of its (i, j) is
 * visible.  Output triples (b, row_tile_start, key_tile_start) in the order
 * b, row tile, key tile.  Returns the number of pairs (writes at most cap). */
EXPORT int64_t oracle_tiles(int B, const int64_t *offsets, const int32_t *num_targets,
                            int64_t k1, int64_t k2, int64_t ctx, int64_t BM, int64_t BN,
                            int64_t *out, int64_t cap)
{
    int64_t K2e = k2_effective(k2, ctx), n = 0;
    for (int b = 0; b < B; ++b) {
        int64_t L = offsets[b + 1] - offsets[b];
        int64_t U = L - seq_targets(num_targets, b);
        for (int part = 0; part < 2; ++part) {
            int64_t r_begin = part == 0 ? 0 : U, r_end = part == 0 ? U : L;
            for (int64_t r0 = r_begin; r0 < r_end; r0 += BM) {
                int64_t r1 = r0 + BM < r_end ? r0 + BM : r_end;
                for (int64_t c0 = 0; c0 < L; c0 += BN) {
                    int64_t c1 = c0 + BN < L ? c0 + BN : L;
                    int any = 0;
                    for (int64_t i = r0; i < r1 && !any; ++i)
                        for (int64_t j = c0; j < c1 && !any; ++j)
                            any = visible(i, j, U, k1, K2e);
                    if (any) {
                        if (n < cap) {
                            out[3 * n + 0] = b;
                            out[3 * n + 1] = r0;
                            out[3 * n + 2] = c0;
                        }
                        ++n;
                    }
                }
            }
        }
    }
    return n;
}

/* ------------------------------------------------------------------------ */
/* attention                                                                 */
/* ------------------------------------------------------------------------ */

static double silu(double t) { return t / (1.0 + exp(-t)); }
static double sigmoid(double t) { return 1.0 / (1.0 + exp(-t)); }

/* Tensors are dense [T][H][d] in fp64. */
static double dot(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += a[c] * b[c];
    return s;
}

/* O[i] = (1/N) * sum_{j visible} SiLU(alpha * q_i . k_j) * v_j
 * row_sel (nullable, [T]): compute only rows with row_sel != 0 (others left
 * untouched). */
EXPORT void oracle_sla_fwd(int B, const int64_t *offsets, const int32_t *num_targets, int H,
                           int dqk, int dv, int64_t k1, int64_t k2, int64_t ctx, double N,
                           double alpha, const double *q, const double *k, const double *v,
                           double *o, const uint8_t *row_sel)
{
    int64_t K2e = k2_effective(k2, ctx);
    for (int b = 0; b < B; ++b) {
        int64_t base = offsets[b], L = offsets[b + 1] - offsets[b];
        int64_t U = L - seq_targets(num_targets, b);
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
        for (int64_t i = 0; i < L; ++i) {
            for (int h = 0; h < H; ++h) {
                int64_t ti = base + i;
                if (row_sel && !row_sel[ti]) continue;
                double acc[512];
                for (int c = 0; c < dv; ++c) acc[c] = 0.0;
                const double *qi = q + (ti * H + h) * dqk;
                for (int64_t j = 0; j <= i; ++j) { /* no visible key lies after row i */
                    if (!visible(i, j, U, k1, K2e)) continue;
                    int64_t tj = base + j;
                    double a = silu(alpha * dot(qi, k + (tj * H + h) * dqk, dqk));
                    const double *vj = v + (tj * H + h) * dv;
                    for (int c = 0; c < dv; ++c) acc[c] += a * vj[c];
                }
                double *oi = o + (ti * H + h) * dv;
                for (int c = 0; c < dv; ++c) oi[c] = acc[c] / N;
            }
        }
    }
}

/* Candidate scoring against a cached history (M-FALCON; HSTU notes, section
 * 2.6, and the target-aware mask of the ULTRA-HSTU setting): sequence b has a
 * history of U_b = hist_offsets[b+1] - hist_offsets[b] tokens whose keys and
 * values (k_hist, v_hist, [T_hist][H][d]) are computed once, and candidates
 * cand_offsets[b] .. cand_offsets[b+1] with their own q, k, v ([C][H][d]).
 * Candidate c scores against the history keys that the first candidate
 * position U_b sees (j < U_b with U_b - j < K1 or j < K2e) and against
 * itself; candidates never see each other:
 *   o_c = (1/N) ( sum_j SiLU(alpha q_c . k_j) v_j + SiLU(alpha q_c . k_c) v_c ). */
EXPORT void oracle_sla_fwd_candidates(int B, const int64_t *hist_offsets,
                                      const int64_t *cand_offsets, int H, int dqk, int dv,
                                      int64_t k1, int64_t k2, int64_t ctx, double N, double alpha,
                                      const double *k_hist, const double *v_hist,
                                      const double *qc, const double *kc, const double *vc,
                                      double *oc)
{
    int64_t K2e = k2_effective(k2, ctx);
    for (int b = 0; b < B; ++b) {
        const int64_t hb = hist_offsets[b], U = hist_offsets[b + 1] - hist_offsets[b];
        const int64_t cb = cand_offsets[b], nc = cand_offsets[b + 1] - cand_offsets[b];
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
        for (int64_t c = 0; c < nc; ++c) {
            for (int h = 0; h < H; ++h) {
                const int64_t tc = cb + c;
                double acc[512];
                for (int e = 0; e < dv; ++e) acc[e] = 0.0;
                const double *q = qc + (tc * H + h) * dqk;
                for (int64_t j = 0; j < U; ++j) {
                    if (!(U - j < k1 || j < K2e)) continue;
                    const int64_t tj = hb + j;
                    const double a = silu(alpha * dot(q, k_hist + (tj * H + h) * dqk, dqk));
                    const double *vj = v_hist + (tj * H + h) * dv;
                    for (int e = 0; e < dv; ++e) acc[e] += a * vj[e];
                }
                const double a = silu(alpha * dot(q, kc + (tc * H + h) * dqk, dqk));
                const double *vs = vc + (tc * H + h) * dv;
                for (int e = 0; e < dv; ++e) acc[e] += a * vs[e];
                double *o = oc + (tc * H + h) * dv;
                for (int e = 0; e < dv; ++e) o[e] = acc[e] / N;
            }
        }
    }
}

/* Gradients of O = (1/N) sum_j SiLU(alpha q_i.k_j) v_j given dO:
 *   a_ij  = SiLU(alpha s_ij),   s_ij = q_i . k_j
 *   dV_j  = (1/N) sum_i a_ij dO_i
 *   g_ij  = dO_i . v_j
 *   dS_ij = (1/N) g_ij * alpha * SiLU'(alpha s_ij),
 *           SiLU'(t) = sigma(t) * (1 + t * (1 - sigma(t)))
 *   dQ_i  = sum_j dS_ij k_j,    dK_j = sum_i dS_ij q_i
 * dQ rows are gathered over keys, dK/dV rows over the rows that see the key.
 * q_sel / k_sel (nullable, [T]) restrict which dQ rows / dK,dV rows are
 * computed. */
EXPORT void oracle_sla_bwd(int B, const int64_t *offsets, const int32_t *num_targets, int H,
                           int dqk, int dv, int64_t k1, int64_t k2, int64_t ctx, double N,
                           double alpha, const double *q, const double *k, const double *v,
                           const double *dout, double *dq, double *dk, double *dvv,
                           const uint8_t *q_sel, const uint8_t *k_sel)
{
    int64_t K2e = k2_effective(k2, ctx);
    for (int b = 0; b < B; ++b) {
        int64_t base = offsets[b], L = offsets[b + 1] - offsets[b];
        int64_t U = L - seq_targets(num_targets, b);
        /* dQ: one row at a time, over the keys it sees */
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
        for (int64_t i = 0; i < L; ++i) {
            for (int h = 0; h < H; ++h) {
                int64_t ti = base + i;
                if (q_sel && !q_sel[ti]) continue;
                double acc[512];
                for (int c = 0; c < dqk; ++c) acc[c] = 0.0;
                const double *qi = q + (ti * H + h) * dqk;
                const double *gi = dout + (ti * H + h) * dv;
                for (int64_t j = 0; j <= i; ++j) { /* no visible key lies after row i */
                    if (!visible(i, j, U, k1, K2e)) continue;
                    int64_t tj = base + j;
                    const double *kj = k + (tj * H + h) * dqk;
                    double t = alpha * dot(qi, kj, dqk);
                    double sg = sigmoid(t);
                    double ds = dot(gi, v + (tj * H + h) * dv, dv) / N * alpha *
                                (sg * (1.0 + t * (1.0 - sg)));
                    for (int c = 0; c < dqk; ++c) acc[c] += ds * kj[c];
                }
                double *o = dq + (ti * H + h) * dqk;
                for (int c = 0; c < dqk; ++c) o[c] = acc[c];
            }
        }
        /* dK, dV: one key at a time, over the rows that see it */
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
        for (int64_t j = 0; j < L; ++j) {
            for (int h = 0; h < H; ++h) {
                int64_t tj = base + j;
                if (k_sel && !k_sel[tj]) continue;
                double acck[512], accv[512];
                for (int c = 0; c < dqk; ++c) acck[c] = 0.0;
                for (int c = 0; c < dv; ++c) accv[c] = 0.0;
                const double *kj = k + (tj * H + h) * dqk;
                const double *vj = v + (tj * H + h) * dv;
                for (int64_t i = j; i < L; ++i) { /* no row before j sees j */
                    if (!visible(i, j, U, k1, K2e)) continue;
                    int64_t ti = base + i;
                    const double *qi = q + (ti * H + h) * dqk;
                    const double *gi = dout + (ti * H + h) * dv;
                    double t = alpha * dot(qi, kj, dqk);
                    double sg = sigmoid(t);
                    double a = t * sg;
                    for (int c = 0; c < dv; ++c) accv[c] += a / N * gi[c];
                    double ds = dot(gi, vj, dv) / N * alpha * (sg * (1.0 + t * (1.0 - sg)));
                    for (int c = 0; c < dqk; ++c) acck[c] += ds * qi[c];
                }
                double *ok = dk + (tj * H + h) * dqk;
                double *ov = dvv + (tj * H + h) * dv;
                for (int c = 0; c < dqk; ++c) ok[c] = acck[c];
                for (int c = 0; c < dv; ++c) ov[c] = accv[c];
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* bfloat16 rounding (storage-matched mode)                                  */
/* ------------------------------------------------------------------------ */

/* Round x to the nearest bfloat16 value (8 significant bits), ties to even. */
EXPORT double oracle_round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(x, &e);                 /* x = m * 2^e, 0.5 <= |m| < 1 */
    int qexp = e - 8;             /* spacing of bf16 numbers around x */
    if (qexp < -133) qexp = -133; /* subnormal spacing 2^-133 */
    double r = nearbyint(ldexp(x, -qexp));
    double y = ldexp(r, qexp);
    if (fabs(y) >= ldexp(1.0, 128)) y = x > 0 ? INFINITY : -INFINITY;
    return y;
}

static void round_all(double *a, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) a[i] = oracle_round_bf16(a[i]);
}

/* Round x to the nearest FP8 E4M3 value (OCP "e4m3fn": 3 mantissa bits,
 * exponent bias 7, largest finite 448, subnormal spacing 2^-9), ties to even;
 * magnitudes past 448 saturate to +-448. */
EXPORT double oracle_round_e4m3(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(x, &e);          /* |x| in [2^(e-1), 2^e) */
    int qexp = e - 4;      /* 3 bits below the leading one */
    if (qexp < -9) qexp = -9;
    double y = ldexp(nearbyint(ldexp(x, -qexp)), qexp);
    if (y > 448.0) y = 448.0;
    if (y < -448.0) y = -448.0;
    return y;
}

/* Row-wise FP8 quantisation (ULTRA-HSTU paper, section 4.2.2, mixed
 * precision: a scale per row, computed and applied where the row is
 * produced): with a = max |x[r][:]|, the row is stored as
 * q = e4m3(x * (448 / a)) and the scale s = a / 448, so x ~ q * s.  An
 * all-zero row has s = 1 and q = 0.  q holds the e4m3 values (as doubles).
 *
 * The code q is an integer that floating point decides, and the paper fixes
 * no precision for that arithmetic, so it is a parameter:
 *   fp32_decision = 1: x taken as an fp32 value, and 448 / a, the product and
 *     a / 448 each one correctly rounded fp32 operation (the precision the
 *     kernels compute in; the mode every comparison with them uses);
 *   fp32_decision = 0: the quotient, the product and the scale in fp64, so
 *     each code is the nearest e4m3 value of the (nearly) exact x / s.
 * The two differ by one e4m3 step, and only where x / s lies within fp32
 * rounding of a point halfway between two e4m3 values. */
EXPORT void oracle_quant_rows_fp8(int64_t rows, int64_t cols, const double *x, double *q,
                                  double *scale, int fp32_decision)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double *qr = q + r * cols;
        if (fp32_decision) {
            float a = 0.0f;
            for (int64_t c = 0; c < cols; ++c) a = fmaxf(a, fabsf((float)xr[c]));
            if (a == 0.0f) {
                scale[r] = 1.0;
                for (int64_t c = 0; c < cols; ++c) qr[c] = 0.0;
                continue;
            }
            const float inv = 448.0f / a;
            scale[r] = (double)(a / 448.0f);
            for (int64_t c = 0; c < cols; ++c) {
                const float prod = (float)xr[c] * inv;
                qr[c] = oracle_round_e4m3((double)prod);
            }
        } else {
            double a = 0.0;
            for (int64_t c = 0; c < cols; ++c) a = fmax(a, fabs(xr[c]));
            if (a == 0.0) {
                scale[r] = 1.0;
                for (int64_t c = 0; c < cols; ++c) qr[c] = 0.0;
                continue;
            }
            const double inv = 448.0 / a;
            scale[r] = a / 448.0;
            for (int64_t c = 0; c < cols; ++c) qr[c] = oracle_round_e4m3(xr[c] * inv);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* LayerNorm and the STU layer                                               */
/* ------------------------------------------------------------------------ */

/* y = (x - mean) / sqrt(var + eps) * w (+ b), biased variance, per row. */
EXPORT void oracle_layernorm(int64_t rows, int64_t cols, const double *x, const double *w,
                             const double *b, double eps, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double mean = 0.0;
        for (int64_t c = 0; c < cols; ++c) mean += xr[c];
        mean /= (double)cols;
        double var = 0.0;
        for (int64_t c = 0; c < cols; ++c) var += (xr[c] - mean) * (xr[c] - mean);
        var /= (double)cols;
        double inv = 1.0 / sqrt(var + eps);
        for (int64_t c = 0; c < cols; ++c)
            y[r * cols + c] = (xr[c] - mean) * inv * w[c] + (b ? b[c] : 0.0);
    }
}

/* y[r][n] = sum_c x[r][c] * W[n][c] (+ bias[n]); W is [nout][nin]. */
static void linear(int64_t rows, int64_t nin, int64_t nout, const double *x, const double *W,
                   const double *bias, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t n = 0; n < nout; ++n) {
            double s = bias ? bias[n] : 0.0;
            const double *xr = x + r * nin, *wn = W + n * nin;
            for (int64_t c = 0; c < nin; ++c) s += xr[c] * wn[c];
            y[r * nout + n] = s;
        }
}

/* One STU layer (ULTRA-HSTU paper, section 3, Eq.1-5; Code Listing 1 order):
 *   n    = LN(x; ln1_w, ln1_b)
 *   z    = n W1^T (+ b1);  [U | V | Q | K] = SiLU(z), each block [H][d]
 *   A    = SLA(Q, K, V)
 *   y    = LN(A; ln2_w, ln2_b) (.) U          (LN over the whole H*dv row)
 *   out  = y W2^T (+ b2) + x
 * x, out: [T][D]; W1: [2*H*dv + 2*H*dqk][D]; W2: [D][H*dv].
 * store_bf16 is a bit mask of storage points rounded to bfloat16:
 *   1 = the branch tensors n, U/V/Q/K, A, y;   2 = the layer output (residual
 *   stream).  3 rounds all five points.
 * uvqk_out (nullable): [T][2*H*dv + 2*H*dqk] after SiLU (and rounding). */
EXPORT void oracle_stu_layer_fwd(int B, const int64_t *offsets, const int32_t *num_targets,
                                 int D, int H, int dqk, int dv, int64_t k1, int64_t k2,
                                 int64_t ctx, double N, double alpha, double eps,
                                 const double *x, const double *ln1_w, const double *ln1_b,
                                 const double *w1, const double *b1, const double *ln2_w,
                                 const double *ln2_b, const double *w2, const double *b2,
                                 int store_bf16, double *out, double *uvqk_out)
{
    int64_t T = offsets[B];
    int64_t NU = (int64_t)H * dv, NQ = (int64_t)H * dqk, NW = 2 * NU + 2 * NQ;
    double *n = malloc(sizeof(double) * T * D);
    double *z = malloc(sizeof(double) * T * NW);
    double *qq = malloc(sizeof(double) * T * NQ), *kk = malloc(sizeof(double) * T * NQ);
    double *vv = malloc(sizeof(double) * T * NU), *uu = malloc(sizeof(double) * T * NU);
    double *a = malloc(sizeof(double) * T * NU), *y = malloc(sizeof(double) * T * NU);

    const int rb = store_bf16 & 1, ro = store_bf16 & 2;
    oracle_layernorm(T, D, x, ln1_w, ln1_b, eps, n);
    if (rb) round_all(n, T * D);
    linear(T, D, NW, n, w1, b1, z);
    for (int64_t i = 0; i < T * NW; ++i) z[i] = silu(z[i]);
    if (rb) round_all(z, T * NW);
    if (uvqk_out) memcpy(uvqk_out, z, sizeof(double) * T * NW);
    for (int64_t t = 0; t < T; ++t) {
        const double *zr = z + t * NW;
        memcpy(uu + t * NU, zr, sizeof(double) * NU);
        memcpy(vv + t * NU, zr + NU, sizeof(double) * NU);
        memcpy(qq + t * NQ, zr + 2 * NU, sizeof(double) * NQ);
        memcpy(kk + t * NQ, zr + 2 * NU + NQ, sizeof(double) * NQ);
    }
    oracle_sla_fwd(B, offsets, num_targets, H, dqk, dv, k1, k2, ctx, N, alpha, qq, kk, vv, a,
                   NULL);
    if (rb) round_all(a, T * NU);
    oracle_layernorm(T, NU, a, ln2_w, ln2_b, eps, y);
    for (int64_t i = 0; i < T * NU; ++i) y[i] *= uu[i];
    if (rb) round_all(y, T * NU);
    linear(T, NU, D, y, w2, b2, out);
    for (int64_t i = 0; i < T * D; ++i) out[i] += x[i];
    if (ro) round_all(out, T * D);

    free(n); free(z); free(qq); free(kk); free(vv); free(uu); free(a); free(y);
}

/* One STU layer forward with both projections in FP8 (ULTRA-HSTU paper,
 * section 4.2.2, mixed precision; everything else as oracle_stu_layer_fwd in
 * its bf16-storage mode): the normalised input n and the gated output y are
 * quantised row-wise where they are produced, the weights row-wise (one scale
 * per output feature), and each projection is the exact product of the
 * quantised operands times the two scales:
 *   z[t][o]   = sn[t] sw1[o] sum_c nq[t][c] w1q[o][c] + b1[o]
 *   out[t][o] = sy[t] sw2[o] sum_c yq[t][c] w2q[o][c] + b2[o] + x[t][o]
 * U/V/Q/K, A and out are rounded to bf16 (stored tensors); n and y are not
 * (they go straight into the quantiser).  Codes are decided in fp32 (the
 * kernels' precision; the paper fixes none). */
EXPORT void oracle_stu_layer_fwd_fp8(int B, const int64_t *offsets, const int32_t *num_targets,
                                     int D, int H, int dqk, int dv, int64_t k1, int64_t k2,
                                     int64_t ctx, double N, double alpha, double eps,
                                     const double *x, const double *ln1_w, const double *ln1_b,
                                     const double *w1, const double *b1, const double *ln2_w,
                                     const double *ln2_b, const double *w2, const double *b2,
                                     double *out, double *uvqk_out)
{
    const int64_t T = offsets[B];
    const int64_t NU = (int64_t)H * dv, NQ = (int64_t)H * dqk, NW = 2 * NU + 2 * NQ;
    double *n = malloc(sizeof(double) * T * D), *nq = malloc(sizeof(double) * T * D);
    double *sn = malloc(sizeof(double) * T), *sy = malloc(sizeof(double) * T);
    double *w1q = malloc(sizeof(double) * NW * D), *sw1 = malloc(sizeof(double) * NW);
    double *w2q = malloc(sizeof(double) * D * NU), *sw2 = malloc(sizeof(double) * D);
    double *z = malloc(sizeof(double) * T * NW);
    double *qq = malloc(sizeof(double) * T * NQ), *kk = malloc(sizeof(double) * T * NQ);
    double *vv = malloc(sizeof(double) * T * NU), *uu = malloc(sizeof(double) * T * NU);
    double *a = malloc(sizeof(double) * T * NU), *y = malloc(sizeof(double) * T * NU);
    double *yq = malloc(sizeof(double) * T * NU);

    oracle_quant_rows_fp8(NW, D, w1, w1q, sw1, 1);
    oracle_quant_rows_fp8(D, NU, w2, w2q, sw2, 1);
    oracle_layernorm(T, D, x, ln1_w, ln1_b, eps, n);
    oracle_quant_rows_fp8(T, D, n, nq, sn, 1);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t o = 0; o < NW; ++o) {
            double acc = 0.0;
            for (int64_t c = 0; c < D; ++c) acc += nq[t * D + c] * w1q[o * D + c];
            const double zz = sn[t] * sw1[o] * acc + (b1 ? b1[o] : 0.0);
            z[t * NW + o] = oracle_round_bf16(silu(zz));
        }
    if (uvqk_out) memcpy(uvqk_out, z, sizeof(double) * T * NW);
    for (int64_t t = 0; t < T; ++t) {
        const double *zr = z + t * NW;
        memcpy(uu + t * NU, zr, sizeof(double) * NU);
        memcpy(vv + t * NU, zr + NU, sizeof(double) * NU);
        memcpy(qq + t * NQ, zr + 2 * NU, sizeof(double) * NQ);
        memcpy(kk + t * NQ, zr + 2 * NU + NQ, sizeof(double) * NQ);
    }
    oracle_sla_fwd(B, offsets, num_targets, H, dqk, dv, k1, k2, ctx, N, alpha, qq, kk, vv, a,
                   NULL);
    round_all(a, T * NU);
    oracle_layernorm(T, NU, a, ln2_w, ln2_b, eps, y);
    for (int64_t i = 0; i < T * NU; ++i) y[i] *= uu[i];
    oracle_quant_rows_fp8(T, NU, y, yq, sy, 1);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t o = 0; o < D; ++o) {
            double acc = 0.0;
            for (int64_t c = 0; c < NU; ++c) acc += yq[t * NU + c] * w2q[o * NU + c];
            out[t * D + o] =
                oracle_round_bf16(sy[t] * sw2[o] * acc + (b2 ? b2[o] : 0.0) + x[t * D + o]);
        }
    free(n); free(nq); free(sn); free(sy); free(w1q); free(sw1); free(w2q); free(sw2); free(z);
    free(qq); free(kk); free(vv); free(uu); free(a); free(y); free(yq);
}

/* Row statistics of LayerNorm: xh = (x - mean) * rstd, rstd = 1/sqrt(var + eps)
 * (biased variance), as in oracle_layernorm. */
static void ln_stats(int64_t rows, int64_t cols, const double *x, double eps, double *xh,
                     double *rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double mean = 0.0;
        for (int64_t c = 0; c < cols; ++c) mean += xr[c];
        mean /= (double)cols;
        double var = 0.0;
        for (int64_t c = 0; c < cols; ++c) var += (xr[c] - mean) * (xr[c] - mean);
        var /= (double)cols;
        rstd[r] = 1.0 / sqrt(var + eps);
        for (int64_t c = 0; c < cols; ++c) xh[r * cols + c] = (xr[c] - mean) * rstd[r];
    }
}

/* Backward of y = xh * w + b with xh the row-normalised x: given dy, adds the
 * column sums dw += sum_r dy * xh and db += sum_r dy (if non-NULL) and writes
 * dx = rstd * (g - mean(g) - xh * mean(g * xh)) with g = dy * w, per row. */
static void ln_backward(int64_t rows, int64_t cols, const double *dy, const double *xh,
                        const double *rstd, const double *w, double *dx, double *dw, double *db)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            dw[c] += dy[r * cols + c] * xh[r * cols + c];
            if (db) db[c] += dy[r * cols + c];
        }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double m1 = 0.0, m2 = 0.0;
        for (int64_t c = 0; c < cols; ++c) {
            const double g = dy[r * cols + c] * w[c];
            m1 += g;
            m2 += g * xh[r * cols + c];
        }
        m1 /= (double)cols;
        m2 /= (double)cols;
        for (int64_t c = 0; c < cols; ++c) {
            const double g = dy[r * cols + c] * w[c];
            dx[r * cols + c] = rstd[r] * (g - m1 - xh[r * cols + c] * m2);
        }
    }
}

/* SiLU'(z) = sigma(z) (1 + z (1 - sigma(z))). */
static double dsilu(double z)
{
    const double s = 1.0 / (1.0 + exp(-z));
    return s * (1.0 + z * (1.0 - s));
}

/* Gradients of one STU layer (the forward of oracle_stu_layer_fwd) given
 * dout = dL/dout: recomputes the forward in fp64, then applies the chain rule
 * step by step backwards through
 *   out = y W2^T + b2 + x,  y = (ah * g2 + b2n) (.) U,  ah = LN-normalised A,
 *   A = SLA(Q, K, V),  [U V Q K] = SiLU(z),  z = n W1^T + b1,
 *   n = xh * g1 + b1n,  xh = LN-normalised x.
 * Outputs (all overwritten; biases' gradients only where the pointer is
 * non-NULL): dx [T][D], dln1_w/b [D], dw1 [NW][D], db1 [NW], dln2_w/b [NU],
 * dw2 [D][NU], db2 [D].
 * store_bf16 != 0 rounds to bfloat16 every tensor a bf16 implementation
 * stores between steps: the recomputed n, z (the stored pre-activation that
 * SiLU' is evaluated at), U/V/Q/K = SiLU(z) (taken of the unrounded z), A and
 * y; the gradients dy, dU, dA, dQ, dK, dV, dz, dn and the output dx.  The
 * parameter gradients are sums of products of those stored values. */
EXPORT void oracle_stu_layer_bwd(int B, const int64_t *offsets, const int32_t *num_targets,
                                 int D, int H, int dqk, int dv, int64_t k1, int64_t k2,
                                 int64_t ctx, double N, double alpha, double eps,
                                 const double *x, const double *ln1_w, const double *ln1_b,
                                 const double *w1, const double *b1, const double *ln2_w,
                                 const double *ln2_b, const double *w2, const double *b2,
                                 const double *dout, int store_bf16, double *dx, double *dln1_w,
                                 double *dln1_b, double *dw1, double *db1, double *dln2_w,
                                 double *dln2_b, double *dw2, double *db2)
{
    (void)b2;
    const int rb = store_bf16 != 0;
    const int64_t T = offsets[B];
    const int64_t NU = (int64_t)H * dv, NQ = (int64_t)H * dqk, NW = 2 * NU + 2 * NQ;
    double *xh1 = malloc(sizeof(double) * T * D), *rstd1 = malloc(sizeof(double) * T);
    double *n = malloc(sizeof(double) * T * D);
    double *z = malloc(sizeof(double) * T * NW), *s = malloc(sizeof(double) * T * NW);
    double *qq = malloc(sizeof(double) * T * NQ), *kk = malloc(sizeof(double) * T * NQ);
    double *vv = malloc(sizeof(double) * T * NU), *uu = malloc(sizeof(double) * T * NU);
    double *a = malloc(sizeof(double) * T * NU), *ah = malloc(sizeof(double) * T * NU);
    double *rstd2 = malloc(sizeof(double) * T), *yh = malloc(sizeof(double) * T * NU);
    double *y = malloc(sizeof(double) * T * NU), *dy = malloc(sizeof(double) * T * NU);
    double *dyh = malloc(sizeof(double) * T * NU), *da = malloc(sizeof(double) * T * NU);
    double *dq = malloc(sizeof(double) * T * NQ), *dk = malloc(sizeof(double) * T * NQ);
    double *dvv = malloc(sizeof(double) * T * NU), *dz = malloc(sizeof(double) * T * NW);
    double *dn = malloc(sizeof(double) * T * D);

    /* forward */
    ln_stats(T, D, x, eps, xh1, rstd1);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < D; ++c)
            n[t * D + c] = xh1[t * D + c] * ln1_w[c] + (ln1_b ? ln1_b[c] : 0.0);
    if (rb) round_all(n, T * D);
    linear(T, D, NW, n, w1, b1, z);
    for (int64_t i = 0; i < T * NW; ++i) s[i] = silu(z[i]);
    if (rb) {
        round_all(z, T * NW);
        round_all(s, T * NW);
    }
    for (int64_t t = 0; t < T; ++t) {
        const double *sr = s + t * NW;
        memcpy(uu + t * NU, sr, sizeof(double) * NU);
        memcpy(vv + t * NU, sr + NU, sizeof(double) * NU);
        memcpy(qq + t * NQ, sr + 2 * NU, sizeof(double) * NQ);
        memcpy(kk + t * NQ, sr + 2 * NU + NQ, sizeof(double) * NQ);
    }
    oracle_sla_fwd(B, offsets, num_targets, H, dqk, dv, k1, k2, ctx, N, alpha, qq, kk, vv, a,
                   NULL);
    if (rb) round_all(a, T * NU);
    ln_stats(T, NU, a, eps, ah, rstd2);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < NU; ++c) {
            yh[t * NU + c] = ah[t * NU + c] * ln2_w[c] + (ln2_b ? ln2_b[c] : 0.0);
            y[t * NU + c] = yh[t * NU + c] * uu[t * NU + c];
        }
    if (rb) round_all(y, T * NU);

    /* out = y W2^T + b2 + x:  dW2 = dout^T y, db2 = colsum(dout), dy = dout W2 */
    for (int64_t i = 0; i < D * NU; ++i) dw2[i] = 0.0;
    if (db2)
        for (int64_t c = 0; c < D; ++c) db2[c] = 0.0;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t d = 0; d < D; ++d) {
            const double g = dout[t * D + d];
            if (db2) db2[d] += g;
            for (int64_t c = 0; c < NU; ++c) dw2[d * NU + c] += g * y[t * NU + c];
        }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < NU; ++c) {
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d) acc += dout[t * D + d] * w2[d * NU + c];
            dy[t * NU + c] = acc;
        }
    if (rb) round_all(dy, T * NU);

    /* y = yh (.) U:  dU = dy (.) yh, dyh = dy (.) U; yh = ah * g2 + b2n */
    for (int64_t i = 0; i < T * NU; ++i) dyh[i] = dy[i] * uu[i];
    for (int64_t c = 0; c < NU; ++c) {
        dln2_w[c] = 0.0;
        if (dln2_b) dln2_b[c] = 0.0;
    }
    ln_backward(T, NU, dyh, ah, rstd2, ln2_w, da, dln2_w, dln2_b);
    if (rb) round_all(da, T * NU);

    /* A = SLA(Q, K, V) */
    oracle_sla_bwd(B, offsets, num_targets, H, dqk, dv, k1, k2, ctx, N, alpha, qq, kk, vv, da, dq,
                   dk, dvv, NULL, NULL);
    if (rb) {
        round_all(dq, T * NQ);
        round_all(dk, T * NQ);
        round_all(dvv, T * NU);
    }

    /* [U V Q K] = SiLU(z):  dz = d[U V Q K] (.) SiLU'(z) */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double *dzr = dz + t * NW;
        const double *zr = z + t * NW;
        for (int64_t c = 0; c < NU; ++c) {
            const double du = dy[t * NU + c] * yh[t * NU + c];
            dzr[c] = rb ? oracle_round_bf16(du) : du;
        }
        for (int64_t c = 0; c < NU; ++c) dzr[NU + c] = dvv[t * NU + c];
        for (int64_t c = 0; c < NQ; ++c) dzr[2 * NU + c] = dq[t * NQ + c];
        for (int64_t c = 0; c < NQ; ++c) dzr[2 * NU + NQ + c] = dk[t * NQ + c];
        for (int64_t c = 0; c < NW; ++c) {
            dzr[c] *= dsilu(zr[c]);
            if (rb) dzr[c] = oracle_round_bf16(dzr[c]);
        }
    }

    /* z = n W1^T + b1:  dW1 = dz^T n, db1 = colsum(dz), dn = dz W1 */
    for (int64_t i = 0; i < NW * D; ++i) dw1[i] = 0.0;
    if (db1)
        for (int64_t c = 0; c < NW; ++c) db1[c] = 0.0;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t o = 0; o < NW; ++o) {
            const double g = dz[t * NW + o];
            if (db1) db1[o] += g;
            for (int64_t c = 0; c < D; ++c) dw1[o * D + c] += g * n[t * D + c];
        }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int64_t o = 0; o < NW; ++o) acc += dz[t * NW + o] * w1[o * D + c];
            dn[t * D + c] = acc;
        }
    if (rb) round_all(dn, T * D);

    /* n = xh * g1 + b1n, plus the residual path of out */
    for (int64_t c = 0; c < D; ++c) {
        dln1_w[c] = 0.0;
        if (dln1_b) dln1_b[c] = 0.0;
    }
    ln_backward(T, D, dn, xh1, rstd1, ln1_w, dx, dln1_w, dln1_b);
    for (int64_t i = 0; i < T * D; ++i) dx[i] += dout[i];
    if (rb) round_all(dx, T * D);

    free(xh1); free(rstd1); free(n); free(z); free(s); free(qq); free(kk); free(vv); free(uu);
    free(a); free(ah); free(rstd2); free(yh); free(y); free(dy); free(dyh); free(da); free(dq);
    free(dk); free(dvv); free(dz); free(dn);
}

/* ------------------------------------------------------------------------ */
/* attention truncation                                                      */
/* ------------------------------------------------------------------------ */

/* Per sequence keep, in order: the contextual prefix [0, c), the most recent
 * tail_len history tokens [c + max(0, H_b - tail_len), c + H_b), and the
 * targets [U, L), where U = L - T_b, c = min(ctx, U), H_b = U - c.
 * Writes new_offsets [B+1] and gather_idx [new T] (global source rows).
 * Returns the new total. */
EXPORT int64_t oracle_truncate(int B, const int64_t *offsets, const int32_t *num_targets,
                               int64_t ctx, int64_t tail_len, int64_t *new_offsets,
                               int64_t *gather_idx)
{
    int64_t n = 0;
    new_offsets[0] = 0;
    for (int b = 0; b < B; ++b) {
        int64_t base = offsets[b], L = offsets[b + 1] - offsets[b];
        int64_t U = L - seq_targets(num_targets, b);
        int64_t c = ctx < U ? ctx : U;
        int64_t Hb = U - c;
        int64_t keep_from = c + (Hb > tail_len ? Hb - tail_len : 0);
        for (int64_t i = 0; i < L; ++i) {
            int keep = (i < c) || (i >= keep_from && i < U) || (i >= U);
            if (keep) {
                if (gather_idx) gather_idx[n] = base + i;
                ++n;
            }
        }
        new_offsets[b + 1] = n;
    }
    return n;
}

EXPORT int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
