// sla_kernels.h -- kernel parameter blocks and the host-side launch functions
// that each .hip translation unit provides to the C-ABI layer (sla_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sla_internal.h"

namespace sla {

// Record msg as the calling thread's last error (sla_last_error) and return
// status: for entry points implemented outside sla_api.cpp.
int set_last_error(int status, const char *msg);

struct AttnParams {
    const void *q, *k, *v;
    void *o;
    const void *dout;
    void *dq, *dk, *dv;
    int64_t ldq, ldk, ldv, ldo, lddo, lddq, lddk, lddv;  // token strides, elements
    const int64_t *offsets;
    const int32_t *num_targets;
    int64_t T;              // total tokens
    int B, H, d, d_v, k1, k2e;  // d: the Q / K head width d_qk, d_v: the V width
    float alpha;            // pre-activation factor
    float inv_n;            // 1 / N
    float out_scale;        // alpha / N
    float neg_alpha_log2e;  // -alpha * log2(e)
    Sched s;
    float *partials;        // fp32 partial dK|dV of split prefix key tiles
    // stored-dS backward (null: dQ recomputes S and dP): the dK/dV kernel
    // writes each 64-row step x 128-key tile of dS (DS_BLOCK_BYTES, bf16) to
    // block (h * ds_head_blocks + ds_base[key tile] + step), which dQ reads
    uint8_t *ds;
    int64_t ds_head_blocks;
    int grid_fwd;           // upper bound of forward / dQ work items (x heads)
    int grid_bwd;           // upper bound of dK/dV work items (x heads)
    int grid_red;           // upper bound of reduce items (x heads)
    int out_f32;            // bf16 path: O, dQ, dK, dV written as fp32
    // candidate scoring against a cached history (null: the ordinary forward).
    // Sequence b is then the history offsets[b] .. offsets[b+1] (keys k, v)
    // followed by the candidates cand_offsets[b] .. cand_offsets[b+1] (rows
    // q, o; their own keys kc, vc); only the candidate rows are computed.
    const int64_t *cand_offsets;
    const void *kc, *vc;
    int64_t ldkc, ldvc;
};

// Head widths (d_qk, d_v) the attention kernels are built for: each of 32,
// 64 and 128, in any pair.
inline bool attn_dims_supported(int dqk, int dv)
{
    const bool ok_qk = dqk == 32 || dqk == 64 || dqk == 128;
    const bool ok_v = dv == 32 || dv == 64 || dv == 128;
    return ok_qk && ok_v;
}

// f(integral_constant<int, d_qk>, integral_constant<int, d_v>) for the head
// widths of p
template <typename F>
hipError_t with_head_dims(const AttnParams &p, F &&f)
{
    using I32 = std::integral_constant<int, 32>;
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    auto v = [&](auto QK) -> hipError_t {
        switch (p.d_v) {
        case 32: return f(QK, I32{});
        case 64: return f(QK, I64{});
        case 128: return f(QK, I128{});
        default: return hipErrorInvalidValue;
        }
    };
    switch (p.d) {
    case 32: return v(I32{});
    case 64: return v(I64{});
    case 128: return v(I128{});
    default: return hipErrorInvalidValue;
    }
}

// Sizes (int32 counts / bytes) of the workspace regions, from host-known data.
struct WsLayout {
    size_t sched_off, part_off, total;
    int64_t fwd_items, bwd_items, red_items, part_slots;  // upper bounds (per head)
    // stored-dS backward (ds_blocks == 0: dQ recomputes S and dP)
    size_t ktile_off, dsb_off, ds_off;
    int64_t ds_blocks;  // upper bound of dS blocks per head
};

hipError_t launch_sched(const AttnParams &p, hipStream_t st);
// forward over candidate rows only (p.cand_offsets set), bf16
hipError_t launch_fwd_candidates_bf16(const AttnParams &p, hipStream_t st);
// Optional check of the jagged layout; result: int32[2] device scratch
// (code, sequence).  ctx < 0 skips the truncation check.
hipError_t launch_validate(const int64_t *offsets, const int32_t *num_targets, int B, int64_t T,
                           int ctx, int32_t *result, hipStream_t st);
hipError_t launch_sched_dump(const AttnParams &p, int op, int32_t *records, int64_t capacity,
                             int32_t *count, hipStream_t st);
hipError_t launch_fwd_bf16(const AttnParams &p, hipStream_t st);
hipError_t launch_bwd_dkdv_bf16(const AttnParams &p, hipStream_t st);  // + prefix reduce
hipError_t launch_bwd_dq_bf16(const AttnParams &p, hipStream_t st);
hipError_t launch_fwd_f32(const AttnParams &p, hipStream_t st);
hipError_t launch_bwd_dkdv_f32(const AttnParams &p, hipStream_t st);
hipError_t launch_bwd_dq_f32(const AttnParams &p, hipStream_t st);

// STU layer pieces (bf16 storage)
hipError_t launch_layernorm_bf16(const void *x, const float *w, const float *b, void *y,
                                 int64_t rows, int cols, float eps, hipStream_t st);
hipError_t launch_gated_layernorm_bf16(const void *a, int64_t lda, const void *u, int64_t ldu,
                                       const float *w, const float *b, void *y, int64_t rows,
                                       int cols, float eps, hipStream_t st);
// C[M][N] = epilogue(A[M][K] . W[N][K]^T), z = acc + bias: epi 0 = SiLU(z),
// 1 = z + R, 2 = z, 3 = SiLU(z) with z also stored to Z
hipError_t launch_gemm_bf16(const void *A, int64_t lda, const void *W, int64_t ldw,
                            const float *bias, const void *R, int64_t ldr, void *C, int64_t ldc,
                            void *Z, int64_t ldz, int64_t M, int N, int K, int epi,
                            hipStream_t st);

// The projection GEMM core (gemm_nt.hip): 256 x 128|256 tiles, DMA-fed
// four-stage ring, row-contiguous stores.  bf16: N % 128, K % 32; FP8: N % 128,
// K % 64, epi 0..2 (sa, sw the row scales of A and W).
hipError_t launch_gemm_nt_bf16(const void *A, int64_t lda, const void *W, int64_t ldw,
                               const float *bias, const void *R, int64_t ldr, void *C, int64_t ldc,
                               void *Z, int64_t ldz, int64_t M, int N, int K, int epi,
                               hipStream_t st);
hipError_t launch_gemm_nt_fp8(const void *A, const float *sa, const void *W, const float *sw,
                              const float *bias, const void *R, int64_t ldr, void *C, int64_t ldc,
                              int64_t M, int N, int K, int epi, hipStream_t st);

// STU layer backward pieces (stu_bwd.hip)
// C[M][N] = sum_t A[t][m] B[t][n] over T rows, fp32: tn_plan(T, M, N).splits
// token ranges into part [splits][M][N], then summed in range order into out.
// M, N multiples of 128; zero: >= 512 bytes of zeros (16-byte aligned).
struct TnPlan {
    int tile, splits;
    int64_t rows;  // tokens per range (a multiple of 32)
};
TnPlan tn_plan(int64_t T, int M, int N);
hipError_t launch_gemm_tn_bf16(const void *A, int64_t lda, const void *B, int64_t ldb, int64_t T,
                               int M, int N, const void *zero, float *part, float *out,
                               hipStream_t st);
// out[i] = sum_s part[s][i] (count % 4 == 0) in a fixed order; mid (nullable,
// SUM_MID_FLOATS floats) spreads a short range with many splits over more
// workgroups.
constexpr int64_t SUM_MID_FLOATS = 131072;
hipError_t sum_splits(const float *part, int64_t count, int splits, float *out, float *mid,
                      hipStream_t st);
int colsum_blocks(int64_t T);
hipError_t launch_colsum_bf16(const void *X, int64_t ld, int64_t T, int C, float *part, float *out,
                              float *mid, hipStream_t st);
int ln_bwd_blocks(int64_t rows);
// LayerNorm backward (gated: y = (LN(x) w + b) (.) u; du and, when y is
// non-NULL, y also written); part_w / part_b: [ln_bwd_blocks(rows)][cols];
// db nullable; res (plain only, nullable) is added to dx.
// MFMA-only throughput probe (sla_probe.hip): `blocks` workgroups of four
// waves, each wave `iters` rounds of four bf16 32x32x16 MFMAs; clk[0] gets the
// shader clocks and clk[1] the 100 MHz ticks that wave 0 of workgroup 0 saw.
hipError_t launch_mfma_peak(int blocks, int iters, float *sink, unsigned long long *clk,
                            hipStream_t st);
double mfma_peak_flops(int blocks, int iters);
// modes of the issue-rate probe (sla_probe.hip); one workgroup of 512
// threads per CU, `sink` one float per thread
enum IssueMode { ISSUE_MFMA = 0, ISSUE_VALU, ISSUE_SPLIT, ISSUE_MIXED, ISSUE_SPLIT_A, ISSUE_EXP, ISSUE_RCP,
                 ISSUE_MODES };
hipError_t launch_issue_probe(int mode, int blocks, int iters, float *sink, hipStream_t st);
hipError_t launch_ln_bwd_bf16(bool gated, const void *x, int64_t ldx, const void *dy, int64_t lddy,
                              const void *u, int64_t ldu, const float *w, const float *b,
                              const void *res, int64_t ldres, void *dx, int64_t lddx, void *du,
                              int64_t lddu, void *y, int64_t ldy, float *part_w, float *part_b,
                              float *mid, float *dw, float *db,
                              int64_t rows, int cols, float eps, hipStream_t st);
hipError_t launch_dsilu_bf16(void *ds, int64_t ldd, const void *z, int64_t ldz, int64_t rows,
                             int cols, hipStream_t st);
hipError_t launch_transpose_bf16(const void *src, int R, int C, void *dst, hipStream_t st);
hipError_t launch_fill_f32(float *dst, size_t n, float v, hipStream_t st);
// target rows of each sequence into rows toffs[b] .. of out, bytes
// [col_bytes, col_bytes + row_bytes) of each out row; toffs [B+1] written
hipError_t launch_gather_targets(int B, const int64_t *offsets, const int32_t *num_targets,
                                 const void *x, int row_bytes, int64_t *toffs, void *out,
                                 int64_t ld_out_bytes, int64_t col_bytes, int64_t capacity,
                                 hipStream_t st);

// FP8 projections (stu_fp8.hip): row-wise e4m3 quantisation q = e4m3(x 448 /
// max|x|), scale = max|x| / 448; cols % 8 == 0, <= 2048
hipError_t launch_quant_rows_fp8(const void *x, int64_t ldx, int64_t rows, int cols, void *q,
                                 float *scale, hipStream_t st);
hipError_t launch_ln_quant_fp8(bool gated, const void *x, int64_t ldx, const void *u, int64_t ldu,
                               const float *w, const float *b, void *q, float *scale, int64_t rows,
                               int cols, float eps, hipStream_t st);
// C[M][N] = epi(sa[m] sw[n] A[m][:] . W[n][:] + bias[n]); epi 0 = SiLU, 1 = + R
hipError_t launch_gemm_fp8(const void *A, const float *sa, const void *W, const float *sw,
                           const float *bias, const void *R, int64_t ldr, void *C, int64_t ldc,
                           int64_t M, int N, int K, int epi, hipStream_t st);
// adjoint of the truncation gather: dx [T][hidden] fully written
hipError_t launch_truncate_bwd(int B, int64_t T, const int64_t *offsets,
                               const int32_t *num_targets, int ctx, int tail,
                               const int64_t *new_offsets, const void *dy, int hidden,
                               int elem_bytes, void *dx, hipStream_t st);
hipError_t launch_truncate(int B, int64_t T, const int64_t *offsets, const int32_t *num_targets,
                           int ctx, int tail, const void *x, int hidden, int elem_bytes,
                           int64_t *new_offsets, int32_t *new_num_targets, int64_t *gather_idx,
                           void *x_out, int64_t capacity, int32_t *scratch_base,
                           hipStream_t st);

}  // namespace sla
