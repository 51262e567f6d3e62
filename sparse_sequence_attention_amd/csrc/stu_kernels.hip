// stu_kernels.hip -- the STU layer around the attention (ULTRA-HSTU paper,
// section 3 Eq.1-5, operation order of Code Listing 1) and attention
// truncation (section 4.3), for gfx950:
//   - row LayerNorm (Eq.1) and the gated LayerNorm(A) (.) U (Eq.4), fp32
//     statistics over the whole row, bf16 in/out;
//   - a bf16 MFMA GEMM C = A W^T with fused epilogues: SiLU(acc + b) for the
//     U,V,Q,K projection (Eq.2, one fused projection as in HSTU notes section
//     2.4 Eq.1) and acc + b + residual for the output projection (Eq.4-5; the
//     residual as a 2-D bias in the GEMM epilogue, ULTRA-HSTU section 4.2.2);
//   - the truncation index and row gather.
#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

// ---------------------------------------------------------------------------
// LayerNorm: a wave per row (two rows for up to 512 columns), up to 2048 columns
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Each wave normalises RPW rows of up to 512 * NCH columns; every load of a
// row (x, the gate u, the weight and bias) is issued before the reductions,
// so a wave waits for memory once.  Lane l holds the 16-byte chunks l,
// l + 64, ... of a row.
template <bool GATED, int NCH, int RPW>
__global__ __launch_bounds__(256) void layernorm_bf16_kernel(const uint16_t *x, int64_t ldx,
                                                             const uint16_t *u, int64_t ldu,
                                                             const float *w, const float *bias,
                                                             uint16_t *y, int64_t ldy,
                                                             int64_t rows, int cols, float eps)
{
    const int lane = threadIdx.x & 63;
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
    if (row0 >= rows) return;
    const int nchunk = cols / 8;
    uint4 xr[RPW][NCH], ur[RPW][NCH];
    float4 wv[NCH][2], bv[NCH][2];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nchunk) {
#pragma unroll
            for (int k = 0; k < RPW; ++k) {
                if (row0 + k < rows) {
                    xr[k][c] = ld16(x + (row0 + k) * ldx + 8 * ch);
                    if (GATED) ur[k][c] = ld16(u + (row0 + k) * ldu + 8 * ch);
                }
            }
            wv[c][0] = *reinterpret_cast<const float4 *>(w + 8 * ch);
            wv[c][1] = *reinterpret_cast<const float4 *>(w + 8 * ch + 4);
            if (bias) {
                bv[c][0] = *reinterpret_cast<const float4 *>(bias + 8 * ch);
                bv[c][1] = *reinterpret_cast<const float4 *>(bias + 8 * ch + 4);
            } else {
                bv[c][0] = bv[c][1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        const int64_t row = row0 + k;
        if (row >= rows) break;
        float v[NCH][8];
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (lane + 64 * c < nchunk) {
                const uint32_t wd[4] = {xr[k][c].x, xr[k][c].y, xr[k][c].z, xr[k][c].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[c][2 * e] = bf16_lo(wd[e]);
                    v[c][2 * e + 1] = bf16_hi(wd[e]);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) s += v[c][e];
            }
        }
        const float mean = wave_sum(s) / (float)cols;
        float q = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (lane + 64 * c < nchunk) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float d = v[c][e] - mean;
                    q += d * d;
                }
            }
        }
        const float rstd = rsqrtf(wave_sum(q) / (float)cols + eps);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = lane + 64 * c;
            if (ch < nchunk) {
                const float wf[8] = {wv[c][0].x, wv[c][0].y, wv[c][0].z, wv[c][0].w,
                                     wv[c][1].x, wv[c][1].y, wv[c][1].z, wv[c][1].w};
                const float bf[8] = {bv[c][0].x, bv[c][0].y, bv[c][0].z, bv[c][0].w,
                                     bv[c][1].x, bv[c][1].y, bv[c][1].z, bv[c][1].w};
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = (v[c][e] - mean) * rstd * wf[e] + bf[e];
                if (GATED) {
                    const uint32_t uw[4] = {ur[k][c].x, ur[k][c].y, ur[k][c].z, ur[k][c].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        o[2 * e] *= bf16_lo(uw[e]);
                        o[2 * e + 1] *= bf16_hi(uw[e]);
                    }
                }
                const uint2 lo = cvt4_u2(o[0], o[1], o[2], o[3]);
                const uint2 hi = cvt4_u2(o[4], o[5], o[6], o[7]);
                *reinterpret_cast<uint4 *>(y + row * ldy + 8 * ch) = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
        }
    }
}

// cols % 8 == 0 and cols <= 2048 (checked by the callers)
template <bool GATED>
static hipError_t launch_ln(const uint16_t *x, int64_t ldx, const uint16_t *u, int64_t ldu,
                            const float *w, const float *b, uint16_t *y, int64_t ldy, int64_t rows,
                            int cols, float eps, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    if (cols % 8 != 0 || cols > 2048) return hipErrorInvalidValue;
    const dim3 block(256);
    if (cols <= 512) {
        constexpr int RPW = 2;
        hipLaunchKernelGGL((layernorm_bf16_kernel<GATED, 1, RPW>),
                           dim3((unsigned)((rows + 4 * RPW - 1) / (4 * RPW))), block, 0, st, x, ldx,
                           u, ldu, w, b, y, ldy, rows, cols, eps);
    } else if (cols <= 1024) {
        hipLaunchKernelGGL((layernorm_bf16_kernel<GATED, 2, 1>), dim3((unsigned)((rows + 3) / 4)),
                           block, 0, st, x, ldx, u, ldu, w, b, y, ldy, rows, cols, eps);
    } else {
        hipLaunchKernelGGL((layernorm_bf16_kernel<GATED, 4, 1>), dim3((unsigned)((rows + 3) / 4)),
                           block, 0, st, x, ldx, u, ldu, w, b, y, ldy, rows, cols, eps);
    }
    return hipGetLastError();
}

hipError_t launch_layernorm_bf16(const void *x, const float *w, const float *b, void *y,
                                 int64_t rows, int cols, float eps, hipStream_t st)
{
    return launch_ln<false>((const uint16_t *)x, (int64_t)cols, nullptr, 0, w, b, (uint16_t *)y,
                            (int64_t)cols, rows, cols, eps, st);
}

hipError_t launch_gated_layernorm_bf16(const void *a, int64_t lda, const void *u, int64_t ldu,
                                       const float *w, const float *b, void *y, int64_t rows,
                                       int cols, float eps, hipStream_t st)
{
    return launch_ln<true>((const uint16_t *)a, lda, (const uint16_t *)u, ldu, w, b, (uint16_t *)y,
                           (int64_t)cols, rows, cols, eps, st);
}

// ---------------------------------------------------------------------------
// GEMM  C[M][N] = epi(A[M][K] . W[N][K]^T), with z = acc (+ bias[n]):
//   EPI 0: C = SiLU(z)        EPI 1: C = z + R (residual)
//   EPI 2: C = z              EPI 3: C = SiLU(z) and Z = z (the pre-activation)
// (the kernel lives in gemm_nt.hip, shared with the FP8 projections)
// ---------------------------------------------------------------------------
hipError_t launch_gemm_bf16(const void *A, int64_t lda, const void *W, int64_t ldw,
                            const float *bias, const void *R, int64_t ldr, void *C, int64_t ldc,
                            void *Z, int64_t ldz, int64_t M, int N, int K, int epi, hipStream_t st)
{
    return launch_gemm_nt_bf16(A, lda, W, ldw, bias, R, ldr, C, ldc, Z, ldz, M, N, K, epi, st);
}

// ---------------------------------------------------------------------------
// attention truncation
// ---------------------------------------------------------------------------
// Per sequence: c = min(ctx, U) contextual tokens, history [c, U), kept history
// [keep_from, U) with keep_from = c + max(0, (U - c) - tail), then the targets
// [U, L).  The kept tokens after the contextual prefix are the contiguous run
// [keep_from, L).
__device__ __forceinline__ void trunc_dims(const int64_t *offsets, const int32_t *num_targets,
                                           int b, int ctx, int tail, int &L, int &c,
                                           int &keep_from)
{
    L = (int)(offsets[b + 1] - offsets[b]);
    const int U = L - (num_targets ? num_targets[b] : 0);
    c = imin(ctx, U);
    const int hb = U - c;
    keep_from = c + (hb > tail ? hb - tail : 0);
}

__global__ __launch_bounds__(1024) void truncate_offsets_kernel(int B, const int64_t *offsets,
                                                                const int32_t *num_targets,
                                                                int ctx, int tail,
                                                                int64_t *new_offsets,
                                                                int32_t *new_num_targets)
{
    __shared__ int64_t buf[2][1024];
    __shared__ int64_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int start = 0; start < B; start += 1024) {
        const int b = start + tid;
        int64_t v = 0;
        if (b < B) {
            int L, c, kf;
            trunc_dims(offsets, num_targets, b, ctx, tail, L, c, kf);
            v = c + (L - kf);
            if (new_num_targets) new_num_targets[b] = num_targets ? num_targets[b] : 0;
        }
        int cur = 0;
        buf[cur][tid] = v;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            int64_t a = buf[cur][tid];
            if (tid >= off) a += buf[cur][tid - off];
            buf[cur ^ 1][tid] = a;
            cur ^= 1;
            __syncthreads();
        }
        const int64_t inc = buf[cur][tid];
        const int64_t c0 = carry;
        if (b < B) new_offsets[b] = c0 + inc - v;
        __syncthreads();
        if (tid == 1023) carry = c0 + inc;
        __syncthreads();
    }
    if (tid == 0) new_offsets[B] = carry;
}

// one wave per kept row: index + 16-byte chunks of the row
__global__ __launch_bounds__(256) void truncate_gather_kernel(
    int B, const int64_t *offsets, const int32_t *num_targets, int ctx, int tail,
    const int64_t *new_offsets, const uint8_t *x, int row_bytes, int64_t *gather_idx,
    uint8_t *x_out, int64_t capacity)
{
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t total = new_offsets[B];
    if (r >= total || r >= capacity) return;
    int lo = 0, hi = B - 1;  // last b with new_offsets[b] <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (new_offsets[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    const int b = lo;
    int L, c, kf;
    trunc_dims(offsets, num_targets, b, ctx, tail, L, c, kf);
    const int li = (int)(r - new_offsets[b]);
    const int src = li < c ? li : kf + (li - c);
    const int64_t srow = offsets[b] + src;
    if (lane == 0 && gather_idx) gather_idx[r] = srow;
    if (x_out) {
        const uint8_t *s = x + srow * row_bytes;
        uint8_t *d = x_out + r * row_bytes;
        for (int e = 16 * lane; e < row_bytes; e += 16 * 64)
            *reinterpret_cast<uint4 *>(d + e) = *reinterpret_cast<const uint4 *>(s + e);
    }
}

hipError_t launch_truncate(int B, int64_t T, const int64_t *offsets, const int32_t *num_targets,
                           int ctx, int tail, const void *x, int hidden, int elem_bytes,
                           int64_t *new_offsets, int32_t *new_num_targets, int64_t *gather_idx,
                           void *x_out, int64_t capacity, int32_t *, hipStream_t st)
{
    hipLaunchKernelGGL(truncate_offsets_kernel, dim3(1), dim3(1024), 0, st, B, offsets,
                       num_targets, ctx, tail, new_offsets, new_num_targets);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = capacity < T ? capacity : T;
    if (rows <= 0 || (!gather_idx && !x_out)) return hipSuccess;
    dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    hipLaunchKernelGGL(truncate_gather_kernel, grid, block, 0, st, B, offsets, num_targets, ctx,
                       tail, (const int64_t *)new_offsets, (const uint8_t *)x,
                       hidden * elem_bytes, gather_idx, (uint8_t *)x_out, capacity);
    return hipGetLastError();
}

// The adjoint of the gather (the truncation backward): one wave per SOURCE
// row s.  Row s of sequence b (li = s - offsets[b]) was kept iff li < c or li
// >= keep_from, as row new_offsets[b] + (li < c ? li : c + li - keep_from);
// dx[s] is that row of dy, or zero for a dropped token.  Every dx row is
// written once, and no two waves write the same row: no atomics.
__global__ __launch_bounds__(256) void truncate_scatter_kernel(
    int B, int64_t T, const int64_t *offsets, const int32_t *num_targets, int ctx, int tail,
    const int64_t *new_offsets, const uint8_t *dy, int row_bytes, uint8_t *dx)
{
    const int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (s >= T) return;
    int lo = 0, hi = B - 1;  // last b with offsets[b] <= s
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= s) lo = mid;
        else hi = mid - 1;
    }
    const int b = lo;
    int L, c, kf;
    trunc_dims(offsets, num_targets, b, ctx, tail, L, c, kf);
    const int li = (int)(s - offsets[b]);
    const bool kept = li < c || li >= kf;
    const int64_t r = new_offsets[b] + (li < c ? li : c + (li - kf));
    uint8_t *d = dx + s * row_bytes;
    if (kept) {  // uniform per wave: dy is read only for kept rows
        const uint8_t *src = dy + r * row_bytes;
        for (int e = 16 * lane; e < row_bytes; e += 16 * 64)
            *reinterpret_cast<uint4 *>(d + e) = *reinterpret_cast<const uint4 *>(src + e);
    } else {
        const uint4 z = {0u, 0u, 0u, 0u};
        for (int e = 16 * lane; e < row_bytes; e += 16 * 64)
            *reinterpret_cast<uint4 *>(d + e) = z;
    }
}

hipError_t launch_truncate_bwd(int B, int64_t T, const int64_t *offsets,
                               const int32_t *num_targets, int ctx, int tail,
                               const int64_t *new_offsets, const void *dy, int hidden,
                               int elem_bytes, void *dx, hipStream_t st)
{
    if (T <= 0 || B <= 0) return hipSuccess;
    dim3 grid((unsigned)((T + 3) / 4)), block(256);
    hipLaunchKernelGGL(truncate_scatter_kernel, grid, block, 0, st, B, T, offsets, num_targets,
                       ctx, tail, new_offsets, (const uint8_t *)dy, hidden * elem_bytes,
                       (uint8_t *)dx);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// target rows (candidates) of a jagged batch, gathered into a column block of
// a [total targets][ld_out] output (Mixture of Transducers: each channel's
// candidate embeddings side by side)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void target_offsets_kernel(int B, const int32_t *num_targets,
                                                              int64_t *toffs)
{
    __shared__ int64_t buf[2][1024];
    __shared__ int64_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int start = 0; start < B; start += 1024) {
        const int b = start + tid;
        const int64_t v = b < B ? (num_targets ? num_targets[b] : 0) : 0;
        int cur = 0;
        buf[cur][tid] = v;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            int64_t a = buf[cur][tid];
            if (tid >= off) a += buf[cur][tid - off];
            buf[cur ^ 1][tid] = a;
            cur ^= 1;
            __syncthreads();
        }
        const int64_t c0 = carry;
        if (b < B) toffs[b] = c0 + buf[cur][tid] - v;
        __syncthreads();
        if (tid == 1023) carry = c0 + buf[cur][tid];
        __syncthreads();
    }
    if (tid == 0) toffs[B] = carry;
}

__global__ __launch_bounds__(256) void gather_targets_kernel(
    int B, const int64_t *offsets, const int32_t *num_targets, const int64_t *toffs,
    const uint8_t *x, int row_bytes, uint8_t *out, int64_t ld_out_bytes, int64_t col_bytes,
    int64_t capacity)
{
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t total = toffs[B];
    if (r >= total || r >= capacity) return;
    int lo = 0, hi = B - 1;  // last b with toffs[b] <= r (sequences without targets skipped)
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (toffs[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    const int b = lo;
    const int64_t srow = offsets[b + 1] - num_targets[b] + (r - toffs[b]);
    const uint8_t *src = x + srow * row_bytes;
    uint8_t *dst = out + r * ld_out_bytes + col_bytes;
    for (int e = 16 * lane; e < row_bytes; e += 16 * 64)
        *reinterpret_cast<uint4 *>(dst + e) = *reinterpret_cast<const uint4 *>(src + e);
}

hipError_t launch_gather_targets(int B, const int64_t *offsets, const int32_t *num_targets,
                                 const void *x, int row_bytes, int64_t *toffs, void *out,
                                 int64_t ld_out_bytes, int64_t col_bytes, int64_t capacity,
                                 hipStream_t st)
{
    hipLaunchKernelGGL(target_offsets_kernel, dim3(1), dim3(1024), 0, st, B, num_targets, toffs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !out || capacity <= 0) return e;
    hipLaunchKernelGGL(gather_targets_kernel, dim3((unsigned)((capacity + 3) / 4)), dim3(256), 0,
                       st, B, offsets, num_targets, (const int64_t *)toffs, (const uint8_t *)x,
                       row_bytes, (uint8_t *)out, ld_out_bytes, col_bytes, capacity);
    return hipGetLastError();
}

}  // namespace sla
