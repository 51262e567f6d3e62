// stu_fp8.hip -- FP8 projections of the STU layer (ULTRA-HSTU paper, section
// 4.2.2, mixed precision: both projections in FP8, every other step bf16; the
// row-wise scale and quantisation fused into the LayerNorm that produces the
// operand, and the post-attention projection's 2-D residual fused into its
// epilogue).
//
// Format: FP8 E4M3 (OCP e4m3fn, largest finite 448).  A row x is stored as
// q = e4m3(x * (448 / max|x|)) with the scale s = max|x| / 448 (an all-zero
// row: q = 0, s = 1), so x ~ q * s.  The conversion is v_cvt_pk_fp8_f32
// (round to nearest even); values are clamped to +-448 first, because the
// conversion turns magnitudes past 464 into NaN.
//
// GEMM: v_mfma_f32_32x32x64_f8f6f4 (fp8 x fp8, fp32 accumulation).  Lane l
// holds operand row l % 32, bytes 32 * (l / 32) .. +32 of the 64-deep slice;
// the accumulator layout is that of the bf16 32x32 products.
#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

typedef int intx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float wave_max_f(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum_f(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// 8 floats -> 8 e4m3 bytes (clamped to +-448), as a uint2
__device__ __forceinline__ uint2 to_e4m3x8(const float *v, float inv)
{
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = fminf(fmaxf(v[4 * h + e] * inv, -448.0f), 448.0f);
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        w[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
    }
    return make_uint2(w[0], w[1]);
}

__device__ __forceinline__ void bf16x8_to_f(const uint4 &r, float *f)
{
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_lo(w[e]);
        f[2 * e + 1] = bf16_hi(w[e]);
    }
}

// ---------------------------------------------------------------------------
// Row quantisation of a bf16 [rows][cols] matrix (weights), one wave per row,
// cols % 8 == 0 and cols <= 2048.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_rows_fp8_kernel(const uint16_t *x, int64_t ldx,
                                                             int64_t rows, int cols, uint8_t *q,
                                                             float *scale)
{
    constexpr int MAXC = 4;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int nchunk = cols / 8;
    float v[MAXC][8];
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nchunk) {
            bf16x8_to_f(ld16(x + row * ldx + 8 * ch), v[c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[c][e]));
        }
    }
    a = wave_max_f(a);
    const float inv = a > 0.0f ? 448.0f / a : 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nchunk)
            *reinterpret_cast<uint2 *>(q + row * cols + 8 * ch) = to_e4m3x8(v[c], inv);
    }
    if (lane == 0) scale[row] = a > 0.0f ? a / 448.0f : 1.0f;
}

hipError_t launch_quant_rows_fp8(const void *x, int64_t ldx, int64_t rows, int cols, void *q,
                                 float *scale, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    if (cols % 8 != 0 || cols > 2048) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                       (const uint16_t *)x, ldx, rows, cols, (uint8_t *)q, scale);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LayerNorm (gated: (LN(a) w + b) (.) u) of a bf16 row, quantised: one wave
// per row; writes q [rows][cols] e4m3 and scale [rows].  Same statistics as
// the bf16 LayerNorm kernels (fp32, biased variance, two passes).
// ---------------------------------------------------------------------------
template <bool GATED>
__global__ __launch_bounds__(256) void ln_quant_fp8_kernel(const uint16_t *x, int64_t ldx,
                                                           const uint16_t *u, int64_t ldu,
                                                           const float *w, const float *bias,
                                                           uint8_t *q, float *scale, int64_t rows,
                                                           int cols, float eps)
{
    constexpr int MAXC = 4;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int nchunk = cols / 8;
    float v[MAXC][8];
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nchunk) {
            bf16x8_to_f(ld16(x + row * ldx + 8 * ch), v[c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += v[c][e];
        }
    }
    const float mean = wave_sum_f(s) / (float)cols;
    float qs = 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
        if (lane + 64 * c < nchunk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = v[c][e] - mean;
                qs += d * d;
            }
    const float rstd = rsqrtf(wave_sum_f(qs) / (float)cols + eps);
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nchunk) {
            float uv[8];
            if (GATED) bf16x8_to_f(ld16(u + row * ldu + 8 * ch), uv);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int col = 8 * ch + e;
                float o = (v[c][e] - mean) * rstd * w[col] + (bias ? bias[col] : 0.0f);
                if (GATED) o *= uv[e];
                v[c][e] = o;
                a = fmaxf(a, fabsf(o));
            }
        }
    }
    a = wave_max_f(a);
    const float inv = a > 0.0f ? 448.0f / a : 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nchunk)
            *reinterpret_cast<uint2 *>(q + row * cols + 8 * ch) = to_e4m3x8(v[c], inv);
    }
    if (lane == 0) scale[row] = a > 0.0f ? a / 448.0f : 1.0f;
}

hipError_t launch_ln_quant_fp8(bool gated, const void *x, int64_t ldx, const void *u, int64_t ldu,
                               const float *w, const float *b, void *q, float *scale, int64_t rows,
                               int cols, float eps, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    if (cols % 8 != 0 || cols > 2048) return hipErrorInvalidValue;
    dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (gated)
        hipLaunchKernelGGL(ln_quant_fp8_kernel<true>, grid, block, 0, st, (const uint16_t *)x, ldx,
                           (const uint16_t *)u, ldu, w, b, (uint8_t *)q, scale, rows, cols, eps);
    else
        hipLaunchKernelGGL(ln_quant_fp8_kernel<false>, grid, block, 0, st, (const uint16_t *)x,
                           ldx, (const uint16_t *)u, ldu, w, b, (uint8_t *)q, scale, rows, cols,
                           eps);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// FP8 GEMM  C[M][N] = epi(sa[m] sw[n] sum_k A[m][k] W[n][k] + bias[n])
//   EPI 0: SiLU(.)          EPI 1: . + R[m][n] (the residual)
// A [M][K], W [N][K] e4m3 (row strides K bytes); sa [M], sw [N] fp32; C bf16.
// Workgroup tile 128 x 128, 4 waves in 2 x 2, K steps of 128; as the bf16
// kernel the waves compute C^T blocks so that each lane ends with four
// consecutive output columns of one row.  N % 128 == 0, K % 128 == 0.
// ---------------------------------------------------------------------------
constexpr int F8M = 128, F8N = 128, F8K = 128;

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_fp8_kernel(const uint8_t *A, const float *sa,
                                                          const uint8_t *W, const float *sw,
                                                          const float *bias, const uint16_t *R,
                                                          int64_t ldr, uint16_t *C, int64_t ldc,
                                                          int64_t M, int N, int K)
{
    __shared__ __align__(16) uint8_t la[2][F8M * F8K];
    __shared__ __align__(16) uint8_t lw[2][F8N * F8K];
    const int ntn = N / F8N;
    const int64_t ntm = (M + F8M - 1) / F8M;
    const int item = xcd_remap(blockIdx.x, (int)(ntm * ntn));
    if (item < 0) return;
    const int64_t m0 = (int64_t)(item / ntn) * F8M;
    const int n0 = (item % ntn) * F8N;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;
    const int wm = wv & 1, wn = wv >> 1;

    // staging: thread loads 16-byte chunk tid % 8 of rows tid / 8 + 32 i
    const int sr = tid >> 3, sc = tid & 7;
    uint4 ra[4], rw[4];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = m0 + sr + 32 * i;
            const int64_t rr = r < M ? r : M - 1;
            uint4 v = *reinterpret_cast<const uint4 *>(A + rr * K + k0 + 16 * sc);
            const bool ok = r < M;
            v.x = ok ? v.x : 0u;
            v.y = ok ? v.y : 0u;
            v.z = ok ? v.z : 0u;
            v.w = ok ? v.w : 0u;
            ra[i] = v;
            rw[i] = *reinterpret_cast<const uint4 *>(W + (int64_t)(n0 + sr + 32 * i) * K + k0 +
                                                     16 * sc);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = sr + 32 * i;
            *reinterpret_cast<uint4 *>(&la[buf][r * F8K + 16 * (sc ^ (r & 7))]) = ra[i];
            *reinterpret_cast<uint4 *>(&lw[buf][r * F8K + 16 * (sc ^ (r & 7))]) = rw[i];
        }
    };
    // operand of row r for the 64-deep slice kk: bytes 64 kk + 32 hl .. +32
    auto operand = [&](const uint8_t *tile, int r, int kk) {
        const int c = 4 * kk + 2 * hl;
        const uint4 lo = *reinterpret_cast<const uint4 *>(tile + r * F8K + 16 * (c ^ (r & 7)));
        const uint4 hi =
            *reinterpret_cast<const uint4 *>(tile + r * F8K + 16 * ((c + 1) ^ (r & 7)));
        intx8 v;
        v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
        v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
        return v;
    };

    floatx16 acc[2][2];  // [n block][m block] of C^T
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

    const int nk = K / F8K;
    load(0);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        store(buf);
        if (kt + 1 < nk) load((kt + 1) * F8K);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < F8K / 64; ++kk) {
            intx8 wa[2], xb[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) wa[nb] = operand(lw[buf], 64 * wn + 32 * nb + l32, kk);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) xb[mb] = operand(la[buf], 64 * wm + 32 * mb + l32, kk);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        wa[nb], xb[mb], acc[nb][mb], 0, 0, 0, 0, 0, 0);
        }
    }

    // epilogue: lane owns row m, registers hold columns n = 8*(r/4) + 4*hl + r%4
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int64_t m = m0 + 64 * wm + 32 * mb + l32;
        if (m >= M) continue;
        const float am = sa[m];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + 64 * wn + 32 * nb + 8 * g + 4 * hl;
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = acc[nb][mb][4 * g + e] * am * sw[n + e] + (bias ? bias[n + e] : 0.0f);
                if (EPI == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = o[e] * sigmoid_fast(o[e], -1.4426950408889634f);
                } else {
                    const uint2 rr = *reinterpret_cast<const uint2 *>(R + m * ldr + n);
                    o[0] += bf16_lo(rr.x);
                    o[1] += bf16_hi(rr.x);
                    o[2] += bf16_lo(rr.y);
                    o[3] += bf16_hi(rr.y);
                }
                *reinterpret_cast<uint2 *>(C + m * ldc + n) = cvt4_u2(o[0], o[1], o[2], o[3]);
            }
        }
    }
}

hipError_t launch_gemm_fp8(const void *A, const float *sa, const void *W, const float *sw,
                           const float *bias, const void *R, int64_t ldr, void *C, int64_t ldc,
                           int64_t M, int N, int K, int epi, hipStream_t st)
{
    if (M <= 0) return hipSuccess;
    if (N % F8N != 0 || K % F8K != 0 || (epi == 1 && !R) || epi < 0 || epi > 1)
        return hipErrorInvalidValue;
    const int64_t tiles = ((M + F8M - 1) / F8M) * (N / F8N);
    dim3 grid((unsigned)tiles), block(256);
    if (epi == 0)
        hipLaunchKernelGGL(gemm_fp8_kernel<0>, grid, block, 0, st, (const uint8_t *)A, sa,
                           (const uint8_t *)W, sw, bias, (const uint16_t *)R, ldr, (uint16_t *)C,
                           ldc, M, N, K);
    else
        hipLaunchKernelGGL(gemm_fp8_kernel<1>, grid, block, 0, st, (const uint8_t *)A, sa,
                           (const uint8_t *)W, sw, bias, (const uint16_t *)R, ldr, (uint16_t *)C,
                           ldc, M, N, K);
    return hipGetLastError();
}

}  // namespace sla
