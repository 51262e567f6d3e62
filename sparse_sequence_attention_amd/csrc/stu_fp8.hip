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
// GEMM (gemm_nt.hip): v_mfma_f32_32x32x64_f8f6f4 (fp8 x fp8, fp32
// accumulation).  Lane l holds operand row l % 32, bytes 32 * (l / 32) .. +32
// of the 64-deep slice; the accumulator layout is that of the bf16 32x32
// products.
#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {


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
// the bf16 LayerNorm kernels (fp32, biased variance, two passes).  Every
// load of the row (x, the gate u, weight and bias) is issued before the
// reductions; lane l holds the 16-byte chunks l, l + 64, ... (NCH of them).
// ---------------------------------------------------------------------------
template <bool GATED, int NCH>
__global__ __launch_bounds__(256) void ln_quant_fp8_kernel(const uint16_t *x, int64_t ldx,
                                                           const uint16_t *u, int64_t ldu,
                                                           const float *w, const float *bias,
                                                           uint8_t *q, float *scale, int64_t rows,
                                                           int cols, float eps)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int nchunk = cols / 8;
    uint4 xr[NCH], ur[NCH];
    float4 wv[NCH][2], bv[NCH][2];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nchunk) {
            xr[c] = ld16(x + row * ldx + 8 * ch);
            if (GATED) ur[c] = ld16(u + row * ldu + 8 * ch);
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
    float v[NCH][8];
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (lane + 64 * c < nchunk) {
            bf16x8_to_f(xr[c], v[c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += v[c][e];
        }
    }
    const float mean = wave_sum_f(s) / (float)cols;
    float qs = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if (lane + 64 * c < nchunk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = v[c][e] - mean;
                qs += d * d;
            }
    const float rstd = rsqrtf(wave_sum_f(qs) / (float)cols + eps);
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nchunk) {
            float uv[8];
            if (GATED) bf16x8_to_f(ur[c], uv);
            const float wf[8] = {wv[c][0].x, wv[c][0].y, wv[c][0].z, wv[c][0].w,
                                 wv[c][1].x, wv[c][1].y, wv[c][1].z, wv[c][1].w};
            const float bf[8] = {bv[c][0].x, bv[c][0].y, bv[c][0].z, bv[c][0].w,
                                 bv[c][1].x, bv[c][1].y, bv[c][1].z, bv[c][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float o = (v[c][e] - mean) * rstd * wf[e] + bf[e];
                if (GATED) o *= uv[e];
                v[c][e] = o;
                a = fmaxf(a, fabsf(o));
            }
        }
    }
    a = wave_max_f(a);
    const float inv = a > 0.0f ? 448.0f / a : 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
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
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, (const uint16_t *)x, ldx, (const uint16_t *)u,
                           ldu, w, b, (uint8_t *)q, scale, rows, cols, eps);
    };
    if (gated) {
        if (cols <= 512) go(ln_quant_fp8_kernel<true, 1>);
        else if (cols <= 1024) go(ln_quant_fp8_kernel<true, 2>);
        else go(ln_quant_fp8_kernel<true, 4>);
    } else {
        if (cols <= 512) go(ln_quant_fp8_kernel<false, 1>);
        else if (cols <= 1024) go(ln_quant_fp8_kernel<false, 2>);
        else go(ln_quant_fp8_kernel<false, 4>);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_fp8(const void *A, const float *sa, const void *W, const float *sw,
                           const float *bias, const void *R, int64_t ldr, void *C, int64_t ldc,
                           int64_t M, int N, int K, int epi, hipStream_t st)
{
    return launch_gemm_nt_fp8(A, sa, W, sw, bias, R, ldr, C, ldc, M, N, K, epi, st);
}

}  // namespace sla
