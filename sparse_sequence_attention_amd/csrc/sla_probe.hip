// sla_probe.hip -- measurement aids, not part of the attention path.
//
// MFMA-only throughput probe: the bf16 dense MFMA rate this GPU sustains at
// the shader clock it runs, so that measured kernel rates can be set against
// a peak measured on the same device as well as against the data-sheet
// figure.
//
// Every wave runs `iters` rounds of four independent chains of
// v_mfma_f32_32x32x16_bf16 (32,768 flops each; four chains cover the
// instruction's dependency latency); four waves per workgroup, four
// workgroups per CU.  Wave 0 of workgroup 0 reads the shader-clock counter
// (s_memtime) and the 100 MHz constant clock (s_memrealtime) at its start and
// end, which gives the shader clock during the run.
#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

constexpr int PROBE_CHAINS = 4;

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float *sink,
                                                        unsigned long long *clk)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    floatx16 acc[PROBE_CHAINS];
#pragma unroll
    for (int j = 0; j < PROBE_CHAINS; ++j) acc[j] = zero16();
    const bool stamp = blockIdx.x == 0 && threadIdx.x == 0;
    unsigned long long c0 = 0, r0 = 0;
    if (stamp) {
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < PROBE_CHAINS; ++j) acc[j] = mfma32(a, b, acc[j]);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < PROBE_CHAINS; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (stamp) {
        const unsigned long long c1 = __builtin_amdgcn_s_memtime();
        const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
        clk[0] = c1 - c0;
        clk[1] = r1 - r0;
    }
}

hipError_t launch_mfma_peak(int blocks, int iters, float *sink, unsigned long long *clk,
                            hipStream_t st)
{
    if (blocks <= 0 || iters <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink, clk);
    return hipGetLastError();
}

double mfma_peak_flops(int blocks, int iters)
{
    return (double)blocks * 4.0 * (double)iters * PROBE_CHAINS * 32.0 * 32.0 * 16.0 * 2.0;
}

// Issue-rate probe: how far one SIMD runs MFMA and VALU work concurrently,
// and the cost of the two transcendentals of the SiLU.  One workgroup of
// eight waves per CU (its 96 KB of LDS admit no second one), i.e. two waves
// per SIMD (waves w and w + 4 share a SIMD).  Per SIMD every MFMA mode issues
// 2 iters x 4 MFMAs (v_mfma_f32_32x32x16_bf16, four independent chains) and
// every VALU mode 2 iters x 32 v_fma_f32 (eight independent chains), in
// these arrangements:
//   ISSUE_MFMA    both waves MFMA only          ISSUE_VALU   both waves FMA only
//   ISSUE_SPLIT   wave w < 4 all the MFMAs, wave w + 4 all the FMAs
//   ISSUE_MIXED   both waves half of each, interleaved
//   ISSUE_SPLIT_A ISSUE_SPLIT with the accumulators in AGPRs
//   ISSUE_EXP / ISSUE_RCP  both waves 32 v_exp_f32 / v_rcp_f32 per round
// Perfect overlap makes SPLIT and MIXED as fast as the slower of MFMA and
// VALU; none makes them as slow as the two added.
__device__ __forceinline__ void probe_mfma_agpr(floatx16 &acc, const bf16x8 &a, const bf16x8 &b)
{
    // the compiler's hazard checks do not look inside inline assembly: the
    // asm waits the two states a VALU write of a source needs before an MFMA
    // reads it, and probe_agpr_settle the MFMA's write latency before the
    // accumulator is read
    asm("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ void probe_agpr_settle(floatx16 &acc)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc));
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void issue_probe_kernel(int iters, float y, float z, float *sink)
{
    __shared__ float pad[24 * 1024];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    floatx16 acc[PROBE_CHAINS];
#pragma unroll
    for (int j = 0; j < PROBE_CHAINS; ++j) acc[j] = zero16();
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.01f * (float)threadIdx.x + (float)i;
    constexpr bool AG = MODE == ISSUE_SPLIT_A;
    constexpr bool split = MODE == ISSUE_SPLIT || MODE == ISSUE_SPLIT_A;
    const bool do_m = MODE == ISSUE_MFMA || MODE == ISSUE_MIXED || (split && wv < 4);
    const bool do_v = MODE == ISSUE_VALU || MODE == ISSUE_MIXED || (split && wv >= 4);
    const int n = split ? 2 * iters : iters;
    auto mfmas = [&](int j) __attribute__((always_inline)) {
        if constexpr (AG) probe_mfma_agpr(acc[j], a, b);
        else acc[j] = mfma32(a, b, acc[j]);
    };
    auto fmas = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], y, z);
    };
    if constexpr (MODE == ISSUE_EXP || MODE == ISSUE_RCP) {
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    x[i] = MODE == ISSUE_EXP ? __builtin_amdgcn_exp2f(x[i]) : __builtin_amdgcn_rcpf(x[i]);
    } else if (do_m && do_v) {
        for (int it = 0; it < n; ++it) {
#pragma unroll
            for (int j = 0; j < PROBE_CHAINS; ++j) {
                mfmas(j);
                fmas();
            }
        }
    } else if (do_m) {
        for (int it = 0; it < n; ++it)
#pragma unroll
            for (int j = 0; j < PROBE_CHAINS; ++j) mfmas(j);
    } else if (do_v) {
        for (int it = 0; it < n; ++it)
#pragma unroll
            for (int k = 0; k < 4; ++k) fmas();
    }
    if constexpr (AG) {
#pragma unroll
        for (int j = 0; j < PROBE_CHAINS; ++j) probe_agpr_settle(acc[j]);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < PROBE_CHAINS; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += x[i];
    pad[threadIdx.x] = s;
    __syncthreads();
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = pad[511 - threadIdx.x];
}

hipError_t launch_issue_probe(int mode, int blocks, int iters, float *sink, hipStream_t st)
{
    if (blocks <= 0 || iters <= 0) return hipErrorInvalidValue;
    const dim3 g((unsigned)blocks), t(512);
    const float y = 0.999f, z = 0.001f;
    switch (mode) {
    case ISSUE_MFMA: hipLaunchKernelGGL(issue_probe_kernel<ISSUE_MFMA>, g, t, 0, st, iters, y, z, sink); break;
    case ISSUE_VALU: hipLaunchKernelGGL(issue_probe_kernel<ISSUE_VALU>, g, t, 0, st, iters, y, z, sink); break;
    case ISSUE_SPLIT: hipLaunchKernelGGL(issue_probe_kernel<ISSUE_SPLIT>, g, t, 0, st, iters, y, z, sink); break;
    case ISSUE_MIXED: hipLaunchKernelGGL(issue_probe_kernel<ISSUE_MIXED>, g, t, 0, st, iters, y, z, sink); break;
    case ISSUE_SPLIT_A: hipLaunchKernelGGL(issue_probe_kernel<ISSUE_SPLIT_A>, g, t, 0, st, iters, y, z, sink); break;
    case ISSUE_EXP: hipLaunchKernelGGL(issue_probe_kernel<ISSUE_EXP>, g, t, 0, st, iters, y, z, sink); break;
    case ISSUE_RCP: hipLaunchKernelGGL(issue_probe_kernel<ISSUE_RCP>, g, t, 0, st, iters, y, z, sink); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sla
