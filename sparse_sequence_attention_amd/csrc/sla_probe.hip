// sla_probe.hip -- MFMA-only throughput probe: the bf16 dense MFMA rate this
// GPU sustains at the shader clock it runs, so that measured kernel rates can
// be set against a peak measured on the same device as well as against the
// data-sheet figure.
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

}  // namespace sla
