// sla_sched.hip -- on-device tile schedule of the SLA kernels.
//
// One workgroup turns the jagged offsets (and target counts) into per-sequence
// prefix sums of the work items each kernel runs; the attention kernels then
// locate their item without any host synchronisation (the WHALE notes'
// observation that syncing on runtime shapes costs milliseconds per call is the
// reason the schedule lives on the device).
#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

constexpr int SCHED_THREADS = 1024;

__global__ __launch_bounds__(SCHED_THREADS) void sla_sched_kernel(const int64_t *offsets,
                                                                  const int32_t *num_targets,
                                                                  int B, int k2e, Sched s,
                                                                  const float *absmax_part,
                                                                  float *grad_scale,
                                                                  uint4 *zero_block,
                                                                  const int64_t *cand_offsets)
{
    // the stored-dS zero block (DS_BM x DS_BN fp16 = 1024 x 16 bytes)
    if (zero_block != nullptr)
        for (int i = threadIdx.x; i < DS_BM * DS_BN / 8; i += SCHED_THREADS)
            zero_block[i] = make_uint4(0u, 0u, 0u, 0u);
    __shared__ int4 buf[2][SCHED_THREADS];
    __shared__ int buf2[2][SCHED_THREADS];
    __shared__ int4 carry;
    __shared__ int carry2;
    __shared__ float red[SCHED_THREADS / 64];
    const int tid = threadIdx.x;
    if (tid == 0) {
        carry = make_int4(0, 0, 0, 0);
        carry2 = 0;
    }
    if (absmax_part) {
        // gradient scale: the power of two that maps max|dO| into [1, 2)
        float m = 0.0f;
        for (int i = tid; i < ABSMAX_BLOCKS; i += SCHED_THREADS) m = fmaxf(m, absmax_part[i]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        if (tid == 0) {
            float mx = 0.0f;
            for (int i = 0; i < SCHED_THREADS / 64; ++i) mx = fmaxf(mx, red[i]);
            float sc = 1.0f;
            if (mx > 0.0f && mx < INFINITY) {
                int e = ilogbf(mx);
                e = e < -100 ? -100 : (e > 100 ? 100 : e);
                sc = ldexpf(1.0f, -e);
            }
            *grad_scale = sc;
        }
    }
    __syncthreads();
    for (int start = 0; start < B; start += SCHED_THREADS) {
        const int b = start + tid;
        int4 v = make_int4(0, 0, 0, 0);
        int v2 = 0;
        if (b < B && cand_offsets) {
            // candidate scoring: forward row tiles over the candidates only
            v.x = cdiv((int)(cand_offsets[b + 1] - cand_offsets[b]), FWD_BM);
            s.nch[b] = 1;
        } else if (b < B) {
            SeqDims sd = seq_dims<false>(offsets, num_targets, b);
            int np, nch;
            v.x = row_tiles(sd.L, sd.U, FWD_BM);
            v.y = bwd_items(sd.L, sd.U, k2e, BWD_BN, BWD_BM, np, nch);
            v.z = nch > 1 ? np : 0;
            v.w = nch > 1 ? np * nch : 0;
            v2 = row_tiles(sd.L, sd.U, DS_BM);
            s.nch[b] = nch;
        }
        // inclusive Hillis-Steele scan of the five counters
        int cur = 0;
        buf[cur][tid] = v;
        buf2[cur][tid] = v2;
        __syncthreads();
        for (int off = 1; off < SCHED_THREADS; off <<= 1) {
            int4 a = buf[cur][tid];
            int a2 = buf2[cur][tid];
            if (tid >= off) {
                int4 c = buf[cur][tid - off];
                a.x += c.x; a.y += c.y; a.z += c.z; a.w += c.w;
                a2 += buf2[cur][tid - off];
            }
            buf[cur ^ 1][tid] = a;
            buf2[cur ^ 1][tid] = a2;
            cur ^= 1;
            __syncthreads();
        }
        int4 inc = buf[cur][tid];
        int inc2 = buf2[cur][tid];
        int4 c0 = carry;
        int c02 = carry2;
        if (b < B) {
            s.fwd_base[b] = c0.x + inc.x - v.x;
            s.bwd_base[b] = c0.y + inc.y - v.y;
            s.red_base[b] = c0.z + inc.z - v.z;
            s.part_base[b] = c0.w + inc.w - v.w;
            s.rt_base[b] = c02 + inc2 - v2;
        }
        __syncthreads();
        if (tid == SCHED_THREADS - 1) {
            carry = make_int4(c0.x + inc.x, c0.y + inc.y, c0.z + inc.z, c0.w + inc.w);
            carry2 = c02 + inc2;
        }
        __syncthreads();
    }
    if (tid == 0) {
        int4 c = carry;
        s.fwd_base[B] = c.x;
        s.bwd_base[B] = c.y;
        s.red_base[B] = c.z;
        s.part_base[B] = c.w;
        s.rt_base[B] = carry2;
    }
}

hipError_t launch_sched(const AttnParams &p, hipStream_t st)
{
    hipLaunchKernelGGL(sla_sched_kernel, dim3(1), dim3(SCHED_THREADS), 0, st, p.offsets,
                       p.num_targets, p.B, p.k2e, p.s, (const float *)p.absmax_part,
                       p.grad_scale, reinterpret_cast<uint4 *>(p.ds), p.cand_offsets);
    return hipGetLastError();
}

// Per-block max |x| over the [T][H*d] rows (token stride ld) of a bf16 tensor;
// a fixed grid and a fixed reduction order, so the result is deterministic.
__global__ __launch_bounds__(256) void absmax_bf16_kernel(const uint16_t *x, int64_t ld,
                                                          int64_t rows, int cols, float *part)
{
    __shared__ float red[4];
    const int cpr = cols / 8;  // 16-byte chunks per row
    // the block covers `rpi` rows per pass, cpr threads per row (strided when
    // a row has more chunks than the block has threads)
    const int tpr = cpr < (int)blockDim.x ? cpr : (int)blockDim.x;
    const int rpi = blockDim.x / tpr;
    const int ro = threadIdx.x / tpr, ko = threadIdx.x % tpr;
    // four rows per iteration, their loads issued together (a max is
    // independent of the order)
    constexpr int U = 4;
    float m = 0.0f;
    if (ro < rpi) {
        const int64_t stride = (int64_t)gridDim.x * rpi;
        for (int64_t r = (int64_t)blockIdx.x * rpi + ro; r < rows; r += U * stride) {
            for (int k = ko; k < cpr; k += tpr) {
                uint4 v[U];
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    const int64_t rj = r + j * stride;
                    v[j] = rj < rows ? ld16(x + rj * ld + 8 * k) : make_uint4(0u, 0u, 0u, 0u);
                }
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
                }
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

hipError_t launch_absmax(const AttnParams &p, hipStream_t st)
{
    hipLaunchKernelGGL(absmax_bf16_kernel, dim3(ABSMAX_BLOCKS), dim3(256), 0, st,
                       (const uint16_t *)p.dout, p.lddo, p.T, p.H * p.d, p.absmax_part);
    return hipGetLastError();
}

// Checks of the device-resident preconditions of the jagged layout (the
// optional validation mode).  One workgroup; result[0] = the smallest failing
// code (0: none), result[1] = the first sequence it fails for.  Codes: 1
// offsets[0] != 0, 2 offsets decrease at b, 3 offsets[B] != T, 4 num_targets[b]
// outside [0, L_b], 5 contextual_len + num_targets[b] > L_b (ctx >= 0 only).
constexpr int VALIDATE_THREADS = 256;

__global__ __launch_bounds__(VALIDATE_THREADS) void sla_validate_kernel(
    const int64_t *offsets, const int32_t *num_targets, int B, int64_t T, int ctx, int32_t *result)
{
    __shared__ int64_t best[VALIDATE_THREADS];
    int64_t mine = INT64_MAX;  // (code << 32) | b of this thread's first failure
    auto note = [&](int code, int b) {
        const int64_t v = ((int64_t)code << 32) | (uint32_t)b;
        mine = v < mine ? v : mine;
    };
    if (threadIdx.x == 0) {
        if (offsets[0] != 0) note(1, 0);
        if (offsets[B] != T) note(3, B);
    }
    for (int b = threadIdx.x; b < B; b += VALIDATE_THREADS) {
        const int64_t L = offsets[b + 1] - offsets[b];
        if (L < 0) note(2, b);
        if (num_targets) {
            const int64_t nt = num_targets[b];
            if (nt < 0 || nt > L) note(4, b);
            else if (ctx >= 0 && nt < L && ctx + nt > L) note(5, b);
        }
    }
    best[threadIdx.x] = mine;
    __syncthreads();
    for (int o = VALIDATE_THREADS / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) {
            const int64_t a = best[threadIdx.x], c = best[threadIdx.x + o];
            best[threadIdx.x] = a < c ? a : c;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const int64_t v = best[0];
        result[0] = v == INT64_MAX ? 0 : (int32_t)(v >> 32);
        result[1] = v == INT64_MAX ? -1 : (int32_t)(v & 0xffffffff);
    }
}

hipError_t launch_validate(const int64_t *offsets, const int32_t *num_targets, int B, int64_t T,
                           int ctx, int32_t *result, hipStream_t st)
{
    hipLaunchKernelGGL(sla_validate_kernel, dim3(1), dim3(VALIDATE_THREADS), 0, st, offsets,
                       num_targets, B, T, ctx, result);
    return hipGetLastError();
}

// Materialise the work list (one thread per record) so that it can be checked.
__global__ void sla_sched_dump_kernel(const int64_t *offsets, const int32_t *num_targets, int B,
                                      int k1, int k2e, Sched s, int op, int32_t *records,
                                      int64_t capacity, int32_t *count)
{
    const int32_t *base = op == 0 ? s.fwd_base : (op == 1 ? s.bwd_base : s.rt_base);
    const int total = base[B];
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r == 0) *count = total;
    if (r >= total || r >= capacity) return;
    const int b = find_seq<false>(base, B, (int)r);
    const SeqDims sd = seq_dims<false>(offsets, num_targets, b);
    const int li = (int)r - base[b];
    int32_t rec[12];
    fill_record(op, b, sd.L, sd.U, k1, k2e, li, rec);
    for (int i = 0; i < 12; ++i) records[r * 12 + i] = rec[i];
}

hipError_t launch_sched_dump(const AttnParams &p, int op, int32_t *records, int64_t capacity,
                             int32_t *count, hipStream_t st)
{
    int64_t n = capacity > 0 ? capacity : 1;
    int blocks = (int)((n + 255) / 256);
    hipLaunchKernelGGL(sla_sched_dump_kernel, dim3(blocks), dim3(256), 0, st, p.offsets,
                       p.num_targets, p.B, p.k1, p.k2e, p.s, op, records, capacity, count);
    return hipGetLastError();
}

}  // namespace sla
