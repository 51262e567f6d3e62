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

// Exclusive prefix sums of v over the workgroup's threads, continued from
// *carry (LDS, updated to include this round).  Every thread calls it.
__device__ inline int block_exclusive_scan(int v, int (*buf)[SCHED_THREADS], int *carry)
{
    const int tid = threadIdx.x;
    int cur = 0;
    buf[cur][tid] = v;
    __syncthreads();
    for (int off = 1; off < SCHED_THREADS; off <<= 1) {
        int a = buf[cur][tid];
        if (tid >= off) a += buf[cur][tid - off];
        buf[cur ^ 1][tid] = a;
        cur ^= 1;
        __syncthreads();
    }
    const int inc = buf[cur][tid];
    const int c = *carry;
    __syncthreads();
    if (tid == SCHED_THREADS - 1) *carry = c + inc;
    __syncthreads();
    return c + inc - v;
}

__global__ __launch_bounds__(SCHED_THREADS) void sla_sched_kernel(const int64_t *offsets,
                                                                  const int32_t *num_targets,
                                                                  int B, int k1, int k2e, Sched s,
                                                                  const int64_t *cand_offsets)
{
    __shared__ int4 buf[2][SCHED_THREADS];
    __shared__ int4 carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = make_int4(0, 0, 0, 0);
    __syncthreads();
    for (int start = 0; start < B; start += SCHED_THREADS) {
        const int b = start + tid;
        int4 v = make_int4(0, 0, 0, 0);
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
            s.nch[b] = nch;
        }
        // inclusive Hillis-Steele scan of the four counters
        int cur = 0;
        buf[cur][tid] = v;
        __syncthreads();
        for (int off = 1; off < SCHED_THREADS; off <<= 1) {
            int4 a = buf[cur][tid];
            if (tid >= off) {
                int4 c = buf[cur][tid - off];
                a.x += c.x; a.y += c.y; a.z += c.z; a.w += c.w;
            }
            buf[cur ^ 1][tid] = a;
            cur ^= 1;
            __syncthreads();
        }
        int4 inc = buf[cur][tid];
        int4 c0 = carry;
        if (b < B) {
            s.fwd_base[b] = c0.x + inc.x - v.x;
            s.bwd_base[b] = c0.y + inc.y - v.y;
            s.red_base[b] = c0.z + inc.z - v.z;
            s.part_base[b] = c0.w + inc.w - v.w;
        }
        __syncthreads();
        if (tid == SCHED_THREADS - 1)
            carry = make_int4(c0.x + inc.x, c0.y + inc.y, c0.z + inc.z, c0.w + inc.w);
        __syncthreads();
    }
    if (tid == 0) {
        int4 c = carry;
        s.fwd_base[B] = c.x;
        s.bwd_base[B] = c.y;
        s.red_base[B] = c.z;
        s.part_base[B] = c.w;
    }
    if (!s.ds_base || cand_offsets) return;

    // Stored-dS backward: key tiles per sequence, then the dS blocks of every
    // key tile (its 64-row steps, all chunks together), as prefix sums.
    __shared__ int ibuf[2][SCHED_THREADS];
    __shared__ int icarry;
    if (tid == 0) icarry = 0;
    __syncthreads();
    for (int start = 0; start < B; start += SCHED_THREADS) {
        const int b = start + tid;
        int v = 0;
        if (b < B) v = cdiv((int)(offsets[b + 1] - offsets[b]), BWD_BN);
        const int e = block_exclusive_scan(v, ibuf, &icarry);
        if (b < B) s.ktile_base[b] = e;
    }
    const int ntiles = icarry;
    __syncthreads();  // every thread has read icarry before it is reset
    if (tid == 0) {
        s.ktile_base[B] = ntiles;
        icarry = 0;
    }
    __syncthreads();  // ktile_base (global, this workgroup's writes) is read below
    for (int start = 0; start < ntiles; start += SCHED_THREADS) {
        const int g = start + tid;
        int v = 0;
        if (g < ntiles) {
            const int b = find_seq<false>(s.ktile_base, B, g);
            const SeqDims sd = seq_dims<false>(offsets, num_targets, b);
            const int c0 = (g - s.ktile_base[b]) * BWD_BN;
            const TileSteps ts = tile_steps(sd.L, sd.U, k1, k2e, c0, imin(c0 + BWD_BN, sd.L), BWD_BM);
            v = ts.nh + ts.nt;
        }
        const int e = block_exclusive_scan(v, ibuf, &icarry);
        if (g < ntiles) s.ds_base[g] = e;
    }
    if (tid == 0) s.ds_base[ntiles] = icarry;
}

hipError_t launch_sched(const AttnParams &p, hipStream_t st)
{
    hipLaunchKernelGGL(sla_sched_kernel, dim3(1), dim3(SCHED_THREADS), 0, st, p.offsets,
                       p.num_targets, p.B, p.k1, p.k2e, p.s, p.cand_offsets);
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
    const int32_t *base = op == 0 ? s.fwd_base : s.bwd_base;
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
