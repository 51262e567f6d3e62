// sla_dq_ds.hip -- SLA backward dQ from the dS blocks the dK/dV kernel stored
// (bf16 path, d in {64, 128}): dQ = (alpha / (N G)) dS K over the visited key
// tiles, with dS and K already in fp16, so no S, dP or SiLU' recomputation.
// The chain rule and the notation are those of sla_bwd_bf16.hip (ULTRA-HSTU
// paper, section 3 Eq.3 under the semi-local mask of section 4.2.1 Eq.7).
#include <type_traits>

#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

// ---------------------------------------------------------------------------
// dQ from the stored dS blocks: dQ_i = (alpha / (N G)) sum_j dS_ij k_j
// ---------------------------------------------------------------------------
// Work item: one 128-row tile of one head (the forward's row tiles: its two
// 64-row halves are the dS block rows), 8 waves, two workgroups per CU.  Step
// t covers half t%2 (64 keys) of the (t/2)-th key tile of the 128-row tile
// (the union of the halves' key tiles): the fp16 K rows and each half's
// stored dS for those keys.  A half that does not visit that key tile reads
// the zero block instead, and so do steps past the end, so every step does
// the same work.  The data is copied HBM -> LDS by the DMA path one step
// ahead into the other of two stages; with at most eight DMA loads per
// thread and stage the compiler keeps exact wait counts.
// Wave w owns rows 32*(w%4) .. +32 and d-columns (D/2)*(w/4) .. +D/2:
//   dQ^T (d x 32 rows) += K^T (d x 64 keys) . dS^T (64 keys x 32 rows)
// with both operands read by the transposing LDS read, keys (the
// contraction index) in natural order.
template <int D>
__device__ __forceinline__ int kh_swz(int key)  // chunk swizzle of the LDS K tile
{
    return (4 * (key & 3)) & (D / 8 - 1);
}

template <int N>
using stage_t = std::integral_constant<int, N>;

constexpr int DQ_THREADS = 512;
constexpr int DQ_KEYS = DS_BN / 2;  // keys per step

template <int D>
__global__ __launch_bounds__(DQ_THREADS, 2) void sla_bwd_dq_ds_kernel(AttnParams p)
{
    constexpr int NT = DQ_THREADS;
    constexpr int CPR = D / 8;                  // 16-byte chunks per K row
    constexpr int KCH = DQ_KEYS * CPR;          // chunks of K per step
    constexpr int HCH = DS_BM * DQ_KEYS / 8;    // chunks of one half block (64 rows x 64 keys)
    constexpr int SCH = 2 * HCH;                // both row halves
    constexpr int KPT = KCH / NT, SPT = SCH / NT;  // DMA loads per thread and step
    constexpr int NDBW = D / 64;                // 32-wide d blocks per wave
    static_assert(KCH % NT == 0 && SCH % NT == 0, "whole DMA rounds");
    static_assert(KPT + SPT <= 8, "at most 8 DMA loads per thread and stage");
    // one array per stage: K rows, then the two halves' dS
    __shared__ __align__(16) uint16_t st0[(KCH + SCH) * 8], st1[(KCH + SCH) * 8];
    // per step: key tile start and the two halves' dS block indices, computed
    // once per item (each half visits at most DS_MAX_SLOTS key tiles, so a
    // 128-row tile has at most 2 * 2 * DS_MAX_SLOTS steps)
    constexpr int DQ_TAB = 4 * DS_MAX_SLOTS;
    __shared__ int4 steptab[DQ_TAB];

    const int nrec = uniform(p.s.fwd_base[p.B]);
    const int item = xcd_remap(blockIdx.x, nrec * p.H);
    if (item < 0) return;
    const int h = item / nrec;
    const int rec = item - h * nrec;
    const int b = find_seq(p.s.fwd_base, p.B, rec);
    const SeqDims sd = seq_dims(p.offsets, p.num_targets, b);
    int r0, r1;
    row_tile(sd.L, sd.U, FWD_BM, rec - uniform(p.s.fwd_base[b]), r0, r1);
    r0 = uniform(r0);
    r1 = uniform(r1);
    const int rh = imin(r0 + DS_BM, r1);  // first row of the second half
    const Ranges kr = fwd_key_ranges(sd.L, sd.U, p.k1, p.k2e, r0, r1, DS_BN);
    const Ranges kr0 = fwd_key_ranges(sd.L, sd.U, p.k1, p.k2e, r0, rh, DS_BN);
    const Ranges kr1 = fwd_key_ranges(sd.L, sd.U, p.k1, p.k2e, rh, r1, DS_BN);  // empty if rh == r1
    const TileCursor cur(kr, DS_BN);
    const int ntiles = uniform(cur.total);
    const int nsteps = 2 * ntiles;
    // 64-row tile index of the first half (history halves from 0, targets from U)
    const int rt0 = uniform(p.s.rt_base[b]) +
                    (r0 < sd.U ? r0 / DS_BM : cdiv(sd.U, DS_BM) + (r0 - sd.U) / DS_BM);

    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int rb = wv & 3, dh = wv >> 2;
    const int64_t ldkh = (int64_t)p.H * D;
    const uint16_t *khg = p.kh + sd.base * ldkh + h * D;
    constexpr int64_t BLK = DS_BM * DS_BN;
    // block index (0 = the zero block) of half `half` for the key tile at c0
    // (arithmetic rather than selects: branches here would cost the compiler
    // its exact DMA wait counts)
    auto block_of = [&](int half, const Ranges &krh, int c0, bool live) -> int64_t {
        const bool in0 = (c0 >= krh.lo0) & (c0 < krh.hi0);
        const bool in1 = (c0 >= krh.lo1) & (c0 < krh.hi1);
        const bool in2 = (c0 >= krh.lo2) & (c0 < krh.hi2);
        const int n0 = (krh.hi0 - krh.lo0 + DS_BN - 1) / DS_BN;
        const int n01 = n0 + (krh.hi1 - krh.lo1 + DS_BN - 1) / DS_BN;
        const int i0 = in0, i1 = !in0 & in1, i2 = !in0 & !in1 & in2;
        const int slot = i0 * ((c0 - krh.lo0) / DS_BN) + i1 * (n0 + (c0 - krh.lo1) / DS_BN) +
                         i2 * (n01 + (c0 - krh.lo2) / DS_BN);
        const int ok = (int)live & (i0 | i1 | i2) & (slot < p.ds_slots);
        return (int64_t)ok * (1 + ((int64_t)(rt0 + half) * p.H + h) * p.ds_slots + slot);
    };

    auto kst = [&](auto S) -> uint16_t * {
        if constexpr (decltype(S)::value == 0) return st0;
        else return st1;
    };
    auto dst = [&](auto S) -> uint16_t * { return kst(S) + KCH * 8; };

    for (int t = tid; t < imin(nsteps, DQ_TAB); t += NT) {
        const int c0 = cur.start(t >> 1, DS_BN);
        steptab[t] = make_int4(c0, (int)block_of(0, kr0, c0, true), (int)block_of(1, kr1, c0, true), 0);
    }
    __syncthreads();

    // DMA of step t (t >= nsteps: the last keys again, with zero dS): K row
    // chunk P (key P / CPR of the step, physical chunk P % CPR) holds logical
    // chunk (P % CPR) ^ kh_swz(key), keys past L read key L - 1 (their dS is
    // zero); dS chunks 0..HCH-1 from half 0's block, HCH.. from half 1's, each
    // the key half t%2 of the stored block (the dK/dV kernel stores its waves'
    // 32-key fragments one after another, so a key half is contiguous).  The
    // K rows are a workgroup-uniform base plus a 32-bit lane offset.
    const uint32_t ldkh_b = (uint32_t)ldkh * 2u;
    auto issue = [&](int t, auto S) {
        const int tt = imin(imin(t, nsteps - 1), DQ_TAB - 1);
        const int4 e = steptab[tt];
        const int kh = tt & 1;
        const int live = t < nsteps;
        // rows kbase + key, clamped to L - 1, as base kb0 = min(kbase, L - 1)
        // plus a lane offset in [0, L - 1 - kb0] (kbase may lie past the end
        // of the sequence for the second half of its last key tile)
        const int kbase = uniform(e.x) + DQ_KEYS * kh;
        const int kb0 = imin(kbase, sd.L - 1);
        const int last = sd.L - 1 - kb0, skip = kbase - kb0;
        const uint16_t *b0 = p.ds + BLK * (int64_t)(live * uniform(e.y)) + 8 * HCH * kh;
        const uint16_t *b1 = p.ds + BLK * (int64_t)(live * uniform(e.z)) + 8 * HCH * kh;
        const char *krow = reinterpret_cast<const char *>(khg + (int64_t)kb0 * ldkh);
        uint16_t *ks = kst(S), *ds = dst(S);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int P = i * NT + wv * 64 + lane;
            const int key = P / CPR;
            const uint32_t c = (uint32_t)((P % CPR) ^ kh_swz<D>(key));
            const uint32_t row = (uint32_t)imin(key + skip, last);
            gl_lds16(krow + (row * ldkh_b + 16u * c), ks + (i * NT + wv * 64) * 8);
        }
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int P = i * NT + wv * 64 + lane;  // uniform half per DMA round
            const uint16_t *src = (i * NT < HCH) ? b0 + 8 * P : b1 + 8 * (P - HCH);
            gl_lds16_nt(src, ds + (i * NT + wv * 64) * 8);  // each dS block is read once
        }
    };

    // per-lane offsets (elements) of the transposing reads for k-chunk 0;
    // chunk kc adds a constant.  Quarter q = lane / 16 and role j = lane % 16:
    // read r covers keys 8*(q/2) + 4*r + j/4 of the chunk.
    const int q = lane >> 4, j = lane & 15;
    int ds_off[2], kh_off[2][NDBW];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int k0 = 8 * (q >> 1) + 4 * r + (j >> 2);  // key within a 16-key chunk
        // dS^T operand: rows 32*(rb%2) + 16*(q%2) + 4*(j%4) .. +3 of key k0 in
        // the half block of row half rb / 2
        const int x4 = 8 * (rb & 1) + 4 * (q & 1) + (j & 3);  // 4-row run index 0..15
        const int qc = 2 * (x4 >> 3) + ((x4 >> 2) & 1), half = (x4 >> 1) & 1, hl = x4 & 1;
        ds_off[r] = 8 * ((rb >> 1) * HCH + ds_frag_chunk(0, qc, k0, hl)) + 4 * half;
        // K^T operand: d-columns 32*db' + 16*(q%2) + 4*(j%4) .. +3 of key k0
#pragma unroll
        for (int db = 0; db < NDBW; ++db) {
            const int dcol = 32 * (dh * NDBW + db) + 16 * (q & 1) + 4 * (j & 3);
            kh_off[r][db] = k0 * D + 8 * ((dcol >> 3) ^ kh_swz<D>(k0)) + (dcol & 7);
        }
    }

    floatx16 acc[NDBW];
#pragma unroll
    for (int i = 0; i < NDBW; ++i) acc[i] = zero16();

    // step t: wait for its DMA, publish it (the barrier also frees the other
    // stage, read by step t - 1), refill the other stage with step t + 1, then
    // the products
    auto step = [&](int t, auto S) {
        constexpr int s = decltype(S)::value;
        vm_wait<0>();
        barrier_lds_dma();
        issue(t + 1, stage_t<1 - s>{});
        __builtin_amdgcn_sched_barrier(0);  // keep the refill ahead of this step's reads
        const uint16_t *ks = kst(S), *dss = dst(S);
#pragma unroll
        for (int kc = 0; kc < DQ_KEYS / 16; ++kc) {
            // key 16*kc + k0 of the step: 32-key fragment kc / 2, key 16*(kc % 2) + k0
            const int ds_kc = 8 * ds_frag_chunk(kc >> 1, 0, 16 * (kc & 1), 0);
            const uint2 b0 = tr_read_b64(dss + ds_off[0] + ds_kc);
            const uint2 b1 = tr_read_b64(dss + ds_off[1] + ds_kc);
            const halfx8 bfr = __builtin_bit_cast(halfx8, make_uint4(b0.x, b0.y, b1.x, b1.y));
#pragma unroll
            for (int db = 0; db < NDBW; ++db) {
                const uint2 a0 = tr_read_b64(ks + kh_off[0][db] + 16 * kc * D);
                const uint2 a1 = tr_read_b64(ks + kh_off[1][db] + 16 * kc * D);
                const halfx8 afr = __builtin_bit_cast(halfx8, make_uint4(a0.x, a0.y, a1.x, a1.y));
                acc[db] = mfma32h(afr, bfr, acc[db]);
            }
        }
    };

    if (nsteps > 0) {
        issue(0, stage_t<0>{});
        for (int t = 0; t < nsteps; t += 2) {
            step(t, stage_t<0>{});
            step(t + 1, stage_t<1>{});
        }
        vm_wait<0>();  // no DMA left in flight at exit
    }

    // acc[db] register r of lane l: dQ^T[d = 32*db' + 8*(r/4) + 4*(l/32) + r%4][row 32*rb + l%32]
    const int qi = r0 + 32 * rb + (lane & 31), hl = lane >> 5;
    if (qi < r1) {
        uint16_t *orow = reinterpret_cast<uint16_t *>(p.dq) + (sd.base + qi) * p.lddq + h * D;
        const float sc = p.out_scale / *p.grad_scale;
#pragma unroll
        for (int db = 0; db < NDBW; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 v = cvt4_u2(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc,
                                  acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc);
                *reinterpret_cast<uint2 *>(orow + 32 * (dh * NDBW + db) + 8 * g + 4 * hl) = v;
            }
        }
    }
}

hipError_t launch_bwd_dq_ds_bf16(const AttnParams &p, hipStream_t st)
{
    dim3 grid(p.grid_fwd), block(DQ_THREADS);
    switch (p.d) {
    case 64: hipLaunchKernelGGL(sla_bwd_dq_ds_kernel<64>, grid, block, 0, st, p); break;
    case 128: hipLaunchKernelGGL(sla_bwd_dq_ds_kernel<128>, grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sla
