// sla_dq_ds.hip -- SLA backward dQ from the dS blocks the dK/dV kernel stored
// (bf16 path, d in {64, 128}): dQ = (alpha / (N G)) dS K over the visited key
// tiles, with dS and K already in fp16, so no S, dP or SiLU' recomputation.
// The chain rule and the notation are those of sla_bwd_bf16.hip (ULTRA-HSTU
// paper, section 3 Eq.3 under the semi-local mask of section 4.2.1 Eq.7).
#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

// ---------------------------------------------------------------------------
// dQ from the stored dS blocks: dQ_i = (alpha / (N G)) sum_j dS_ij k_j
// ---------------------------------------------------------------------------
// Work item: one 64-row tile of one head, 2*(D/32) waves.  It reads, in slot
// order, the dS block the dK/dV kernel stored for each key tile it visits and
// the fp16 copy of that key tile (no conversion: both are already fp16).
// Loads run two steps ahead in registers and are written to the other of two
// LDS stages after the current stage's products.  Wave w owns rows
// 32*(w%2) .. +32 and d-columns 32*(w/2) .. +32:
//   dQ^T (32 d x 32 rows) += K^T (32 d x 128 keys) . dS^T (128 keys x 32 rows)
// with both operands read by the transposing LDS read, the keys (contraction
// index) in natural order.
template <int D>
__device__ __forceinline__ int kh_swz(int key)  // chunk swizzle of the LDS K tile
{
    return (4 * (key & 3)) & (D / 8 - 1);
}

template <int D>
__global__ __launch_bounds__(64 * 2 * (D / 32), 1) void sla_bwd_dq_ds_kernel(AttnParams p)
{
    constexpr int NT = 64 * 2 * (D / 32);       // threads
    constexpr int CPR = D / 8;                  // 16-byte chunks per K row
    constexpr int KCH = DS_BN * CPR;            // chunks per K tile
    constexpr int SCH = DS_BM * DS_BN / 8;      // chunks per dS block
    constexpr int KPT = KCH / NT, SPT = SCH / NT, LPT = KPT + SPT;  // loads per thread and step
    static_assert(KCH % NT == 0 && SCH % NT == 0, "whole load rounds");
    __shared__ __align__(16) uint16_t lds[2][(KCH + SCH) * 8];

    const int nrec = uniform(p.s.rt_base[p.B]);
    const int item = xcd_remap(blockIdx.x, nrec * p.H);
    if (item < 0) return;
    const int h = item / nrec;
    const int rec = item - h * nrec;  // global 64-row tile index
    const int b = find_seq(p.s.rt_base, p.B, rec);
    const SeqDims sd = seq_dims(p.offsets, p.num_targets, b);
    int r0, r1;
    row_tile(sd.L, sd.U, DS_BM, rec - uniform(p.s.rt_base[b]), r0, r1);
    r0 = uniform(r0);
    r1 = uniform(r1);
    const Ranges kr = fwd_key_ranges(sd.L, sd.U, p.k1, p.k2e, r0, r1, DS_BN);
    const TileCursor cur(kr, DS_BN);
    const int ntiles = uniform(imin(cur.total, p.ds_slots));  // the slot count bounds cur.total

    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int rb = wv & 1, dbk = wv >> 1;
    const int64_t ldkh = (int64_t)p.H * D;
    const uint16_t *khg = p.kh + sd.base * ldkh + h * D;
    const uint16_t *dsg = p.ds + ((int64_t)rec * p.H + h) * ((int64_t)p.ds_slots * DS_BM * DS_BN);

    // loads of step t (clamped to the last tile past the end: L2 hits, so the
    // pipeline has no special cases).  K tile chunk P = key P / CPR, logical
    // chunk P % CPR (keys past L read key L - 1: their dS is zero); dS chunk
    // P as stored.
    auto load = [&](int t, uint4 (&r)[LPT]) {
        t = imin(t, ntiles - 1);
        const int c0 = cur.start(t, DS_BN);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int P = i * NT + tid;
            const int row = imin(c0 + P / CPR, sd.L - 1);
            r[i] = ld16(khg + (int64_t)row * ldkh + 8 * (P % CPR));
        }
        const uint16_t *blk = dsg + (int64_t)t * (DS_BM * DS_BN);
#pragma unroll
        for (int i = 0; i < SPT; ++i) r[KPT + i] = ld16(blk + 8 * (i * NT + tid));
    };
    // into LDS: K chunk (key, c) at physical chunk c ^ kh_swz(key)
    auto store = [&](const uint4 (&r)[LPT], uint16_t *sb) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int P = i * NT + tid;
            const int key = P / CPR;
            *reinterpret_cast<uint4 *>(sb + 8 * (key * CPR + ((P % CPR) ^ kh_swz<D>(key)))) = r[i];
        }
#pragma unroll
        for (int i = 0; i < SPT; ++i)
            *reinterpret_cast<uint4 *>(sb + 8 * (KCH + i * NT + tid)) = r[KPT + i];
    };

    // per-lane offsets (elements) of the transposing reads for k-chunk 0;
    // chunk kc adds a constant.  Quarter q = lane / 16 and role j = lane % 16:
    // read r covers keys 8*(q/2) + 4*r + j/4 of the chunk.
    const int q = lane >> 4, j = lane & 15;
    int ds_off[2], kh_off[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int k0 = 8 * (q >> 1) + 4 * r + (j >> 2);  // key within a 16-key chunk
        // dS^T operand: rows 32*rb + 16*(q%2) + 4*(j%4) .. +3 of key k0
        const int x4 = 8 * rb + 4 * (q & 1) + (j & 3);   // 4-row run index 0..15
        const int qc = 2 * (x4 >> 3) + ((x4 >> 2) & 1), half = (x4 >> 1) & 1, hl = x4 & 1;
        ds_off[r] = 8 * KCH + 8 * ds_frag_chunk(0, qc, k0, hl) + 4 * half;
        // K^T operand: d-columns 32*dbk + 16*(q%2) + 4*(j%4) .. +3 of key k0
        const int dcol = 32 * dbk + 16 * (q & 1) + 4 * (j & 3);
        kh_off[r] = k0 * D + 8 * ((dcol >> 3) ^ kh_swz<D>(k0)) + (dcol & 7);
    }

    floatx16 acc = zero16();
    auto compute = [&](const uint16_t *sb) {
#pragma unroll
        for (int kc = 0; kc < DS_BN / 16; ++kc) {
            // key 16*kc + k0 of the tile: chunk of dK/dV wave kc / 2, key 16*(kc % 2) + k0
            const int ds_kc = 8 * ds_frag_chunk(kc >> 1, 0, 16 * (kc & 1), 0);
            const uint2 b0 = tr_read_b64(sb + ds_off[0] + ds_kc);
            const uint2 b1 = tr_read_b64(sb + ds_off[1] + ds_kc);
            const uint2 a0 = tr_read_b64(sb + kh_off[0] + 16 * kc * D);
            const uint2 a1 = tr_read_b64(sb + kh_off[1] + 16 * kc * D);
            const halfx8 bfr = __builtin_bit_cast(halfx8, make_uint4(b0.x, b0.y, b1.x, b1.y));
            const halfx8 afr = __builtin_bit_cast(halfx8, make_uint4(a0.x, a0.y, a1.x, a1.y));
            acc = mfma32h(afr, bfr, acc);
        }
    };

    if (ntiles > 0) {
        uint4 ra[LPT], rbf[LPT];
        load(0, ra);
        store(ra, lds[0]);
        load(1, ra);
        load(2, rbf);
        __syncthreads();
        // even step t: stage 0 holds t, ra holds t + 1, rbf holds t + 2
        for (int t = 0; t < ntiles; t += 2) {
            compute(lds[0]);
            store(ra, lds[1]);      // waits for ra's loads only
            load(t + 3, ra);
            lds_barrier();
            if (t + 1 >= ntiles) break;
            compute(lds[1]);
            store(rbf, lds[0]);
            load(t + 4, rbf);
            lds_barrier();
        }
    }

    // register r of lane l: dQ^T[d = 32*dbk + 8*(r/4) + 4*(l/32) + r%4][row 32*rb + l%32]
    const int qi = r0 + 32 * rb + (lane & 31), hl = lane >> 5;
    if (qi < r1) {
        uint16_t *orow = reinterpret_cast<uint16_t *>(p.dq) + (sd.base + qi) * p.lddq + h * D;
        const float sc = p.out_scale / *p.grad_scale;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint2 v = cvt4_u2(acc[4 * g] * sc, acc[4 * g + 1] * sc, acc[4 * g + 2] * sc,
                              acc[4 * g + 3] * sc);
            *reinterpret_cast<uint2 *>(orow + 32 * dbk + 8 * g + 4 * hl) = v;
        }
    }
}

hipError_t launch_bwd_dq_ds_bf16(const AttnParams &p, hipStream_t st)
{
    dim3 grid(p.grid_rt);
    switch (p.d) {
    case 64: hipLaunchKernelGGL(sla_bwd_dq_ds_kernel<64>, grid, dim3(256), 0, st, p); break;
    case 128: hipLaunchKernelGGL(sla_bwd_dq_ds_kernel<128>, grid, dim3(512), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sla
