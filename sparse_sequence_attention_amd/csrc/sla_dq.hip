// sla_dq.hip -- SLA backward dQ on gfx950: bf16 MFMA, fp32 accumulation, no
// atomics (the row tile owns its dQ rows).
//
// With a_ij = SiLU(alpha s_ij), s_ij = q_i . k_j and O_i = (1/N) sum_j a_ij v_j
// (ULTRA-HSTU paper, section 3 Eq.3 under the semi-local mask of section
// 4.2.1 Eq.7), the chain rule gives over the visible pairs of row i
//   g_ij  = dO_i . v_j
//   dS_ij = (alpha / N) g_ij sigma_ij (1 + t_ij (1 - sigma_ij)),  t = alpha s
//   dQ_i  = sum_j dS_ij k_j.
// Two kernels.  The first recomputes s and g for its row tile: the path of a
// workspace without room for dS.  The second (further down) reads the bf16
// dS that the key-tile (dK/dV) kernel stored: 2 bytes per pair written and
// read back through HBM (about a gigabyte at 16K-token histories) in place
// of two products and the SiLU' arithmetic per pair.
//
// Work item: one row tile of up to 128 rows (4 waves x 32) of one head, two
// workgroups per CU, over the same key tiles as the forward (prefix, band, and
// for target rows the window of the first target slot plus the diagonal), 64
// keys per step.  Per 32-key block each wave computes
//   S^T  (32 keys x 32 rows) = K Q^T          K rows from LDS, Q^T in registers
//   dP^T (32 keys x 32 rows) = V dO^T         V rows from LDS, dO^T in registers
//   dS^T = mask(dP^T * sigma (1 + t (1 - sigma)))   in registers, rounded to bf16
//   dQ^T (D x 32 rows)     += K^T dS^T        K^T by transposing LDS reads
// Computing S and dP transposed puts the rows in the lane dimension, so dS^T
// feeds the third product as its B operand straight from the accumulator.
// The K and V rows of the next step come HBM -> LDS by DMA into the idle one
// of two stages (the forward's swizzled layout); one LDS-only barrier per
// step keeps that DMA in flight across it.
#include <type_traits>

#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

// 16-byte chunk swizzle of the [64][D] K and V stage tiles (as the forward):
// logical chunk c of row r sits at c ^ qswz<D>(r), u = r*D/128 (the 256-byte
// bank row), Q4 = D/32.
template <int D>
__device__ __forceinline__ int qswz(int r)
{
    constexpr int Q4 = D / 32;
    const int u = r * D / 128;
    return 4 * (u % Q4) + (u / Q4) % 4;
}

// DQK: the Q / K (and dQ) head width, DV: the V and dO width.
template <int DQK, int DV, bool OUTF32>
__global__ __launch_bounds__(256, 2) void sla_bwd_dq_kernel(AttnParams p)
{
    constexpr int BM = FWD_BM, BN = FWD_BN;
    constexpr int NT = 256;
    constexpr int NC = DQK / 16, NCV = DV / 16;  // 16-wide contraction chunks of Q.K, dO.V
    constexpr int NDB = DQK / 32;                // 32-wide output blocks
    constexpr int CPR = DQK / 8, CPRV = DV / 8;     // 16-byte chunks per K / V row
    constexpr int TCH = BN * CPR, TCHV = BN * CPRV;  // chunks of one 64-key K / V tile
    constexpr int KPT = TCH / NT, KPTV = TCHV / NT;  // DMA loads per thread and tile
    static_assert(BN == 64 && BM == 128, "64-key steps over 128-row tiles");
    static_assert(TCH % NT == 0 && TCHV % NT == 0 && KPT + KPTV <= 8,
                  "whole DMA rounds, at most 8 per stage");
    __shared__ __align__(16) uint16_t st0[BN * (DQK + DV)], st1[BN * (DQK + DV)];

    const int nrec = p.s.fwd_base[p.B];
    const int item = xcd_remap(blockIdx.x, nrec * p.H);
    if (item < 0) return;
    const int h = item / nrec;
    const int rec = item - h * nrec;
    const int b = find_seq(p.s.fwd_base, p.B, rec);
    const SeqDims sd = seq_dims(p.offsets, p.num_targets, b);
    int r0, r1;
    row_tile(sd.L, sd.U, BM, rec - uniform(p.s.fwd_base[b]), r0, r1);
    r0 = uniform(r0);
    r1 = uniform(r1);
    const Ranges kr = fwd_key_ranges(sd.L, sd.U, p.k1, p.k2e, r0, r1, BN);

    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int l32 = lane & 31, hl = lane >> 5;

    const uint16_t *qg = reinterpret_cast<const uint16_t *>(p.q) + sd.base * p.ldq + h * DQK;
    const uint16_t *kg = reinterpret_cast<const uint16_t *>(p.k) + sd.base * p.ldk + h * DQK;
    const uint16_t *vg = reinterpret_cast<const uint16_t *>(p.v) + sd.base * p.ldv + h * DV;
    const uint16_t *gg = reinterpret_cast<const uint16_t *>(p.dout) + sd.base * p.lddo + h * DV;

    // Q^T and dO^T operands: lane holds row qi, d-slots 16c + 8*hl .. +8; rows
    // at or past r1 read as zero (then g = 0 and dS = 0)
    const int qi = r0 + 32 * wv + l32;
    bf16x8 qb[NC], gb[NCV];
#pragma unroll
    for (int c = 0; c < (NC > NCV ? NC : NCV); ++c) {
        if (c < NC) qb[c] = as_bf16x8(ld16_row(qg, p.ldq, qi, r1, 16 * c + 8 * hl));
        if (c < NCV) gb[c] = as_bf16x8(ld16_row(gg, p.lddo, qi, r1, 16 * c + 8 * hl));
    }

    const TileCursor cur(kr, BN);
    const int ntiles = uniform(cur.total);

    floatx16 dqacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dqacc[i] = zero16();

    auto stage = [&](auto S) -> uint16_t * {
        if constexpr (decltype(S)::value == 0) return st0;
        else return st1;
    };
    // DMA of the K and V rows of key tile t into a stage ([K | V], the V rows
    // after the BN * DQK elements of K): chunk P = i*NT + tid of a tile is
    // physical chunk P % CPR of key row P / CPR and holds its logical chunk
    // (P % CPR) ^ qswz(row) (CPR, qswz of the tile's own width); keys at or
    // past L read key L - 1 (such tiles are never "full", and the mask
    // removes them)
    const uint32_t ldk_b = (uint32_t)p.ldk * 2u, ldv_b = (uint32_t)p.ldv * 2u;
    auto issue = [&](int t, auto S) {
        const int c0 = uniform(cur.start(t, BN));
        const int last = uniform(sd.L - 1 - c0);
        const char *krow = reinterpret_cast<const char *>(kg + (int64_t)c0 * p.ldk);
        const char *vrow = reinterpret_cast<const char *>(vg + (int64_t)c0 * p.ldv);
        uint16_t *sb = stage(S);
#pragma unroll
        for (int i = 0; i < (KPT > KPTV ? KPT : KPTV); ++i) {
            const int P = i * NT + tid;
            if (i < KPT) {
                const int prow = P / CPR;
                const uint32_t row = (uint32_t)imin(prow, last);
                const uint32_t c = (uint32_t)((P % CPR) ^ qswz<DQK>(prow));
                gl_lds16(krow + (row * ldk_b + 16u * c), sb + (i * NT + wv * 64) * 8);
            }
            if (i < KPTV) {
                const int prow = P / CPRV;
                const uint32_t row = (uint32_t)imin(prow, last);
                const uint32_t c = (uint32_t)((P % CPRV) ^ qswz<DV>(prow));
                gl_lds16(vrow + (row * ldv_b + 16u * c), sb + (BN * DQK + (i * NT + wv * 64) * 8));
            }
        }
    };

    // per-lane LDS offsets (elements).  Row operands: key row 32*kb + l32,
    // logical chunk 2c + hl.  K^T operand by transposing reads (quarter
    // q = lane/16, j = lane%16): keys 32*kb + 16*h2 + 8*rr + 4*(q/2) + j/4,
    // d-columns 32*db + 16*(q%2) + 4*(j%4); the keys come in the order in
    // which the S^T accumulator hands them to dS^T (8*(r/4) + 4*hl + r%4).
    const int q4 = lane >> 4, j16 = lane & 15;
    auto r_off = [&](int kb, int c) {  // K rows
        const int r = 32 * kb + l32;
        return r * DQK + 8 * ((2 * c + hl) ^ qswz<DQK>(r));
    };
    auto rv_off = [&](int kb, int c) {  // V rows
        const int r = 32 * kb + l32;
        return r * DV + 8 * ((2 * c + hl) ^ qswz<DV>(r));
    };
    auto t_off = [&](int kb, int h2, int rr, int db) {
        const int row = 32 * kb + 16 * h2 + 8 * rr + 4 * (q4 >> 1) + (j16 >> 2);
        const int col = 32 * db + 16 * (q4 & 1) + 4 * (j16 & 3);
        return row * DQK + 8 * ((col >> 3) ^ qswz<DQK>(row)) + (col & 7);
    };

    const float nal2e = p.neg_alpha_log2e, alpha = p.alpha;
    const uint32_t k1u = (uint32_t)p.k1;
    auto step = [&](int t, auto S) {
        constexpr int sidx = decltype(S)::value;
        barrier_lds();  // publishes stage S, frees the other (read by step t - 1)
        issue(imin(t + 1, ntiles - 1), std::integral_constant<int, 1 - sidx>{});
        const uint16_t *sk = stage(S), *sv = stage(S) + BN * DQK;
        const int c0 = uniform(cur.start(t, BN));
        // mask: as the forward (workgroup-uniform tests; interval masks for
        // history tiles wholly inside or outside the global prefix)
        const bool full = uniform(((r0 < sd.U) & (c0 + BN <= sd.L) & (c0 + BN - 1 <= r0) &
                                   ((r1 - 1 - c0 < p.k1) | (c0 + BN <= p.k2e))) |
                                  ((r0 >= sd.U) & (c0 + BN <= sd.U) &
                                   ((c0 >= sd.U - p.k1 + 1) | (c0 + BN <= p.k2e)))) != 0;
        const int x0 = qi - c0 - 4 * hl;
        const int mode = uniform(r0 >= sd.U ? 0 : (c0 >= p.k2e ? 1 : (c0 + BN <= p.k2e ? 2 : 0)));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            floatx16 sacc = zero16(), pacc = zero16();
            if constexpr (NC == NCV) {
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(sk + r_off(kb, c));
                    sacc = mfma32(ak, qb[c], sacc);
                    const bf16x8 av = *reinterpret_cast<const bf16x8 *>(sv + r_off(kb, c));
                    pacc = mfma32(av, gb[c], pacc);
                }
            } else {
#pragma unroll
                for (int c = 0; c < (NC > NCV ? NC : NCV); ++c) {
                    if (c < NC) {
                        const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(sk + r_off(kb, c));
                        sacc = mfma32(ak, qb[c], sacc);
                    }
                    if (c < NCV) {
                        const bf16x8 av = *reinterpret_cast<const bf16x8 *>(sv + rv_off(kb, c));
                        pacc = mfma32(av, gb[c], pacc);
                    }
                }
            }
            // dS = g * (sigma + a * (alpha - alpha * sigma)), a = s * sigma:
            // 1 + t (1 - sigma) = 1 + alpha a (1 - sigma) / sigma, times sigma.
            // exp(-t) overflowing to inf gives sigma = 0, a = 0, dS = 0 (its
            // limit) with no NaN.
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float sv_ = sacc[r];
                const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sv_ * nal2e));
                const float a = sv_ * sg;
                ds[r] = pacc[r] * fmaf(a, fmaf(-alpha, sg, alpha), sg);
            }
            if (!full) {
                if (mode == 1) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int x = x0 - (32 * kb + 8 * (r >> 2) + (r & 3));
                        ds[r] = (uint32_t)x < k1u ? ds[r] : 0.0f;
                    }
                } else if (mode == 2) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int x = x0 - (32 * kb + 8 * (r >> 2) + (r & 3));
                        ds[r] = x >= 0 ? ds[r] : 0.0f;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = c0 + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
                        ds[r] = visible(qi, j, sd.U, p.k1, p.k2e) ? ds[r] : 0.0f;
                    }
                }
            }
            const bf16x8 d0 = cvt8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
            const bf16x8 d1 = cvt8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const uint2 k0 = tr_read_b64(sk + t_off(kb, h2, 0, db));
                    const uint2 k1v = tr_read_b64(sk + t_off(kb, h2, 1, db));
                    dqacc[db] = mfma32(__builtin_bit_cast(bf16x8, make_uint4(k0.x, k0.y, k1v.x, k1v.y)),
                                       h2 ? d1 : d0, dqacc[db]);
                }
            }
        }
        // the next stage's DMA (issued at the top of this step) has landed
        // before the barrier that publishes it
        vm_wait<0>();
    };

    if (ntiles > 0) {
        issue(0, std::integral_constant<int, 0>{});
        vm_wait<0>();
        for (int t = 0; t < ntiles; t += 2) {
            step(t, std::integral_constant<int, 0>{});
            if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
        }
    }

    // epilogue: dQ[qi][d] for d = 32*db + 8*g + 4*hl + 0..3, scaled by alpha / N
    if (qi < r1) {
        const float sc = p.out_scale;
        const int64_t row = sd.base + qi;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float o0 = dqacc[db][4 * g] * sc, o1 = dqacc[db][4 * g + 1] * sc;
                const float o2 = dqacc[db][4 * g + 2] * sc, o3 = dqacc[db][4 * g + 3] * sc;
                const int col = h * DQK + 32 * db + 8 * g + 4 * hl;
                if constexpr (OUTF32) {
                    float *orow = reinterpret_cast<float *>(p.dq) + row * p.lddq;
                    *reinterpret_cast<float4 *>(orow + col) = make_float4(o0, o1, o2, o3);
                } else {
                    uint16_t *orow = reinterpret_cast<uint16_t *>(p.dq) + row * p.lddq;
                    *reinterpret_cast<uint2 *>(orow + col) = cvt4_u2(o0, o1, o2, o3);
                }
            }
        }
    }
}

// dQ from stored dS.  When the workspace holds it, the dK/dV kernel writes the
// bf16 dS of each 64-row step x 128-key tile it visits (the operand of its dK
// product: per wave of 32 rows x 32 keys, lane (hl, key) holds the 8 rows
// 16 h2 + 8 (s / 4) + 4 hl + s % 4, s = 0..7, for h2 = 0, 1), and this
// kernel reads those blocks instead of recomputing S, dO.V^T and SiLU': per
// pair 2 bytes read back against 4 d flops and two transcendentals.  The
// fragment has the keys in the lane dimension; dQ contracts over keys, so
// the kernel gathers it with transposing LDS reads into the B operand
// layout, rows in the lane dimension, of
//   dQ^T (D x 32 rows) += K^T dS^T        (as the recomputing kernel).
// Same work items (128-row tiles), key tiles and order as the recomputing
// kernel, and each dQ accumulator adds the same products in the same order,
// so the two kernels give the same bits.  A 64-row half of the row tile that
// the dK/dV schedule does not visit for a key tile sees none of its keys and
// is skipped.
//
// Two workgroups of eight waves per CU (four waves per SIMD, 94 VGPRs), each
// with a ring of two stages of [K rows | dS] (16 + 16 KB at d = 128) filled
// by DMA one step ahead (the dS in the non-temporal form: read once), with
// the wait counts of the dK/dV kernel (gl_lds16_at: the DMA is ordered by the
// kernel's own waits and barriers); measured 5% faster than one workgroup
// with four stages three steps ahead: the second workgroup hides the first
// one's barriers and latencies.  Wave w takes rows
// 32 (w % 4) .. + 32 of the row tile and the d blocks of half w / 4 of dQ.
// Needs d_qk >= 64 (two 32-wide halves).
constexpr int DQS_THREADS = 512;
constexpr int DQS_STAGES = 2;
constexpr int DQS_TABLE = 256;  // step table entries (two halves of 128)

template <int DQK, bool OUTF32>
__global__ __launch_bounds__(DQS_THREADS, 2) void sla_bwd_dq_stored_kernel(AttnParams p)
{
    constexpr int BM = FWD_BM, BN = FWD_BN;
    constexpr int NT = DQS_THREADS, NST = DQS_STAGES;
    constexpr int NDB = DQK / 32, NDBW = NDB / 2;  // 32-wide d blocks: all, per wave
    constexpr int CPR = DQK / 8;                   // 16-byte chunks per K row
    constexpr int TCH = BN * CPR;                  // chunks of a 64-key K tile
    constexpr int DCH = 1024;                      // chunks of a step's dS (16 KB)
    constexpr int SPS = (TCH + DCH) / NT;          // DMA loads per thread and step
    constexpr int STAGE = (TCH + DCH) * 8;         // elements of a stage: [K | dS]
    static_assert(BN == 64 && BM == 128 && BWD_BN == 128 && BWD_BM == 64,
                  "64-key steps over 128-row tiles; dS blocks of 64 rows x 128 keys");
    static_assert(NDB >= 2 && TCH % 128 == 0 && (TCH + DCH) % NT == 0 && SPS <= 8 && (NST & (NST - 1)) == 0,
                  "two d halves; the K / dS split is wave-uniform; whole DMA rounds; a ring of 2^n");
    __shared__ __align__(16) uint16_t lds[NST * STAGE];
    // Step table: {first key, dS block of row half 0, of row half 1 (-1: not
    // visited)} of steps t, entry t % DQS_TABLE, filled 128 steps at a time
    // by vector code (one entry per lane) so that the per-step scalar work
    // stays small: the CU's one scalar unit serves all eight waves.
    __shared__ int4 stab[DQS_TABLE];

    const int nrec = p.s.fwd_base[p.B];
    const int item = xcd_remap(blockIdx.x, nrec * p.H);
    if (item < 0) return;
    const int h = item / nrec;
    const int rec = item - h * nrec;
    const int b = find_seq(p.s.fwd_base, p.B, rec);
    const SeqDims sd = seq_dims(p.offsets, p.num_targets, b);
    int r0, r1;
    row_tile(sd.L, sd.U, BM, rec - uniform(p.s.fwd_base[b]), r0, r1);
    r0 = uniform(r0);
    r1 = uniform(r1);
    const Ranges kr = fwd_key_ranges(sd.L, sd.U, p.k1, p.k2e, r0, r1, BN);
    const int kt_base = uniform(p.s.ktile_base[b]);

    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int rb = wv & 3, dh = wv >> 2;  // 32-row block, d half
    const int l32 = lane & 31, hl = lane >> 5;
    const int qi = r0 + 32 * rb + l32;
    const uint16_t *kg = reinterpret_cast<const uint16_t *>(p.k) + sd.base * p.ldk + h * DQK;

    const TileCursor cur(kr, BN);
    const int ntiles = uniform(cur.total);

    // Entry of step t: its first key c0, and for row half sg (rows r0 + 64 sg
    // ..) the dS block of the pair (row half, 128-key tile holding c0) within
    // this head's blocks, or -1 when the dK/dV schedule does not visit it
    // (ds_block_in_tile: the closed form of the schedule's step numbering).
    const int k1c = imin(p.k1, sd.U);
    auto fill = [&](int t0) __attribute__((always_inline)) {
        if (tid < DQS_TABLE / 2) {
            const int t = t0 + tid;
            int4 e = make_int4(0, -1, -1, 0);
            if (t < ntiles) {
                const int c0 = cur.start(t, BN);
                const int ct = c0 & ~(BWD_BN - 1);
                const int tb = p.s.ds_base[kt_base + (ct >> 7)];
                const int s0 = ds_block_in_tile(sd.L, sd.U, p.k1, k1c, p.k2e, ct, r0);
                const int s1 = r0 + 64 < r1
                                   ? ds_block_in_tile(sd.L, sd.U, p.k1, k1c, p.k2e, ct, r0 + 64)
                                   : -1;
                e = make_int4(c0, s0 < 0 ? -1 : tb + s0, s1 < 0 ? -1 : tb + s1, 0);
            }
            stab[t & (DQS_TABLE - 1)] = e;
        }
    };
    const char *const ds_head = reinterpret_cast<const char *>(p.ds) +
                                (int64_t)h * p.ds_head_blocks * DS_BLOCK_BYTES;

    // dS^T operands by transposing reads.  A stored fragment (32 keys x 32
    // rows) is made of 8-byte runs of four consecutive rows at one key: lane
    // (hl_f, key) of the dK/dV wave holds, for h2 = 0, 1, rows 16 h2 + 4 hl_f
    // .. + 3, then 16 h2 + 8 + 4 hl_f .. + 3.  In a 16-lane pass of
    // ds_read_b64_tr_b16, lane j pointing at the run (key k0 + j / 4, rows
    // 16 h2 + 4 (j % 4) ..) hands lane i row 16 h2 + i at keys k0 .. k0 + 3:
    // four k-slots of the B operand of dQ^T += K^T dS^T, rows in the lane
    // dimension.  Two such reads give the slots of a 16-key chunk h2k in the
    // order of the K^T operand (keys 16 h2k + 4 hl + 0..3, then + 8), the
    // bf16 values the recomputing kernel converts from its accumulator.  The
    // DMA stores key k of the hl_f = 1 half at slot k ^ 4, so that the two
    // halves of a pass fall in different banks.  Element offsets within the
    // stage's dS area, per (32-key block, 16-key chunk, first / second four
    // keys):
    uint32_t dso[2][2][2];
    {
        const int i16 = lane & 15, g = i16 & 3, h2r = (lane >> 4) & 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int h2k = 0; h2k < 2; ++h2k)
#pragma unroll
                for (int part = 0; part < 2; ++part) {
                    const int key = 16 * h2k + 4 * hl + 8 * part + (i16 >> 2);
                    const int hf = g & 1;
                    const int bytes = (2 * rb + kb) * 2048 + h2r * 1024 +
                                      (hf * 32 + (key ^ (4 * hf))) * 16 + (g >> 1) * 8;
                    dso[kb][h2k][part] = (uint32_t)(TCH * 8 + bytes / 2);
                }
    }

    floatx16 dqacc[NDBW];
#pragma unroll
    for (int i = 0; i < NDBW; ++i) dqacc[i] = zero16();

    // DMA of key step t (clamped to the last) into stage t % NST.  Chunk
    // P = i NT + tid: below TCH the K rows (as the recomputing kernel: chunk P
    // of the tile is physical chunk P % CPR of row P / CPR holding logical
    // chunk (P % CPR) ^ qswz(row); keys at or past L read key L - 1), then the
    // dS: fragment f = (P - TCH) / 128 of the stage (row half f / 4, 32-row
    // block (f / 2) % 2, 32-key block f % 2), 2 KB each, from its block; a
    // fragment of an unvisited pair reads the head's first block and is not
    // used.  Every step issues SPS loads per thread.  The per-lane parts of
    // the addresses are fixed for the item; the step adds its key offset and
    // the two blocks.  Returns the two coverage bits of the step.
    const uint32_t ldk_b = (uint32_t)p.ldk * 2u;
    const uint32_t wave_lds = uniform((int)(lds_addr(lds) + 16u * (uint32_t)(wv * 64)));
    uint32_t kprow[SPS], kcol[SPS], dlane[SPS], dfrag[SPS];
    bool dhalf1[SPS];
#pragma unroll
    for (int i = 0; i < SPS; ++i) {
        const int P = i * NT + wv * 64 + lane;
        kprow[i] = (uint32_t)(P / CPR);
        kcol[i] = 16u * (uint32_t)((P % CPR) ^ qswz<DQK>(P / CPR));
        const int f = imax(i * NT + wv * 64 - TCH, 0) / 128;  // wave-uniform
        // LDS chunk c of a fragment (h2 = c / 64, lane (hl_f, key) = c % 64)
        // takes the stored chunk of key key ^ 4 hl_f
        const int c = P & 127, hf = (c >> 5) & 1;
        dlane[i] = 16u * (uint32_t)((c & ~31) | ((c & 31) ^ (4 * hf)));
        dfrag[i] = (uint32_t)(4 * ((f >> 1) & 1) + (f & 1)) * 2048u;
        dhalf1[i] = f >= 4;
    }
    auto issue = [&](int t) __attribute__((always_inline)) -> uint32_t {
        const int4 e = stab[imin(t, ntiles - 1) & (DQS_TABLE - 1)];
        const int c0 = uniform(e.x), blk0 = uniform(e.y), blk1 = uniform(e.z);
        const uint32_t last = (uint32_t)(sd.L - 1 - c0);
        const char *krow = reinterpret_cast<const char *>(kg + (int64_t)c0 * p.ldk);
        const uint32_t kwo = (uint32_t)(c0 & (BWD_BN - 1)) * 64u;  // (key block of c0) x 2 KB
        const char *b0 = ds_head + (blk0 < 0 ? 0 : (int64_t)blk0 * DS_BLOCK_BYTES + kwo);
        const char *b1 = ds_head + (blk1 < 0 ? 0 : (int64_t)blk1 * DS_BLOCK_BYTES + kwo);
        const uint32_t sb = wave_lds + (uint32_t)(t & (NST - 1)) * (2u * STAGE);
#pragma unroll
        for (int ii = 0; ii < SPS; ++ii) {
            const int i = SPS - 1 - ii;  // the dS loads (from HBM) first, then the K rows (L2)
            if ((TCH % NT == 0) ? (i * NT < TCH) : (i * NT + wv * 64 < TCH))
                gl_lds16_at(krow + ((kprow[i] < last ? kprow[i] : last) * ldk_b + kcol[i]),
                            sb + 16u * (uint32_t)(i * NT));
            else  // dS: read once
                gl_lds16_at_stream((dhalf1[i] ? b1 : b0) + (dfrag[i] + dlane[i]),
                                   sb + 16u * (uint32_t)(i * NT));
        }
        return (blk0 >= 0 ? 1u : 0u) | (blk1 >= 0 ? 2u : 0u);
    };

    // K^T operand by transposing reads, as the recomputing kernel
    const int q4 = lane >> 4, j16 = lane & 15;
    auto t_off = [&](int kb, int h2, int rr, int db) {
        const int row = 32 * kb + 16 * h2 + 8 * rr + 4 * (q4 >> 1) + (j16 >> 2);
        const int col = 32 * db + 16 * (q4 & 1) + 4 * (j16 & 3);
        return row * DQK + 8 * ((col >> 3) ^ qswz<DQK>(row)) + (col & 7);
    };

    if (ntiles > 0) {
        fill(0);
        fill(DQS_TABLE / 2);
        __syncthreads();
        // coverage bits of the steps in flight: 2 bits per stage
        uint32_t vis = 0;
#pragma unroll
        for (int i = 0; i < NST - 1; ++i) vis |= issue(i) << (2 * i);
        for (int t = 0; t < ntiles; ++t) {
            // step t's DMA has landed (the newest (NST - 2) SPS loads, those of
            // steps t + 1 .., may still be in flight); the barrier publishes it
            // and frees stage (t + NST - 1) % NST, read by step t - 1
            vm_wait<(NST - 2) * SPS>();
            barrier_lds();
            // entries of steps t + 128 .. t + 255 replace those of steps
            // t - 128 .., all used by now; first read by the issue of step
            // t + 128 (after the barrier of loop step t + 128 - NST + 1), barriers later
            if ((t & (DQS_TABLE / 2 - 1)) == 0 && t > 0 && t + DQS_TABLE / 2 < ntiles)
                fill(t + DQS_TABLE / 2);
            const uint16_t *sk = lds + (t & (NST - 1)) * STAGE;
            // the DMA of step t + NST - 1 into the stage step t - 1 read (free
            // since the barrier), before this step's products so that it is in
            // flight under them
            {
                const uint32_t sh = 2u * (uint32_t)((t + NST - 1) & (NST - 1));
                vis = (vis & ~(3u << sh)) | (issue(t + NST - 1) << sh);
            }
            // this wave's row half sees the step: all LDS reads of the step
            // first (the dS^T and K^T operands), then the products
            if ((vis >> (2 * (t & (NST - 1)) + (rb >> 1))) & 1u) {
                uint2 dt[2][2][2];
                uint2 kt[2][2][NDBW][2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
                        for (int part = 0; part < 2; ++part)
                            dt[kb][h2][part] = tr_read_b64(sk + dso[kb][h2][part]);
#pragma unroll
                        for (int dw = 0; dw < NDBW; ++dw)
#pragma unroll
                            for (int rr = 0; rr < 2; ++rr)
                                kt[kb][h2][dw][rr] = tr_read_b64(sk + t_off(kb, h2, rr, dh * NDBW + dw));
                    }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const uint2 a0 = dt[kb][h2][0], a1 = dt[kb][h2][1];
                        const bf16x8 dsb = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
#pragma unroll
                        for (int dw = 0; dw < NDBW; ++dw) {
                            const uint2 k0 = kt[kb][h2][dw][0], k1v = kt[kb][h2][dw][1];
                            dqacc[dw] = mfma32(
                                __builtin_bit_cast(bf16x8, make_uint4(k0.x, k0.y, k1v.x, k1v.y)), dsb,
                                dqacc[dw]);
                        }
                    }
            }
            // the DMA of step t + NST - 1 into the stage step t - 1 read (free
            // since the barrier), after this step's products: the waves start
            // their products right after the barrier, and the scalar work of
            // the issue, on the CU's one scalar unit, runs under other waves'
            // products
        }
        vm_wait<0>();  // no DMA (of the clamped steps past the end) left in flight
    }

    // epilogue: dQ[qi][d] for d = 32 db + 8 g + 4 hl + 0..3, scaled by alpha / N
    if (qi < r1) {
        const float sc = p.out_scale;
        const int64_t row = sd.base + qi;
#pragma unroll
        for (int dw = 0; dw < NDBW; ++dw) {
            const int db = dh * NDBW + dw;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float o0 = dqacc[dw][4 * g] * sc, o1 = dqacc[dw][4 * g + 1] * sc;
                const float o2 = dqacc[dw][4 * g + 2] * sc, o3 = dqacc[dw][4 * g + 3] * sc;
                const int col = h * DQK + 32 * db + 8 * g + 4 * hl;
                if constexpr (OUTF32) {
                    float *orow = reinterpret_cast<float *>(p.dq) + row * p.lddq;
                    *reinterpret_cast<float4 *>(orow + col) = make_float4(o0, o1, o2, o3);
                } else {
                    uint16_t *orow = reinterpret_cast<uint16_t *>(p.dq) + row * p.lddq;
                    *reinterpret_cast<uint2 *>(orow + col) = cvt4_u2(o0, o1, o2, o3);
                }
            }
        }
    }
}

template <bool OUTF32>
static hipError_t launch_dq_o(const AttnParams &p, hipStream_t st)
{
    return with_head_dims(p, [&](auto QK, auto V) {
        constexpr int DQK = decltype(QK)::value;
        if constexpr (DQK >= 64) {
            if (p.ds) {
                hipLaunchKernelGGL((sla_bwd_dq_stored_kernel<DQK, OUTF32>), dim3(p.grid_fwd),
                                   dim3(DQS_THREADS), 0, st, p);
                return hipGetLastError();
            }
        }
        if (p.ds) return hipErrorInvalidValue;  // no stored dS below d_qk = 64
        hipLaunchKernelGGL((sla_bwd_dq_kernel<DQK, decltype(V)::value, OUTF32>),
                           dim3(p.grid_fwd), dim3(256), 0, st, p);
        return hipGetLastError();
    });
}

hipError_t launch_bwd_dq_bf16(const AttnParams &p, hipStream_t st)
{
    return p.out_f32 ? launch_dq_o<true>(p, st) : launch_dq_o<false>(p, st);
}

}  // namespace sla
