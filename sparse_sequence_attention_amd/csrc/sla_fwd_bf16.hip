// sla_fwd_bf16.hip -- SLA forward on gfx950: bf16 MFMA, fp32 accumulation.
//
// Computes O = (1/N) (SiLU(alpha Q K^T) (.) M) V per jagged sequence and head
// (ULTRA-HSTU paper, section 3 Eq.3 and section 4.2.1 Eq.6-7; pointwise SiLU
// with no softmax, HSTU notes section 2.4 Eq.2).  Because there is no softmax
// there is no running max or rescale: the output accumulates SiLU(S) V
// directly and 1/N is applied once at the end.
//
// Work item: one row tile of up to 128 rows (4 waves x 32) of one head, two
// workgroups per CU.  It visits only the key tiles holding visible keys
// (global prefix, local band, and for target rows the history window of the
// first target plus the diagonal), 64 keys per step.  Per step each wave
// computes, per 32-key block,
//   S^T (32 keys x 32 rows) = K Q^T      (K from LDS, Q^T held in registers)
//   P^T = mask(S^T * sigmoid(alpha S^T))  in registers, rounded to bf16
//   O^T (D x 32 rows)     += V^T P^T     (V^T by transposing LDS reads)
// with the two blocks' products and SiLU interleaved in one wave.
// Computing S transposed puts the rows in the MFMA's lane dimension, so P^T
// feeds the second MFMA as its B operand straight from the accumulator.  Both
// products are bf16 MFMAs with fp32 accumulation: the bf16 inputs are used as
// stored, and only P is rounded (to bf16, 8 significant bits; the rounding
// errors of the ~10^3 terms of a row are independent, so the output moves by
// ~2^-9 / sqrt(3) of its own size, rms).  The K and V rows of the next step
// come HBM -> LDS by DMA into the idle one of two stages, already in the
// swizzled layout.  One LDS-only barrier per step, so the DMA stays in flight
// across it.  O is written in bf16 or, on request, fp32.
#include <type_traits>

#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

// 16-byte chunk swizzle of the [64][D] K and V stage tiles: logical chunk c
// of row r sits at c ^ fswz<D>(r), u = r*D/128 (the 256-byte bank row),
// Q4 = D/32.  The 16 rows of a 16-lane pass of a 16-byte read, and the 4 rows
// x 64 bytes of a 32-lane pass of a transposing read, hit distinct banks.
template <int D>
__device__ __forceinline__ int fswz(int r)
{
    constexpr int Q4 = D / 32;
    const int u = r * D / 128;
    return 4 * (u % Q4) + (u / Q4) % 4;
}

// CAND: candidate scoring against a cached history (p.cand_offsets): the item
// list holds the candidate row tiles only; sequence b is virtually
// [history (U keys) | padding up to a multiple of the key tile | candidates],
// history keys and values come from k, v, the candidates' rows, keys and
// values from q, kc, vc, and O rows go to the candidate layout.  The padding
// (never visible) keeps candidate keys out of the history's key tiles, so a
// candidate's sum runs over the same history tiles in the same order and
// then its own key, wherever it sits among the candidates: scores do not
// depend on which other candidates share the call.
// DQK: the Q / K head width, DV: the V (and O) width.
template <int DQK, int DV, bool CAND, bool OUTF32>
__global__ __launch_bounds__(256, 2) void sla_fwd_bf16_kernel(AttnParams p)
{
    constexpr int BM = FWD_BM, BN = FWD_BN;
    constexpr int NT = 256;
    constexpr int NC = DQK / 16;  // 16-wide contraction chunks of Q.K
    constexpr int NDB = DV / 32;  // 32-wide output blocks
    constexpr int CPR = DQK / 8, CPRV = DV / 8;     // 16-byte chunks per K / V row
    constexpr int TCH = BN * CPR, TCHV = BN * CPRV;  // chunks of one 64-key K / V tile
    constexpr int KPT = TCH / NT, KPTV = TCHV / NT;  // DMA loads per thread and tile
    static_assert(BN == 64 && BM == 128, "64-key steps over 128-row tiles");
    static_assert(TCH % NT == 0 && TCHV % NT == 0 && KPT + KPTV <= 8,
                  "whole DMA rounds, at most 8 per stage");
    // two stages of [K | V] bf16 rows; separate arrays so that the compiler
    // can tell the DMA into one from the reads of the other
    __shared__ __align__(16) uint16_t st0[BN * (DQK + DV)], st1[BN * (DQK + DV)];

    const int nrec = p.s.fwd_base[p.B];
    const int item = xcd_remap(blockIdx.x, nrec * p.H);
    if (item < 0) return;
    const int h = item / nrec;
    const int rec = item - h * nrec;
    const int b = find_seq(p.s.fwd_base, p.B, rec);
    SeqDims sd = seq_dims(p.offsets, CAND ? nullptr : p.num_targets, b);
    int64_t cbase = 0;  // first candidate of the sequence (CAND)
    int uc = sd.U;      // first candidate row of the virtual sequence (CAND)
    if constexpr (CAND) {
        cbase = uniform64(p.cand_offsets[b]);
        const int nc = uniform((int)(p.cand_offsets[b + 1] - cbase));
        sd.U = sd.L;                // the history length: visibility as a target
        uc = cdiv(sd.U, BN) * BN;   // candidates start on a key-tile boundary
        sd.L = uc + nc;
    }
    int r0, r1;
    row_tile(sd.L, uc, BM, rec - uniform(p.s.fwd_base[b]) + (CAND ? cdiv(uc, BM) : 0), r0, r1);
    r0 = uniform(r0);
    r1 = uniform(r1);
    const Ranges kr = fwd_key_ranges(sd.L, sd.U, p.k1, p.k2e, r0, r1, BN);

    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int l32 = lane & 31, hl = lane >> 5;

    const uint16_t *qg = reinterpret_cast<const uint16_t *>(p.q) + sd.base * p.ldq + h * DQK;
    const uint16_t *kg = reinterpret_cast<const uint16_t *>(p.k) + sd.base * p.ldk + h * DQK;
    const uint16_t *vg = reinterpret_cast<const uint16_t *>(p.v) + sd.base * p.ldv + h * DV;

    // Q^T operand: lane holds row qi, d-slots 16c + 8*hl .. +8 (CAND: the
    // candidate rows, qi - U of the sequence's candidates)
    const int qi = r0 + 32 * wv + l32;
    const uint16_t *qsrc = CAND ? reinterpret_cast<const uint16_t *>(p.q) + cbase * p.ldq + h * DQK
                                : qg;
    const int qrow = CAND ? qi - uc : qi, qlim = CAND ? sd.L - uc : sd.L;
    bf16x8 qb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) qb[c] = as_bf16x8(ld16_row(qsrc, p.ldq, qrow, qlim, 16 * c + 8 * hl));

    const TileCursor cur(kr, BN);
    const int ntiles = uniform(cur.total);

    floatx16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = zero16();

    auto stage = [&](auto S) -> uint16_t * {
        if constexpr (decltype(S)::value == 0) return st0;
        else return st1;
    };
    // DMA of the K and V rows of key tile t into a stage ([K | V], the V rows
    // after the BN * DQK elements of K): chunk P = i*NT + tid of a tile is
    // physical chunk P % CPR of key row P / CPR and holds its logical chunk
    // (P % CPR) ^ fswz(row) (CPR, fswz of the tile's own width); keys at or
    // past L read key L - 1 (such tiles are never "full", and the mask
    // removes them)
    const uint32_t ldk_b = (uint32_t)p.ldk * 2u, ldv_b = (uint32_t)p.ldv * 2u;
    // CAND: keys at or past the history length are the candidates' own
    const char *kcg = nullptr, *vcg = nullptr;
    if constexpr (CAND) {
        kcg = reinterpret_cast<const char *>(reinterpret_cast<const uint16_t *>(p.kc) +
                                             cbase * p.ldkc + h * DQK);
        vcg = reinterpret_cast<const char *>(reinterpret_cast<const uint16_t *>(p.vc) +
                                             cbase * p.ldvc + h * DV);
    }
    auto issue = [&](int t, auto S) {
        const int c0 = uniform(cur.start(t, BN));
        int last = uniform(sd.L - 1 - c0);
        const char *krow = reinterpret_cast<const char *>(kg + (int64_t)c0 * p.ldk);
        const char *vrow = reinterpret_cast<const char *>(vg + (int64_t)c0 * p.ldv);
        uint32_t lk = ldk_b, lv = ldv_b;
        if constexpr (CAND) {
            // a key tile lies wholly below uc (history, whose padding keys
            // U <= j < uc, never visible, read history key U - 1) or wholly
            // in the candidates
            if (c0 >= uc) {
                krow = kcg + (int64_t)(c0 - uc) * p.ldkc * 2;
                vrow = vcg + (int64_t)(c0 - uc) * p.ldvc * 2;
                lk = (uint32_t)p.ldkc * 2u;
                lv = (uint32_t)p.ldvc * 2u;
            } else {
                last = uniform(sd.U - 1 - c0);
            }
        }
        uint16_t *sb = stage(S);
#pragma unroll
        for (int i = 0; i < (KPT > KPTV ? KPT : KPTV); ++i) {
            const int P = i * NT + tid;
            if (i < KPT) {
                const int prow = P / CPR;
                const uint32_t row = (uint32_t)imin(prow, last);
                const uint32_t c = (uint32_t)((P % CPR) ^ fswz<DQK>(prow));
                gl_lds16(krow + (row * lk + 16u * c), sb + (i * NT + wv * 64) * 8);
            }
            if (i < KPTV) {
                const int prow = P / CPRV;
                const uint32_t row = (uint32_t)imin(prow, last);
                const uint32_t c = (uint32_t)((P % CPRV) ^ fswz<DV>(prow));
                gl_lds16(vrow + (row * lv + 16u * c), sb + (BN * DQK + (i * NT + wv * 64) * 8));
            }
        }
    };
    // per-lane LDS offsets (elements).  K operand: key row 32*kb + l32,
    // logical chunk 2c + hl.  V^T operand by transposing reads (quarter
    // q = lane/16, j = lane%16): keys 32*kb + 16*h2 + 8*rr + 4*(q/2) + j/4,
    // d-columns 32*db + 16*(q%2) + 4*(j%4); the keys come in the order in
    // which the S^T accumulator hands them to P^T (8*(r/4) + 4*hl + r%4).
    const int q4 = lane >> 4, j16 = lane & 15;
    auto k_off = [&](int kb, int c) {
        const int r = 32 * kb + l32;
        return r * DQK + 8 * ((2 * c + hl) ^ fswz<DQK>(r));
    };
    auto v_off = [&](int kb, int h2, int rr, int db) {
        const int row = 32 * kb + 16 * h2 + 8 * rr + 4 * (q4 >> 1) + (j16 >> 2);
        const int col = 32 * db + 16 * (q4 & 1) + 4 * (j16 & 3);
        return row * DV + 8 * ((col >> 3) ^ fswz<DV>(row)) + (col & 7);
    };

    const float nal2e = p.neg_alpha_log2e;
    const uint32_t k1u = (uint32_t)p.k1;
    auto step = [&](int t, auto S) {
        constexpr int sidx = decltype(S)::value;
        barrier_lds();  // publishes stage S, frees the other (read by step t - 1)
        // unconditional (the last step re-reads its own tile): a DMA under a
        // branch costs the compiler its wait counts
        issue(imin(t + 1, ntiles - 1), std::integral_constant<int, 1 - sidx>{});
        const uint16_t *sk = stage(S), *sv = stage(S) + BN * DQK;
        const int c0 = uniform(cur.start(t, BN));

        // mask (partial tiles only, a workgroup-uniform branch).  Element r of
        // key block kb has x = qi - j = x0 - c with the constant
        // c = 32*kb + 8*(r/4) + r%4: a history row sees key j iff x >= 0 and
        // (x < K1 or j < K2e); keys past L give x < 0.  Tiles wholly inside
        // or outside the global prefix need one interval test per element.
        // Target rows see the same history keys (those of the first target
        // slot), so a history tile wholly inside that view needs no mask
        // either; the diagonal and boundary tiles do.
        // bitwise, not short-circuit: no branch between the DMA issue and
        // the products
        const bool full = uniform(((r0 < sd.U) & (c0 + BN <= sd.L) & (c0 + BN - 1 <= r0) &
                                   ((r1 - 1 - c0 < p.k1) | (c0 + BN <= p.k2e))) |
                                  ((r0 >= sd.U) & (c0 + BN <= sd.U) &
                                   ((c0 >= sd.U - p.k1 + 1) | (c0 + BN <= p.k2e)))) != 0;
        const int x0 = qi - c0 - 4 * hl;
        const int mode = uniform(r0 >= sd.U ? 0 : (c0 >= p.k2e ? 1 : (c0 + BN <= p.k2e ? 2 : 0)));

        auto s_blk = [&](int kb) {
            floatx16 acc = zero16();
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sk + k_off(kb, c));
                acc = mfma32(a, qb[c], acc);
            }
            return acc;
        };
        auto mask_blk = [&](float *sacc, int kb) {
            if (!full) {
                if (mode == 1) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int x = x0 - (32 * kb + 8 * (r >> 2) + (r & 3));
                        sacc[r] = (uint32_t)x < k1u ? sacc[r] : 0.0f;
                    }
                } else if (mode == 2) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int x = x0 - (32 * kb + 8 * (r >> 2) + (r & 3));
                        sacc[r] = x >= 0 ? sacc[r] : 0.0f;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = c0 + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
                        sacc[r] = visible(qi, j, sd.U, p.k1, p.k2e) ? sacc[r] : 0.0f;
                    }
                }
            }
        };
        auto silu_blk = [&](const floatx16 &sacc, float *f) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float sv = sacc[r];
                f[r] = sv * sigmoid_fast(sv, nal2e);
            }
        };
        auto pv_blk = [&](int kb, const float *f) {
            const bf16x8 p0 = cvt8(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
            const bf16x8 p1 = cvt8(f[8], f[9], f[10], f[11], f[12], f[13], f[14], f[15]);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const uint2 v0 = tr_read_b64(sv + v_off(kb, h2, 0, db));
                    const uint2 v1 = tr_read_b64(sv + v_off(kb, h2, 1, db));
                    oacc[db] = mfma32(__builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y)),
                                      h2 ? p1 : p0, oacc[db]);
                }
            }
        };
        // The two 32-key blocks run software-pipelined in one wave: block 1's
        // S^T products under block 0's SiLU, block 0's P.V products under
        // block 1's SiLU (the MFMA pipe and the VALU work concurrently on
        // independent instructions of one wave).  The mask zeroes P after
        // the SiLU (SiLU(0) = 0), so no branch splits a block's products
        // from the other block's SiLU; the next tile's DMA is spread over
        // block 0's products instead of leaving in one burst after the
        // barrier.  Per step: 16 S^T and 16 P.V MFMAs, 2 x 16 SiLU.
        floatx16 sa = s_blk(0);
        floatx16 sb = s_blk(1);
        float fa[16], fb[16];
        silu_blk(sa, fa);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 4, 0);
#pragma unroll
        for (int i = 0; i < 2 * NC; ++i) {
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            if (i < 2 * NC - 2) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
            if (i < NC) {
                if (i < KPT + KPTV) __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(SG_VALU, 10, 0);
            }
        }
        mask_blk(fa, 0);
        pv_blk(0, fa);
        silu_blk(sb, fb);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 4, 1);
        __builtin_amdgcn_sched_group_barrier(SG_VALU, 8, 1);
#pragma unroll
        for (int i = 0; i < 2 * NDB; ++i) {
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 1);
            if (i < 2 * NDB - 2) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 1);
            __builtin_amdgcn_sched_group_barrier(SG_VALU, 10, 1);
        }
        mask_blk(fb, 1);
        pv_blk(1, fb);
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

    // epilogue: O[qi][d] for d = 32*db + 8*g + 4*hl + 0..3
    if (qi < r1) {
        const int64_t orow_i = CAND ? cbase + (qi - uc) : sd.base + qi;
        const float sc = p.out_scale;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float o0 = oacc[db][4 * g] * sc, o1 = oacc[db][4 * g + 1] * sc;
                const float o2 = oacc[db][4 * g + 2] * sc, o3 = oacc[db][4 * g + 3] * sc;
                const int col = h * DV + 32 * db + 8 * g + 4 * hl;
                if constexpr (OUTF32) {
                    float *orow = reinterpret_cast<float *>(p.o) + orow_i * p.ldo;
                    *reinterpret_cast<float4 *>(orow + col) = make_float4(o0, o1, o2, o3);
                } else {
                    uint16_t *orow = reinterpret_cast<uint16_t *>(p.o) + orow_i * p.ldo;
                    *reinterpret_cast<uint2 *>(orow + col) = cvt4_u2(o0, o1, o2, o3);
                }
            }
        }
    }
}

template <bool CAND, bool OUTF32>
static hipError_t launch_fwd_o(const AttnParams &p, hipStream_t st)
{
    return with_head_dims(p, [&](auto QK, auto V) {
        hipLaunchKernelGGL((sla_fwd_bf16_kernel<decltype(QK)::value, decltype(V)::value, CAND, OUTF32>),
                           dim3(p.grid_fwd), dim3(256), 0, st, p);
        return hipGetLastError();
    });
}

template <bool CAND>
static hipError_t launch_fwd(const AttnParams &p, hipStream_t st)
{
    return p.out_f32 ? launch_fwd_o<CAND, true>(p, st) : launch_fwd_o<CAND, false>(p, st);
}

hipError_t launch_fwd_bf16(const AttnParams &p, hipStream_t st) { return launch_fwd<false>(p, st); }

hipError_t launch_fwd_candidates_bf16(const AttnParams &p, hipStream_t st)
{
    if (!p.cand_offsets) return hipErrorInvalidValue;
    return launch_fwd<true>(p, st);
}

}  // namespace sla
