// sla_fwd_bf16.hip -- SLA forward on gfx950: bf16 MFMA, fp32 accumulation.
//
// Computes O = (1/N) (SiLU(alpha Q K^T) (.) M) V per jagged sequence and head
// (ULTRA-HSTU paper, section 3 Eq.3 and section 4.2.1 Eq.6-7; pointwise SiLU
// with no softmax, HSTU notes section 2.4 Eq.2).  Because there is no softmax
// there is no running max or rescale: the output accumulates SiLU(S) V
// directly and 1/N is applied once at the end.
//
// Work item: one row tile of up to 128 rows (4 waves x 32) of one head.  It
// visits only the key tiles holding visible keys (global prefix, local band,
// and for target rows the history window of the first target plus the
// diagonal), 64 keys per step.  Per step each wave computes
//   S^T (64 keys x 32 rows) = K Q^T      (K from LDS, Q^T held in registers)
//   P^T = mask(S^T) * sigmoid(alpha S^T)  in registers, rounded to fp16
//   O^T (D x 32 rows)     += V^T P^T     (V^T from LDS, converted to fp16)
// Computing S transposed puts the rows in the MFMA's lane dimension, so P^T
// feeds the second MFMA as its B operand straight from the accumulator; the
// V tile is transposed once when it is staged into LDS.  K/V tiles are double
// buffered and the next tile's HBM loads are in flight during the MFMAs.
#include "sla_device.h"
#include "sla_kernels.h"
#include "sla_tiles.h"

namespace sla {

template <int D>
__global__ __launch_bounds__(256, 2) void sla_fwd_bf16_kernel(AttnParams p)
{
    constexpr int BM = FWD_BM, BN = FWD_BN;
    constexpr int NC = D / 16;   // 16-wide contraction chunks of Q.K
    constexpr int NDB = D / 32;  // 32-wide output blocks
    static_assert(BN == 64, "transposed tiles assume 64 keys");
    __shared__ __align__(16) uint16_t sk[2][BN * D];
    __shared__ __align__(16) uint16_t svt[2][D * BN];

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

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;

    const uint16_t *qg = reinterpret_cast<const uint16_t *>(p.q) + sd.base * p.ldq + h * D;
    const uint16_t *kg = reinterpret_cast<const uint16_t *>(p.k) + sd.base * p.ldk + h * D;
    const uint16_t *vg = reinterpret_cast<const uint16_t *>(p.v) + sd.base * p.ldv + h * D;

    // Q^T operand: lane holds row qi, d-slots 16c + 8*hl .. +8
    const int qi = r0 + 32 * wv + l32;
    bf16x8 qb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) qb[c] = as_bf16x8(ld16_row(qg, p.ldq, qi, sd.L, 16 * c + 8 * hl));

    const TileCursor cur(kr, BN);
    const int ntiles = uniform(cur.total);

    floatx16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = zero16();

    Tile64<D> kt, vt;
    int c_next = cur.start(0, BN);
    // keys at or past L (last tile of a sequence) hold copies of key L - 1;
    // such tiles are never "full", and the mask removes them
    if (ntiles > 0) {
        kt.load_clamped(kg, p.ldk, c_next, sd.L, tid);
        vt.load_clamped(vg, p.ldv, c_next, sd.L, tid);
    }
    const float nal2e = p.neg_alpha_log2e;
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int c0 = uniform(c_next);
        kt.store_rows(sk[buf], tid);
        store_transposed_f16<D>(vt, svt[buf], tid, 1.0f);
        c_next = cur.start(t + 1, BN);
        if (t + 1 < ntiles) {
            kt.load_clamped(kg, p.ldk, c_next, sd.L, tid);
            vt.load_clamped(vg, p.ldv, c_next, sd.L, tid);
        }
        __syncthreads();

        // mask (partial tiles only, a workgroup-uniform branch).  Element r of
        // key block kb has x = qi - j = x0 - c with the constant
        // c = 32*kb + 8*(r/4) + r%4: a history row sees key j iff x >= 0 and
        // (x < K1 or j < K2e); keys past L give x < 0.  Tiles wholly inside
        // or outside the global prefix need one interval test per element.
        const bool full = uniform((r0 < sd.U) && (c0 + BN <= sd.L) && (c0 + BN - 1 <= r0) &&
                                  ((r1 - 1 - c0 < p.k1) || (c0 + BN <= p.k2e))) != 0;
        const int x0 = qi - c0 - 4 * hl;
        const int mode = uniform(r0 >= sd.U ? 0 : (c0 >= p.k2e ? 1 : (c0 + BN <= p.k2e ? 2 : 0)));
        const uint32_t k1u = (uint32_t)p.k1;

        // per 32-key block: S^T = K Q^T, mask, P = s * sigmoid(alpha s), then
        // O^T += V^T P^T over its two 16-key chunks; one block's S is live at a time
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            floatx16 sacc = zero16();
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                bf16x8 a = lds_row_chunk<D>(sk[buf], 32 * kb + l32, 2 * c + hl);
                sacc = mfma32(a, qb[c], sacc);
            }
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
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float sv = sacc[r];
                sacc[r] = sv * sigmoid_fast(sv, nal2e);
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int kc = 2 * kb + h2, o = 8 * h2;
                halfx8 pb = cvt8h(sacc[o + 0], sacc[o + 1], sacc[o + 2], sacc[o + 3], sacc[o + 4],
                                  sacc[o + 5], sacc[o + 6], sacc[o + 7]);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    halfx8 a = lds_t_chunk_h(svt[buf], 32 * db + l32, 2 * kc + hl);
                    oacc[db] = mfma32h(a, pb, oacc[db]);
                }
            }
        }
    }

    // epilogue: O[qi][d] for d = 32*db + 8*g + 4*hl + 0..3
    if (qi < r1) {
        uint16_t *orow = reinterpret_cast<uint16_t *>(p.o) + (sd.base + qi) * p.ldo + h * D;
        const float sc = p.out_scale;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 v = cvt4_u2(oacc[db][4 * g] * sc, oacc[db][4 * g + 1] * sc,
                                  oacc[db][4 * g + 2] * sc, oacc[db][4 * g + 3] * sc);
                *reinterpret_cast<uint2 *>(orow + 32 * db + 8 * g + 4 * hl) = v;
            }
        }
    }
}

hipError_t launch_fwd_bf16(const AttnParams &p, hipStream_t st)
{
    dim3 grid(p.grid_fwd), block(256);
    switch (p.d) {
    case 32: hipLaunchKernelGGL(sla_fwd_bf16_kernel<32>, grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL(sla_fwd_bf16_kernel<64>, grid, block, 0, st, p); break;
    case 128: hipLaunchKernelGGL(sla_fwd_bf16_kernel<128>, grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sla
