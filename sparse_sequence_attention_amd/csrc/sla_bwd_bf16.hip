// sla_bwd_bf16.hip -- SLA backward on gfx950: bf16 MFMA, fp32 accumulation,
// no atomics.
//
// With a_ij = SiLU(alpha s_ij), s_ij = q_i . k_j, O_i = (1/N) sum_j a_ij v_j
// (ULTRA-HSTU paper, section 3 Eq.3 under the semi-local mask of section
// 4.2.1 Eq.7), the chain rule gives, over visible pairs,
//   dV_j = (1/N) sum_i a_ij dO_i
//   dS_ij = (alpha/N) (dO_i . v_j) sigma_ij (1 + t_ij (1 - sigma_ij)),  t = alpha s
//   dQ_i = sum_j dS_ij k_j,     dK_j = sum_i dS_ij q_i.
// The kernels keep s*sigma and g*sigma*(1 + t(1 - sigma)) (g = dO.v) in the
// MFMA operands and apply 1/N and alpha once in the epilogues.  The products
// that consume P or dS run on fp16 operands (P, dS, dO^T, Q^T, K^T); dS and dO
// are multiplied by a power of two G that maps max|dO| into [1, 2) (computed on
// the device before these kernels) so that fp16's range follows the gradient
// scale, and the epilogues divide it out.
//
// Ownership split (the KV-parallel / Q-parallel pair of backward schedules the
// WHALE notes describe): the dK/dV kernel owns a 128-key tile and walks the row
// tiles that see it; the dQ kernel owns a 128-row tile and walks its key tiles,
// recomputing S and dP.  Global-prefix key tiles are seen by every later row,
// so they are cut into row chunks whose fp32 partial sums a third kernel adds
// in chunk order: results are bitwise reproducible.
#include "sla_device.h"
#include "sla_kernels.h"
#include "sla_tiles.h"

namespace sla {

constexpr int DS_SLOT_TAB = 512;  // steps of a dK/dV item whose dS slot is tabulated

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void sla_bwd_dkdv_bf16_kernel(AttnParams p)
{
    constexpr int BN = BWD_BN, BM = BWD_BM;
    constexpr int NC = D / 16, NDB = D / 32;
    static_assert(BM == 64, "row steps are 64-row tiles");
    __shared__ __align__(16) uint16_t sq[2][BM * D];
    __shared__ __align__(16) uint16_t sdo[2][BM * D];
    __shared__ __align__(16) uint16_t sqt[2][D * BM];
    __shared__ __align__(16) uint16_t sdot[2][D * BM];
    __shared__ int16_t slot_tab[DS_SLOT_TAB];

    const int nrec = p.s.bwd_base[p.B];
    const int item = xcd_remap(blockIdx.x, nrec * p.H);
    if (item < 0) return;
    const int h = item / nrec;
    const int rec = item - h * nrec;
    const int b = find_seq(p.s.bwd_base, p.B, rec);
    const SeqDims sd = seq_dims(p.offsets, p.num_targets, b);
    int np, nch;
    bwd_items(sd.L, sd.U, p.k2e, BN, BM, np, nch);
    const BwdItem it = bwd_item(sd.L, sd.U, p.k1, p.k2e, BN, BM, rec - uniform(p.s.bwd_base[b]),
                                np, nch);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;

    const uint16_t *qg = reinterpret_cast<const uint16_t *>(p.q) + sd.base * p.ldq + h * D;
    const uint16_t *kg = reinterpret_cast<const uint16_t *>(p.k) + sd.base * p.ldk + h * D;
    const uint16_t *vg = reinterpret_cast<const uint16_t *>(p.v) + sd.base * p.ldv + h * D;
    const uint16_t *gg = reinterpret_cast<const uint16_t *>(p.dout) + sd.base * p.lddo + h * D;

    // stationary K^T and V^T operands: lane holds key kj, d-slots 16c + 8*hl .. +8
    const int kj = it.c0 + 32 * wv + l32;
    bf16x8 kb[NC], vb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        kb[c] = as_bf16x8(ld16_row(kg, p.ldk, kj, it.c1, 16 * c + 8 * hl));
        vb[c] = as_bf16x8(ld16_row(vg, p.ldv, kj, it.c1, 16 * c + 8 * hl));
    }
    // stored-dS path: the fp16 copy of this key tile that dQ = dS K reads
    // (written once per key tile, by its first chunk)
    if (p.kh != nullptr && it.chunk == 0 && kj < it.c1) {
        uint16_t *khr = p.kh + (sd.base + kj) * ((int64_t)p.H * D) + h * D + 8 * hl;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            *reinterpret_cast<halfx8 *>(khr + 16 * c) = bf16x8_to_halfx8(kb[c]);
    }
    const int rt_first = p.ds != nullptr ? uniform(p.s.rt_base[b]) : 0;

    // row steps: history tiles covering [ha, hb), then target tiles covering [ta, tb)
    int h_first = 0, nh = 0, t_first = 0, nt = 0;
    if (it.ha < it.hb) {
        h_first = it.ha / BM;
        nh = cdiv(it.hb, BM) - h_first;
    }
    if (it.ta < it.tb) {
        t_first = (it.ta - sd.U) / BM;
        nt = cdiv(it.tb - sd.U, BM) - t_first;
    }
    const int nsteps = nh + nt;

    floatx16 dkacc[NDB], dvacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
        dkacc[i] = zero16();
        dvacc[i] = zero16();
    }

    Tile64<D> qt, gt;
    auto step_rows = [&](int s, int &m0, int &m1) {
        if (s < nh) {
            m0 = (h_first + s) * BM;
            m1 = imin(m0 + BM, sd.U);
        } else {
            m0 = sd.U + (t_first + s - nh) * BM;
            m1 = imin(m0 + BM, sd.L);
        }
    };
    // stored-dS path: the slot of this key tile in the visiting order of the
    // 64-row tile [m0, m1) that step s covers, tabulated for the first
    // DS_SLOT_TAB steps before the loop (scalar work kept out of the steps)
    auto step_slot = [&](int m0, int m1) {
        const Ranges kr = fwd_key_ranges(sd.L, sd.U, p.k1, p.k2e, m0, m1, DS_BN);
        return cursor_slot(kr, it.c0, DS_BN);
    };
    if (p.ds != nullptr) {
        for (int st = tid; st < imin(nsteps, DS_SLOT_TAB); st += blockDim.x) {
            int a0, a1;
            step_rows(st, a0, a1);
            slot_tab[st] = (int16_t)step_slot(a0, a1);
        }
    }

    // rows at or past m1 of a step hold copies of row m1 - 1; such steps are
    // never "full", and the mask removes those rows
    int m0n = 0, m1n = 0;
    if (nsteps > 0) {
        step_rows(0, m0n, m1n);
        qt.load_clamped(qg, p.ldq, m0n, m1n, tid);
        gt.load_clamped(gg, p.lddo, m0n, m1n, tid);
    }
    const float nal2e = p.neg_alpha_log2e, alpha = p.alpha;
    const float gscale = *p.grad_scale;
    const bool key_tile_full = (it.c1 - it.c0 == BN);
    // g = dO.v enters dS only: carry the gradient scale in the stationary V
#pragma unroll
    for (int c = 0; c < NC; ++c) vb[c] = scale_bf16x8(vb[c], gscale);
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        const int m0 = uniform(m0n), m1 = uniform(m1n);
        qt.store_rows(sq[buf], tid);
        store_transposed_f16<D>(qt, sqt[buf], tid, 1.0f);
        gt.store_rows(sdo[buf], tid);
        store_transposed_f16<D>(gt, sdot[buf], tid, gscale);
        if (s + 1 < nsteps) {
            step_rows(s + 1, m0n, m1n);
            qt.load_clamped(qg, p.ldq, m0n, m1n, tid);
            gt.load_clamped(gg, p.lddo, m0n, m1n, tid);
        }
        __syncthreads();

        // mask (partial steps only, a workgroup-uniform branch): rows past m1
        // and invisible pairs get s = g = 0, hence P = dS = 0
        const bool full = uniform((m1 == m0 + BM) && (m1 <= sd.U) && key_tile_full &&
                                  (it.c0 + BN - 1 <= m0) &&
                                  ((m1 - 1 - it.c0 < p.k1) || (it.c0 + BN <= p.k2e))) != 0;
        // in terms of x = i - kj (element r of row block qb2 has x = x0 + c with
        // the constant c = 32*qb2 + 8*(r/4) + r%4): rows before m1 of a history
        // step see the key iff 0 <= x < W, W = m1 - kj, capped at K1 unless kj
        // is a prefix key; rows of a target step iff x < m1 - kj and (x == 0
        // or kj lies in row U's view)
        const int x0 = m0 + 4 * hl - kj;
        const bool tstep = m0 >= sd.U;
        int W = m1 - kj;
        if (!tstep && kj >= p.k2e) W = imin(W, p.k1);
        const uint32_t Wu = (uint32_t)imax(W, 0);
        const bool tv = !tstep || ((kj < sd.U) & ((sd.U - kj < p.k1) | (kj < p.k2e)));

        // stored-dS path: the slot of this key tile among the key tiles the
        // 64-row tile [m0, m1) visits (the order dQ reads them in)
        uint16_t *dsblk = nullptr;
        if (p.ds != nullptr) {
            const int rt = m0 < sd.U ? m0 / DS_BM : cdiv(sd.U, DS_BM) + (m0 - sd.U) / DS_BM;
            const int slot = s < DS_SLOT_TAB ? uniform((int)slot_tab[s])
                                             : uniform(step_slot(m0, m1));
            if (slot >= 0 && slot < p.ds_slots)
                dsblk = p.ds + (1 + ((int64_t)(rt_first + rt) * p.H + h) * p.ds_slots + slot) *
                                   (DS_BM * DS_BN);  // block 0 is the zero block
        }

        // per 32-row block (rows in the registers): S = Q K^T, dP = dO V^T,
        // then P and dS, then dV += P^T dO and dK += dS^T Q over its two
        // 16-row chunks; one block's S and dP are live at a time
#pragma unroll
        for (int qb2 = 0; qb2 < 2; ++qb2) {
            floatx16 sacc = zero16(), pacc = zero16();
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                bf16x8 aq = lds_row_chunk<D>(sq[buf], 32 * qb2 + l32, 2 * c + hl);
                sacc = mfma32(aq, kb[c], sacc);
                bf16x8 ag = lds_row_chunk<D>(sdo[buf], 32 * qb2 + l32, 2 * c + hl);
                pacc = mfma32(ag, vb[c], pacc);
            }
            if (!full) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int x = x0 + 32 * qb2 + 8 * (r >> 2) + (r & 3);
                    const bool vis = ((uint32_t)x < Wu) & (tv | (x == 0));
                    sacc[r] = vis ? sacc[r] : 0.0f;
                    pacc[r] = vis ? pacc[r] : 0.0f;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float sv = sacc[r], g = pacc[r];
                float e;
                const float sg = sigmoid_e(sv, nal2e, e);
                const float a = sv * sg;                       // SiLU(alpha s) / alpha
                sacc[r] = a;
                pacc[r] = g * (sg * (1.0f + alpha * a * e));  // G g SiLU'(t)
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int qc = 2 * qb2 + h2, o = 8 * h2;
                halfx8 pa = cvt8h(sacc[o], sacc[o + 1], sacc[o + 2], sacc[o + 3], sacc[o + 4],
                                  sacc[o + 5], sacc[o + 6], sacc[o + 7]);
                halfx8 da = cvt8h(pacc[o], pacc[o + 1], pacc[o + 2], pacc[o + 3], pacc[o + 4],
                                  pacc[o + 5], pacc[o + 6], pacc[o + 7]);
                if (dsblk != nullptr)
                    *reinterpret_cast<halfx8 *>(dsblk + 8 * ds_frag_chunk(wv, qc, l32, hl)) = da;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    halfx8 bg = lds_t_chunk_h(sdot[buf], 32 * db + l32, 2 * qc + hl);
                    dvacc[db] = mfma32h(pa, bg, dvacc[db]);
                    halfx8 bq = lds_t_chunk_h(sqt[buf], 32 * db + l32, 2 * qc + hl);
                    dkacc[db] = mfma32h(da, bq, dkacc[db]);
                }
            }
        }
    }

    // accumulator: lane holds column d = 32*db + l32, register r holds key
    // 32*wv + 8*(r/4) + 4*hl + r%4 of the tile
    if (it.nchunk == 1) {
        uint16_t *dkg = reinterpret_cast<uint16_t *>(p.dk) + sd.base * p.lddk + h * D;
        uint16_t *dvg = reinterpret_cast<uint16_t *>(p.dv) + sd.base * p.lddv + h * D;
        const float sk_ = p.out_scale / gscale, sv_ = sk_;  // both carry alpha / (N G)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = it.c0 + 32 * wv + 8 * (r >> 2) + 4 * hl + (r & 3);
                if (j < it.c1) {
                    __bf16 kv = (__bf16)(dkacc[db][r] * sk_);
                    __bf16 vv = (__bf16)(dvacc[db][r] * sv_);
                    dkg[(int64_t)j * p.lddk + 32 * db + l32] = __builtin_bit_cast(uint16_t, kv);
                    dvg[(int64_t)j * p.lddv + 32 * db + l32] = __builtin_bit_cast(uint16_t, vv);
                }
            }
        }
    } else {
        const int slot = p.s.part_base[b] + it.tile * nch + it.chunk;
        float *part = p.partials + ((int64_t)slot * p.H + h) * BN * (2 * D);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int jl = 32 * wv + 8 * (r >> 2) + 4 * hl + (r & 3);
                part[jl * (2 * D) + 32 * db + l32] = dkacc[db][r];
                part[jl * (2 * D) + D + 32 * db + l32] = dvacc[db][r];
            }
        }
    }
}

// Sum the chunk partials of each split prefix key tile in chunk order.  Block
// (item, slab) handles 1024 consecutive values of the [BN][2D] tile.
constexpr int RED_SLAB = 1024;

template <int D>
__global__ __launch_bounds__(256) void sla_bwd_reduce_kernel(AttnParams p)
{
    constexpr int BN = BWD_BN, W = 2 * D, SLABS = BN * W / RED_SLAB;
    const int nrec = p.s.red_base[p.B];
    const int item = blockIdx.x / SLABS, slab = blockIdx.x % SLABS;
    if (item >= nrec * p.H) return;
    const int h = item / nrec;
    const int rec = item - h * nrec;
    const int b = find_seq(p.s.red_base, p.B, rec);
    const SeqDims sd = seq_dims(p.offsets, p.num_targets, b);
    const int tile = rec - p.s.red_base[b];
    const int nch = p.s.nch[b];
    const int slot0 = p.s.part_base[b] + tile * nch;
    const int c0 = tile * BN, c1 = imin(c0 + BN, sd.L);
    const int e = slab * RED_SLAB + 4 * threadIdx.x;
    const int jl = e / W, col = e % W;
    if (c0 + jl >= c1) return;
    const float *src = p.partials + ((int64_t)slot0 * p.H + h) * BN * W + e;
    const int64_t stride = (int64_t)p.H * BN * W;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    int c = 0;
    for (; c + 4 <= nch; c += 4) {  // four loads in flight, added in chunk order
        const float4 v0 = *reinterpret_cast<const float4 *>(src + (c + 0) * stride);
        const float4 v1 = *reinterpret_cast<const float4 *>(src + (c + 1) * stride);
        const float4 v2 = *reinterpret_cast<const float4 *>(src + (c + 2) * stride);
        const float4 v3 = *reinterpret_cast<const float4 *>(src + (c + 3) * stride);
        acc.x += v0.x; acc.y += v0.y; acc.z += v0.z; acc.w += v0.w;
        acc.x += v1.x; acc.y += v1.y; acc.z += v1.z; acc.w += v1.w;
        acc.x += v2.x; acc.y += v2.y; acc.z += v2.z; acc.w += v2.w;
        acc.x += v3.x; acc.y += v3.y; acc.z += v3.z; acc.w += v3.w;
    }
    for (; c < nch; ++c) {
        const float4 v = *reinterpret_cast<const float4 *>(src + c * stride);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    const float sc = p.out_scale / *p.grad_scale;
    uint2 o = cvt4_u2(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
    uint16_t *dst = col < D
        ? reinterpret_cast<uint16_t *>(p.dk) + (sd.base + c0 + jl) * p.lddk + h * D + col
        : reinterpret_cast<uint16_t *>(p.dv) + (sd.base + c0 + jl) * p.lddv + h * D + (col - D);
    *reinterpret_cast<uint2 *>(dst) = o;
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void sla_bwd_dq_bf16_kernel(AttnParams p)
{
    constexpr int BM = FWD_BM, BN = FWD_BN;
    constexpr int NC = D / 16, NDB = D / 32;
    __shared__ __align__(16) uint16_t sk[2][BN * D];
    __shared__ __align__(16) uint16_t sv[2][BN * D];
    __shared__ __align__(16) uint16_t skt[2][D * BN];

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
    const uint16_t *gg = reinterpret_cast<const uint16_t *>(p.dout) + sd.base * p.lddo + h * D;

    // rows at or past r1 are zero, so their dS is zero
    const int qi = r0 + 32 * wv + l32;
    bf16x8 qb[NC], gb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        qb[c] = as_bf16x8(ld16_row(qg, p.ldq, qi, r1, 16 * c + 8 * hl));
        gb[c] = as_bf16x8(ld16_row(gg, p.lddo, qi, r1, 16 * c + 8 * hl));
    }

    const TileCursor cur(kr, BN);
    const int ntiles = uniform(cur.total);
    floatx16 dqacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dqacc[i] = zero16();

    Tile64<D> kt, vt;
    // keys at or past L hold copies of key L - 1; such tiles are never "full",
    // and the mask removes them
    int c_next = cur.start(0, BN);
    if (ntiles > 0) {
        kt.load_clamped(kg, p.ldk, c_next, sd.L, tid);
        vt.load_clamped(vg, p.ldv, c_next, sd.L, tid);
    }
    const float nal2e = p.neg_alpha_log2e, alpha = p.alpha;
    const float gscale = *p.grad_scale;
#pragma unroll
    for (int c = 0; c < NC; ++c) gb[c] = scale_bf16x8(gb[c], gscale);
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int c0 = uniform(c_next);
        kt.store_rows(sk[buf], tid);
        store_transposed_f16<D>(kt, skt[buf], tid, 1.0f);
        vt.store_rows(sv[buf], tid);
        c_next = cur.start(t + 1, BN);
        if (t + 1 < ntiles) {
            kt.load_clamped(kg, p.ldk, c_next, sd.L, tid);
            vt.load_clamped(vg, p.ldv, c_next, sd.L, tid);
        }
        __syncthreads();

        // S^T = K Q^T, dP^T = V dO^T (rows in the lane dimension)
        floatx16 sacc[2], pacc[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            sacc[kb2] = zero16();
            pacc[kb2] = zero16();
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                bf16x8 ak = lds_row_chunk<D>(sk[buf], 32 * kb2 + l32, 2 * c + hl);
                sacc[kb2] = mfma32(ak, qb[c], sacc[kb2]);
                bf16x8 av = lds_row_chunk<D>(sv[buf], 32 * kb2 + l32, 2 * c + hl);
                pacc[kb2] = mfma32(av, gb[c], pacc[kb2]);
            }
        }

        // mask (partial tiles only, a workgroup-uniform branch)
        const bool full = uniform((r0 < sd.U) && (c0 + BN <= sd.L) && (c0 + BN - 1 <= r0) &&
                                  ((r1 - 1 - c0 < p.k1) || (c0 + BN <= p.k2e))) != 0;
        if (!full) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = c0 + 32 * kb2 + 8 * (r >> 2) + 4 * hl + (r & 3);
                    const bool vis = visible(qi, j, sd.U, p.k1, p.k2e);
                    sacc[kb2][r] = vis ? sacc[kb2][r] : 0.0f;
                    pacc[kb2][r] = vis ? pacc[kb2][r] : 0.0f;
                }
            }
        }
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float s = sacc[kb2][r], g = pacc[kb2][r];
                float e;
                const float sg = sigmoid_e(s, nal2e, e);
                pacc[kb2][r] = g * (sg * (1.0f + alpha * s * sg * e));
            }
        }

        // dQ^T += K^T dS^T over four 16-key chunks
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const floatx16 &src = pacc[kc >> 1];
            const int o = 8 * (kc & 1);
            halfx8 dsb = cvt8h(src[o], src[o + 1], src[o + 2], src[o + 3], src[o + 4],
                               src[o + 5], src[o + 6], src[o + 7]);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                halfx8 a = lds_t_chunk_h(skt[buf], 32 * db + l32, 2 * kc + hl);
                dqacc[db] = mfma32h(a, dsb, dqacc[db]);
            }
        }
    }

    if (qi < r1) {
        uint16_t *orow = reinterpret_cast<uint16_t *>(p.dq) + (sd.base + qi) * p.lddq + h * D;
        const float sc = p.out_scale / gscale;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 v = cvt4_u2(dqacc[db][4 * g] * sc, dqacc[db][4 * g + 1] * sc,
                                  dqacc[db][4 * g + 2] * sc, dqacc[db][4 * g + 3] * sc);
                *reinterpret_cast<uint2 *>(orow + 32 * db + 8 * g + 4 * hl) = v;
            }
        }
    }
}

template <int D>
static hipError_t launch_dkdv_d(const AttnParams &p, hipStream_t st)
{
    hipLaunchKernelGGL(sla_bwd_dkdv_bf16_kernel<D>, dim3(p.grid_bwd), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.grid_red == 0) return e;
    hipLaunchKernelGGL(sla_bwd_reduce_kernel<D>, dim3(p.grid_red * (BWD_BN * 2 * D / RED_SLAB)),
                       dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const AttnParams &p, hipStream_t st)
{
    switch (p.d) {
    case 32: return launch_dkdv_d<32>(p, st);
    case 64: return launch_dkdv_d<64>(p, st);
    case 128: return launch_dkdv_d<128>(p, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_dq_bf16(const AttnParams &p, hipStream_t st)
{
    if (p.ds != nullptr) return launch_bwd_dq_ds_bf16(p, st);
    dim3 grid(p.grid_fwd), block(256);
    switch (p.d) {
    case 32: hipLaunchKernelGGL(sla_bwd_dq_bf16_kernel<32>, grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL(sla_bwd_dq_bf16_kernel<64>, grid, block, 0, st, p); break;
    case 128: hipLaunchKernelGGL(sla_bwd_dq_bf16_kernel<128>, grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sla
