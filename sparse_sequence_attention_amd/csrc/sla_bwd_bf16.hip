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
#include <type_traits>

#include "sla_device.h"
#include "sla_kernels.h"
#include "sla_tiles.h"

namespace sla {

constexpr int DS_SLOT_TAB = 512;  // steps of a dK/dV item whose dS slot is tabulated

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
// 16-byte chunk swizzle of the fp16 [64][D] Q / G dO tiles of the dK/dV
// kernel: logical chunk c of row r sits at c ^ hswz<D>(r).  With u = r*D/128
// (the 256-byte bank row) and Q4 = D/32, hswz = 4*(u % Q4) + (u / Q4) % 4:
// the 16 rows that a 16-lane pass of a 16-byte read touches, and the 4 rows x
// 64 bytes that a 32-lane pass of a transposing read touches, fall in
// distinct banks (gfx950 serves ds_read_b128 16 lanes and ds_read_b64_tr_b16
// 32 lanes at a time).
template <int D>
__device__ __forceinline__ int hswz(int r)
{
    constexpr int Q4 = D / 32;
    const int u = r * D / 128;
    return 4 * (u % Q4) + (u / Q4) % 4;
}

constexpr int DKDV_THREADS = 512;

template <int D>
__global__ __launch_bounds__(DKDV_THREADS, 1) void sla_bwd_dkdv_bf16_kernel(AttnParams p)
{
    constexpr int BN = BWD_BN, BM = BWD_BM;
    constexpr int NT = DKDV_THREADS;
    constexpr int NC = D / 16, NDB = D / 32, CPR = D / 8;
    constexpr int TILE = BM * D;             // elements of one staged 64-row tile
    constexpr int TCH = BM * CPR;            // 16-byte chunks of one staged tile
    constexpr int KVS = D + 8;               // padded K / V row: 16-byte reads of 16
                                             // consecutive keys hit distinct banks
    static_assert(BM == 64 && BN == 128, "64-row steps over 128-key tiles");
    // kv: K then V of the key tile (fp16, padded rows).  cs0 / cs1: two
    // stages of Q and G dO rows (swizzled); the DMA brings a step's bf16 rows
    // into one stage while the other is read, and each thread then converts
    // its own chunks in place to fp16.  Separate arrays, so that the compiler
    // can tell the DMA into one stage from the reads of the other.
    __shared__ __align__(16) uint16_t kv[2 * BN * KVS];
    __shared__ __align__(16) uint16_t cs0[2 * TILE], cs1[2 * TILE];
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

    // 8 waves: wave w owns keys 32*(w%4) .. +32 of the tile and rows
    // 32*(w/4) .. +32 of every 64-row step; the two row halves of a key block
    // add their dK/dV sums at the end.  Two waves per SIMD.
    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int kw = wv & 3, rh = wv >> 2;
    const int l32 = lane & 31, hl = lane >> 5;
    const int kj = it.c0 + 32 * kw + l32;  // this lane's key (operands, mask)

    const uint16_t *qg = reinterpret_cast<const uint16_t *>(p.q) + sd.base * p.ldq + h * D;
    const uint16_t *kg = reinterpret_cast<const uint16_t *>(p.k) + sd.base * p.ldk + h * D;
    const uint16_t *vg = reinterpret_cast<const uint16_t *>(p.v) + sd.base * p.ldv + h * D;
    const uint16_t *gg = reinterpret_cast<const uint16_t *>(p.dout) + sd.base * p.lddo + h * D;

    // K and V of the tile into LDS as fp16 (keys past c1 as zeros); the first
    // chunk of a key tile also writes the fp16 copy of K that dQ = dS K reads
    // on the stored-dS path
    const bool write_kh = p.kh != nullptr && it.chunk == 0;
    for (int i = tid; i < BN * CPR; i += NT) {
        const int key = i / CPR, c = i % CPR;
        const halfx8 kh8 = bf16x8_to_halfx8(as_bf16x8(ld16_row(kg, p.ldk, it.c0 + key, it.c1, 8 * c)));
        const halfx8 vh8 = bf16x8_to_halfx8(as_bf16x8(ld16_row(vg, p.ldv, it.c0 + key, it.c1, 8 * c)));
        *reinterpret_cast<halfx8 *>(kv + key * KVS + 8 * c) = kh8;
        *reinterpret_cast<halfx8 *>(kv + (BN + key) * KVS + 8 * c) = vh8;
        if (write_kh && it.c0 + key < it.c1)
            *reinterpret_cast<halfx8 *>(p.kh + (sd.base + it.c0 + key) * ((int64_t)p.H * D) +
                                        h * D + 8 * c) = kh8;
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
    const int nsteps = uniform(nh + nt);
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
        for (int st = tid; st < imin(nsteps, DS_SLOT_TAB); st += NT) {
            int a0, a1;
            step_rows(st, a0, a1);
            slot_tab[st] = (int16_t)step_slot(a0, a1);
        }
    }

    const float nal2e = p.neg_alpha_log2e, alpha = p.alpha;
    const float gscale = *p.grad_scale;
    const bool key_tile_full = (it.c1 - it.c0 == BN);

    // Staging is done by the rh = 0 waves alone: the SIMD issues the older
    // wave of a pair first, so these finish their products earlier and would
    // otherwise wait at the barrier.  Staging thread t (< NS) owns chunks
    // P = i*NS + t of a stage: physical chunk P % CPR of row (P % TCH) / CPR
    // of tile P / TCH (0: Q, 1: dO); the DMA fills it with logical chunk
    // (P % CPR) ^ hswz(row) and the same thread converts it in place.
    constexpr int NS = NT / 2;            // staging threads
    constexpr int SPS = 2 * TCH / NS;     // DMA loads per staging thread and step
    static_assert(TCH % NS == 0 && SPS <= 8, "whole DMA rounds, at most 8 per thread");
    auto chunk_tile = [&](int i) { return (i * NS) / TCH; };
    auto stage = [&](auto S) -> uint16_t * {
        if constexpr (decltype(S)::value == 0) return cs0;
        else return cs1;
    };
    // DMA of the bf16 rows of step t (clamped to the last step) into a stage:
    // a workgroup-uniform row base plus a 32-bit per-lane offset; rows at or
    // past m1 read row m1 - 1 (masked: such steps are never full)
    const uint32_t ldq_b = (uint32_t)p.ldq * 2u, lddo_b = (uint32_t)p.lddo * 2u;
    auto issue = [&](int t, auto S) {
        int m0, m1;
        step_rows(imin(t, nsteps - 1), m0, m1);
        m0 = uniform(m0);
        const int last = uniform(m1 - 1 - m0);
        const char *qrow = reinterpret_cast<const char *>(qg + (int64_t)m0 * p.ldq);
        const char *grow = reinterpret_cast<const char *>(gg + (int64_t)m0 * p.lddo);
        uint16_t *sb = stage(S);
#pragma unroll
        for (int i = 0; i < SPS; ++i) {
            const int P = i * NS + wv * 64 + lane;
            const int tile = chunk_tile(i);
            const int prow = (P % TCH) / CPR;
            const uint32_t row = (uint32_t)imin(prow, last);
            const uint32_t c = (uint32_t)((P % CPR) ^ hswz<D>(prow));
            const char *src = tile == 0 ? qrow + (row * ldq_b + 16u * c) : grow + (row * lddo_b + 16u * c);
            gl_lds16(src, sb + (i * NS + wv * 64) * 8);
        }
    };
    // this thread's chunks of a stage, bf16 -> fp16 in place (dO times G)
    auto convert = [&](auto S) {
        uint16_t *sb = stage(S);
        uint4 raw[SPS];
#pragma unroll
        for (int i = 0; i < SPS; ++i) raw[i] = *reinterpret_cast<const uint4 *>(sb + 8 * (i * NS + wv * 64 + lane));
#pragma unroll
        for (int i = 0; i < SPS; ++i) {
            const float sc = chunk_tile(i) == 0 ? 1.0f : gscale;
            const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
            const halfx8 hv = cvt8h(bf16_lo(w[0]) * sc, bf16_hi(w[0]) * sc, bf16_lo(w[1]) * sc,
                                    bf16_hi(w[1]) * sc, bf16_lo(w[2]) * sc, bf16_hi(w[2]) * sc,
                                    bf16_lo(w[3]) * sc, bf16_hi(w[3]) * sc);
            *reinterpret_cast<halfx8 *>(sb + 8 * (i * NS + wv * 64 + lane)) = hv;
        }
    };

    // per-lane LDS offsets (elements).  Row operands: row ar = 32*rh + l32 of
    // a staged tile (logical chunk 2c + hl) and key row br = 32*kw + l32 of
    // K / V.  Transposing reads (quarter q = lane/16, j = lane%16): rows
    // 32*rh + 16*h2 + 8*rr + 4*(q/2) + j/4, columns 32*db + 16*(q%2) + 4*(j%4).
    const int ar = 32 * rh + l32, br = 32 * kw + l32;
    const int q4 = lane >> 4, j16 = lane & 15;
    auto a_off = [&](int c) { return ar * D + 8 * ((2 * c + hl) ^ hswz<D>(ar)); };
    const int b_base = br * KVS + 8 * hl;  // + 16 c (K), + BN*KVS (V)
    auto t_off = [&](int h2, int rr, int db) {
        const int row = 32 * rh + 16 * h2 + 8 * rr + 4 * (q4 >> 1) + (j16 >> 2);
        const int col = 32 * db + 16 * (q4 & 1) + 4 * (j16 & 3);
        return row * D + 8 * ((col >> 3) ^ hswz<D>(row)) + (col & 7);
    };

    floatx16 dkacc[NDB], dvacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
        dkacc[i] = zero16();
        dvacc[i] = zero16();
    }

    // step t in stage S: publish the stage (converted by every thread) with
    // a barrier that also frees the other stage (read by step t - 1), start
    // the DMA of step t + 1 into it, compute S, dP, P, dS, dV and dK, then
    // wait for that DMA and convert this thread's share of it in place.  One
    // barrier per step; it waits for LDS only, so the DMA stays in flight.
    auto step = [&](int t, auto S, auto HAS_DS) {
        constexpr int sidx = decltype(S)::value;
        constexpr bool has_ds = decltype(HAS_DS)::value;
        barrier_lds();
        if (rh == 0) issue(t + 1, std::integral_constant<int, 1 - sidx>{});
        const uint16_t *sq = stage(S), *sg = stage(S) + TILE;
        int m0, m1;
        step_rows(t, m0, m1);
        m0 = uniform(m0);
        m1 = uniform(m1);

        // mask (partial steps only, a workgroup-uniform branch): rows past m1
        // and invisible pairs get s = g = 0, hence P = dS = 0.  In terms of
        // x = i - kj (register r has x = x0 + 8*(r/4) + r%4): rows before m1
        // of a history step see the key iff 0 <= x < W, W = m1 - kj, capped
        // at K1 unless kj is a prefix key; rows of a target step iff
        // x < m1 - kj and (x == 0 or kj lies in row U's view)
        const bool full = uniform((m1 == m0 + BM) && (m1 <= sd.U) && key_tile_full &&
                                  (it.c0 + BN - 1 <= m0) &&
                                  ((m1 - 1 - it.c0 < p.k1) || (it.c0 + BN <= p.k2e))) != 0;
        const int x0 = m0 + 32 * rh + 4 * hl - kj;
        const bool tstep = m0 >= sd.U;
        int W = m1 - kj;
        if (!tstep && kj >= p.k2e) W = imin(W, p.k1);
        const uint32_t Wu = (uint32_t)imax(W, 0);
        const bool tv = !tstep || ((kj < sd.U) & ((sd.U - kj < p.k1) | (kj < p.k2e)));

        // S = Q K^T and G dP = (G dO) V^T for this wave's 32 rows x 32 keys
        floatx16 sacc = zero16(), pacc = zero16();
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const halfx8 aq = *reinterpret_cast<const halfx8 *>(sq + a_off(c));
            const halfx8 bk = *reinterpret_cast<const halfx8 *>(kv + b_base + 16 * c);
            sacc = mfma32h(aq, bk, sacc);
            const halfx8 ag = *reinterpret_cast<const halfx8 *>(sg + a_off(c));
            const halfx8 bv = *reinterpret_cast<const halfx8 *>(kv + BN * KVS + b_base + 16 * c);
            pacc = mfma32h(ag, bv, pacc);
        }
        if (!full) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int x = x0 + 8 * (r >> 2) + (r & 3);
                const bool vis = ((uint32_t)x < Wu) & (tv | (x == 0));
                sacc[r] = vis ? sacc[r] : 0.0f;
                pacc[r] = vis ? pacc[r] : 0.0f;
            }
        }
        // P = s sigma (= SiLU(t) / alpha) and G dS = G g sigma (1 + t (1 - sigma))
        // = G g (sigma + a * (alpha - alpha sigma)).  exp(-t) overflowing to
        // inf gives sigma = 0, a = 0 and dS = 0, its limit, with no NaN.
        float sgv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float sv = sacc[r];
            const float sgm = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sv * nal2e));
            sgv[r] = sgm;
            sacc[r] = sv * sgm;
        }
        halfx8 pa[2], da[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int o = 8 * h2;
            pa[h2] = cvt8h(sacc[o], sacc[o + 1], sacc[o + 2], sacc[o + 3], sacc[o + 4], sacc[o + 5],
                           sacc[o + 6], sacc[o + 7]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            pacc[r] = pacc[r] * fmaf(sacc[r], fmaf(-alpha, sgv[r], alpha), sgv[r]);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int o = 8 * h2;
            da[h2] = cvt8h(pacc[o], pacc[o + 1], pacc[o + 2], pacc[o + 3], pacc[o + 4], pacc[o + 5],
                           pacc[o + 6], pacc[o + 7]);
        }
        // dV += P^T (G dO), dK += (G dS)^T Q over the two 16-row chunks; the
        // accumulator's row order (8*(r/4) + 4*hl + r%4) is the k order of
        // the transposing reads
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const uint2 g0 = tr_read_b64(sg + t_off(h2, 0, db));
                const uint2 g1 = tr_read_b64(sg + t_off(h2, 1, db));
                dvacc[db] = mfma32h(pa[h2], __builtin_bit_cast(halfx8, make_uint4(g0.x, g0.y, g1.x, g1.y)),
                                    dvacc[db]);
            }
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const uint2 q0 = tr_read_b64(sq + t_off(h2, 0, db));
                const uint2 q1 = tr_read_b64(sq + t_off(h2, 1, db));
                dkacc[db] = mfma32h(da[h2], __builtin_bit_cast(halfx8, make_uint4(q0.x, q0.y, q1.x, q1.y)),
                                    dkacc[db]);
            }
        }
        // schedule: P first (5 VALU per element and its conversion), then
        // the dV products with dS (3 VALU per element) issued between them,
        // so that the MFMA pipe and the VALU work at the same time, then dK
        __builtin_amdgcn_sched_group_barrier(SG_VALU, 88, 0);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 4, 0);
#pragma unroll
        for (int i = 0; i < 2 * NDB; ++i) {
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
            __builtin_amdgcn_sched_group_barrier(SG_VALU, 7, 0);
        }
#pragma unroll
        for (int i = 0; i < 2 * NDB; ++i) {
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            if (i < 2 * NDB - 2) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
        }
        // the next stage (its DMA was issued at the top of this step) while
        // the products run, then this step's dS stores: the next wait, a step
        // later, finds both the next DMA and these stores long issued
        if (rh == 0) {
            vm_wait<0>();
            convert(std::integral_constant<int, 1 - sidx>{});
        }
        // stored-dS path: the block of this key tile's slot among the key
        // tiles the 64-row tile [m0, m1) visits (the order dQ reads them
        // in), or the discard block; streamed out (dQ reads it back from HBM
        // after this kernel)
        if constexpr (has_ds) {
            const int rt = m0 < sd.U ? m0 / DS_BM : cdiv(sd.U, DS_BM) + (m0 - sd.U) / DS_BM;
            const int slot = t < DS_SLOT_TAB ? uniform((int)slot_tab[t])
                                             : uniform(step_slot(m0, m1));
            const int64_t blk = (slot >= 0 && slot < p.ds_slots)
                                    ? 1 + ((int64_t)(rt_first + rt) * p.H + h) * p.ds_slots + slot
                                    : p.ds_discard;  // block 0 is the zero block
            uint16_t *dsblk = p.ds + blk * (DS_BM * DS_BN);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
                st16_nt(dsblk + 8 * ds_frag_chunk(kw, 2 * rh + h2, l32, hl), da[h2]);
        }
    };
    // the step loop, compiled once with and once without the dS stores so
    // that the stores are unconditional where they exist; two steps per
    // iteration so that each stage's addresses are compile-time
    auto run = [&](auto HAS_DS) {
        if (nsteps == 0) return;
        if (rh == 0) {
            issue(0, std::integral_constant<int, 0>{});
            vm_wait<0>();
            convert(std::integral_constant<int, 0>{});
        }
        for (int t = 0; t < nsteps; t += 2) {
            step(t, std::integral_constant<int, 0>{}, HAS_DS);
            if (t + 1 < nsteps) step(t + 1, std::integral_constant<int, 1>{}, HAS_DS);
        }
        vm_wait<0>();  // no DMA (of the clamped step past the end) left in flight
    };
    if (p.ds != nullptr) run(std::true_type{});
    else run(std::false_type{});

    // the two row halves of key block kw: the rh = 1 wave hands its dK sum to
    // the rh = 0 wave and takes the rh = 0 wave's dV sum, through LDS (free
    // after the barrier); region e holds 32 keys x D floats
    __syncthreads();
    auto region = [&](int e) -> float * {
        // kv holds regions 0-3, cs0 4-5, cs1 6-7
        uint16_t *a = e < 4 ? kv + (e & 3) * (64 * D) : (e < 6 ? cs0 : cs1) + (e & 1) * (64 * D);
        return reinterpret_cast<float *>(a);
    };
    floatx16 *mine = rh == 0 ? dkacc : dvacc;    // the sum this wave writes out
    floatx16 *other = rh == 0 ? dvacc : dkacc;   // the sum it hands over
    {
        float *xo = region(2 * kw + (1 - rh));
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64 + lane] = other[db][r];
    }
    __syncthreads();
    {
        const float *xi = region(2 * kw + rh);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) mine[db][r] += xi[(db * 16 + r) * 64 + lane];
    }

    // accumulator: lane holds column d = 32*db + l32, register r holds key
    // 32*kw + 8*(r/4) + 4*hl + r%4 of the tile; dV (P carries 1/alpha) and dK
    // both scale by alpha / (N G)
    const float sc = p.out_scale / gscale;
    if (it.nchunk == 1) {
        uint16_t *dst = rh == 0 ? reinterpret_cast<uint16_t *>(p.dk) + sd.base * p.lddk + h * D
                                : reinterpret_cast<uint16_t *>(p.dv) + sd.base * p.lddv + h * D;
        const int64_t ld = rh == 0 ? p.lddk : p.lddv;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = it.c0 + 32 * kw + 8 * (r >> 2) + 4 * hl + (r & 3);
                if (j < it.c1) {
                    const __bf16 v = (__bf16)(mine[db][r] * sc);
                    dst[(int64_t)j * ld + 32 * db + l32] = __builtin_bit_cast(uint16_t, v);
                }
            }
        }
    } else {
        // fp32 partials [key][dK | dV] of this chunk
        const int slot = p.s.part_base[b] + it.tile * nch + it.chunk;
        float *part = p.partials + ((int64_t)slot * p.H + h) * BN * (2 * D) + rh * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int jl = 32 * kw + 8 * (r >> 2) + 4 * hl + (r & 3);
                part[jl * (2 * D) + 32 * db + l32] = mine[db][r];
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
    hipLaunchKernelGGL(sla_bwd_dkdv_bf16_kernel<D>, dim3(p.grid_bwd), dim3(DKDV_THREADS), 0, st,
                       p);
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
