// sla_bwd_bf16.hip -- SLA backward dK / dV on gfx950: bf16 MFMA, fp32
// accumulation, no atomics.
//
// With a_ij = SiLU(alpha s_ij), s_ij = q_i . k_j, O_i = (1/N) sum_j a_ij v_j
// (ULTRA-HSTU paper, section 3 Eq.3 under the semi-local mask of section
// 4.2.1 Eq.7), the chain rule gives, over visible pairs,
//   dV_j = (1/N) sum_i a_ij dO_i
//   dS_ij = (alpha/N) (dO_i . v_j) sigma_ij (1 + t_ij (1 - sigma_ij)),  t = alpha s
//   dK_j = sum_i dS_ij q_i.
// The kernel keeps s*sigma and g*sigma*(1 + t(1 - sigma)) (g = dO.v) as MFMA
// operands and applies alpha/N once in the epilogue.
//
// Ownership (the key-parallel half of the KV- / Q-parallel backward split the
// WHALE notes describe; dQ is sla_dq.hip's row-parallel kernel): a workgroup
// owns a 128-key tile of one head and walks the 64-row steps of the rows that
// see it.  Global-prefix key tiles are seen by every later row, so they are
// cut into row chunks whose fp32 partial sums a second kernel adds in chunk
// order: results are bitwise reproducible.
//
// Layout: eight waves, two per SIMD.  The bf16 K and V rows of the key tile
// sit in LDS for the whole item (64 KB at d = 128); the Q and dO rows of the
// 64-row steps come HBM -> LDS by DMA into a ring of three stages (96 KB),
// two steps ahead, with one LDS-only barrier per step.  Wave w owns keys
// 32 (w % 4) .. + 32 and rows 32 (w / 4) .. + 32 of each step:
//   S  (32 rows x 32 keys) = Q K^T,  dP = dO V^T      row operands from LDS
//   P, dS in registers (masked only on steps that cross the mask's edges)
//   dV (32 keys x D) += P^T dO,  dK += dS^T Q          transposing LDS reads
// and the two row halves of a key block add their dK / dV sums through LDS
// at the end.  The steps that need no mask (full 64-row history steps that
// see every key of the tile) run as one branch-free loop between the masked
// steps before and after them.
//
// Precision.  Q.K^T and dO.V^T take the bf16 inputs as stored.  The computed
// operands of dV = P^T dO and dK = dS^T Q are rounded to bf16 (8 significant
// bits); their rounding errors are independent across the rows a key sums
// over.  The keys of the global prefix are seen by every row of the sequence,
// so their dK and dV are sums of up to L terms and the largest values of the
// two tensors (tens of times their rms at 16K-token histories); there P and
// dS enter the products as the sum of two bf16 numbers, hi = bf16(x) and
// lo = bf16(x - hi) (16 significant bits), at the price of a second MFMA per
// product on those key tiles only.
#include <type_traits>

#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

// 16-byte chunk swizzle of the bf16 [64][D] Q / dO stage tiles: logical chunk
// c of row r sits at c ^ hswz<D>(r).  With u = r*D/128 (the 256-byte bank row)
// and Q4 = D/32, hswz = 4*(u % Q4) + (u / Q4) % 4: the 16 rows that a 16-lane
// pass of a 16-byte read touches, and the 4 rows x 64 bytes that a 32-lane
// pass of a transposing read touches, fall in distinct banks.
template <int D>
__device__ __forceinline__ int hswz(int r)
{
    // unsigned bit operations: the compiler then sees that adding a multiple
    // of 32 rows (the second row block) leaves the swizzle unchanged
    constexpr unsigned Q4 = D / 32;
    const unsigned u = ((unsigned)r * D) >> 7;
    return (int)(4u * (u & (Q4 - 1)) + ((u / Q4) & 3u));
}

constexpr int DKDV_THREADS = 512;
constexpr int DKDV_STAGES = 3;

// x - float(hi) for the 8 values of hi = bf16(x), rounded to bf16: the low
// part of the two-term bf16 representation x ~ hi + lo
__device__ __forceinline__ bf16x8 lo_part(const float *x, const bf16x8 &hi)
{
    const uint4 u = as_u4(hi);
    return cvt8(x[0] - bf16_lo(u.x), x[1] - bf16_hi(u.x), x[2] - bf16_lo(u.y), x[3] - bf16_hi(u.y),
                x[4] - bf16_lo(u.z), x[5] - bf16_hi(u.z), x[6] - bf16_lo(u.w), x[7] - bf16_hi(u.w));
}

// DQK: the Q / K (and dK) head width, DV: the V, dO (and dV) width.
// STORE_DS: also write the bf16 dS of every step (the operand of the dK
// product, as each wave holds it) for the dQ kernel to read back.
template <int DQK, int DV, bool OUTF32, bool STORE_DS>
__global__ __launch_bounds__(DKDV_THREADS, 1) void sla_bwd_dkdv_bf16_kernel(AttnParams p)
{
    constexpr int BN = BWD_BN, BM = BWD_BM;
    constexpr int NT = DKDV_THREADS;
    constexpr int NC = DQK / 16, NCV = DV / 16;     // 16-wide chunks of Q.K, dO.V
    constexpr int NDB = DQK / 32, NDBV = DV / 32;   // 32-wide blocks of dK, dV
    constexpr int CPR = DQK / 8, CPRV = DV / 8;     // 16-byte chunks per Q / K, dO / V row
    constexpr int DW = DQK + DV;                    // a [Q | dO] or [K | V] row pair
    constexpr int TCH = BM * CPR, TCHV = BM * CPRV; // chunks of a staged Q, dO tile
    constexpr int SPS = (TCH + TCHV + NT - 1) / NT; // DMA loads per thread and step
    // chunk slots of a stage: [Q | dO], then, when the two tiles do not make
    // whole DMA rounds, padding that the surplus loads fill
    constexpr int SLOTS = SPS * NT;
    constexpr int KCH = BN * CPR, KCHV = BN * CPRV; // chunks of the K, V tile
    constexpr int KPT = (KCH + KCHV) / NT;          // DMA loads per thread of the K and V tiles
    constexpr int NST = DKDV_STAGES;
    static_assert(BM == 64 && BN == 128, "64-row steps over 128-key tiles");
    static_assert(SPS <= 8, "at most 8 DMA loads per thread and step");
    static_assert(TCH % 64 == 0 && TCHV % 64 == 0 && KCH % NT == 0,
                  "the Q / dO / padding and K / V splits are wave-uniform");
    static_assert((KCH + KCHV) % NT == 0 && KPT <= 8, "whole DMA rounds of the key tile");
    // [K | V] of the key tile (bf16, swizzled rows), then a ring of NST stages
    // of [Q | dO] rows filled by DMA NST - 1 steps ahead: 64 + 96 KB at d = 128
    __shared__ __align__(16) uint16_t lds[BN * DW + NST * SLOTS * 8];
    uint16_t *const kvs = lds;
    uint16_t *const ring = lds + BN * DW;

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

    // 8 waves, two per SIMD: wave w owns keys 32*(w%4) .. +32 of the tile and
    // rows 32*(w/4) .. +32 of every 64-row step; the two row halves of a key
    // block add their dK/dV sums at the end (fixed order, deterministic).
    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int kw = wv & 3, rh = wv >> 2;
    const int l32 = lane & 31, hl = lane >> 5;
    const int kj = it.c0 + 32 * kw + l32;  // this lane's key (mask)

    const uint16_t *qg = reinterpret_cast<const uint16_t *>(p.q) + sd.base * p.ldq + h * DQK;
    const uint16_t *kg = reinterpret_cast<const uint16_t *>(p.k) + sd.base * p.ldk + h * DQK;
    const uint16_t *vg = reinterpret_cast<const uint16_t *>(p.v) + sd.base * p.ldv + h * DV;
    const uint16_t *gg = reinterpret_cast<const uint16_t *>(p.dout) + sd.base * p.lddo + h * DV;

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
    // Stored dS: the blocks of a key tile are its 64-row steps over all its
    // chunks, history steps first; item step t is block t + ds_dh (history)
    // or t + ds_dt (targets) of the tile.  Wave wv writes bytes
    // 2048 wv .. + 2048 of a block: for h2 = 0, 1, lane l's 16 bytes at
    // 1024 h2 + 16 l (the bf16 A fragment of its dK product).
    uint8_t *ds_wave = nullptr;
    int ds_dh = 0, ds_dt = 0;
    if constexpr (STORE_DS) {
        const TileSteps ts = tile_steps(sd.L, sd.U, p.k1, p.k2e, it.c0, it.c1, BM);
        const int gtile = uniform(p.s.ktile_base[b]) + it.c0 / BN;
        const int64_t blk0 = (int64_t)h * p.ds_head_blocks + uniform(p.s.ds_base[gtile]);
        ds_dh = uniform(h_first - ts.h_first);
        ds_dt = uniform(ts.nh + t_first - nh - ts.t_first);
        ds_wave = p.ds + blk0 * DS_BLOCK_BYTES + wv * 2048;
    }
    auto step_rows = [&](int s, int &m0, int &m1) __attribute__((always_inline)) {
        const bool hist = s < nh;
        m0 = hist ? (h_first + s) * BM : sd.U + (t_first + s - nh) * BM;
        m1 = imin(m0 + BM, hist ? sd.U : sd.L);
    };
    // A full step needs no mask: 64 history rows, all of which see every key
    // of a whole key tile.  Such steps form one run [s_lo, s_hi) (rows from
    // the diagonal on, up to the end of the window or of the history); the
    // steps before and after it run the masked body.
    const bool key_tile_full = (it.c1 - it.c0 == BN);
    auto is_full = [&](int s) __attribute__((always_inline)) {
        int m0, m1;
        step_rows(s, m0, m1);
        return (m1 == m0 + BM) && (m1 <= sd.U) && key_tile_full && (it.c0 + BN - 1 <= m0) &&
               ((m1 - 1 - it.c0 < p.k1) || (it.c0 + BN <= p.k2e));
    };
    int s_lo = 0;
    while (s_lo < nsteps && !is_full(s_lo)) ++s_lo;
    int s_hi = s_lo;
    while (s_hi < nsteps && is_full(s_hi)) ++s_hi;
    s_lo = uniform(s_lo);
    s_hi = uniform(s_hi);

    const float nal2e = p.neg_alpha_log2e, alpha = p.alpha;

    // DMA (gl_lds16_at: the kernel's own waits and barriers order it
    // against the reads).  Thread t owns chunks P = i*NT + t of the [K | V]
    // (or [Q | dO]) pair, K (Q) first: chunk P' of a tile of row width w is
    // physical chunk P' % (w/8) of row P' / (w/8), filled with logical chunk
    // (P' % (w/8)) ^ hswz<w>(row).  Key rows at or past c1 read
    // row c1 - 1 (keys never stored); step rows at or past m1 read row m1 - 1
    // (masked: such steps are never full).  Every step issues exactly SPS
    // loads per thread, so the wait counts are static.
    // wave-uniform LDS byte addresses of this wave's DMA destinations
    const uint32_t kv_lds = uniform((int)(lds_addr(kvs) + 16u * (uint32_t)(wv * 64)));
    const uint32_t ring_lds = uniform((int)(lds_addr(ring) + 16u * (uint32_t)(wv * 64)));
    auto issue_kv = [&]() __attribute__((always_inline)) {
        const int last = uniform(it.c1 - 1 - it.c0);
        const char *krow = reinterpret_cast<const char *>(kg + (int64_t)it.c0 * p.ldk);
        const char *vrow = reinterpret_cast<const char *>(vg + (int64_t)it.c0 * p.ldv);
        const uint32_t ldk_b = (uint32_t)p.ldk * 2u, ldv_b = (uint32_t)p.ldv * 2u;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int P = i * NT + wv * 64 + lane;
            const char *src;
            if constexpr (DQK == DV) {
                const int tile = P / KCH;  // K or V (uniform per wave)
                const int prow = (P % KCH) / CPR;
                const uint32_t row = (uint32_t)imin(prow, last);
                const uint32_t c = (uint32_t)((P % CPR) ^ hswz<DQK>(prow));
                src = tile == 0 ? krow + (row * ldk_b + 16u * c) : vrow + (row * ldv_b + 16u * c);
            } else if (i * NT < KCH) {  // K (whole rounds: KCH is a multiple of NT)
                const int prow = P / CPR;
                const uint32_t row = (uint32_t)imin(prow, last);
                const uint32_t c = (uint32_t)((P % CPR) ^ hswz<DQK>(prow));
                src = krow + (row * ldk_b + 16u * c);
            } else {
                const int Pv = P - KCH;
                const int prow = Pv / CPRV;
                const uint32_t row = (uint32_t)imin(prow, last);
                const uint32_t c = (uint32_t)((Pv % CPRV) ^ hswz<DV>(prow));
                src = vrow + (row * ldv_b + 16u * c);
            }
            gl_lds16_at(src, kv_lds + 16u * (uint32_t)(i * NT));
        }
    };
    const uint32_t ldq_b = (uint32_t)p.ldq * 2u, lddo_b = (uint32_t)p.lddo * 2u;
    auto issue = [&](int t) __attribute__((always_inline)) {
        int m0, m1;
        step_rows(imin(t, nsteps - 1), m0, m1);
        m0 = uniform(m0);
        const int last = uniform(m1 - 1 - m0);
        const char *qrow = reinterpret_cast<const char *>(qg + (int64_t)m0 * p.ldq);
        const char *grow = reinterpret_cast<const char *>(gg + (int64_t)m0 * p.lddo);
        const uint32_t sb = ring_lds + (uint32_t)(t % NST) * (16u * SLOTS);
#pragma unroll
        for (int i = 0; i < SPS; ++i) {
            const int P = i * NT + wv * 64 + lane;
            const char *src;
            if constexpr (DQK == DV) {
                const int tile = P / TCH;  // Q or dO (uniform per wave)
                const int prow = (P % TCH) / CPR;
                const uint32_t row = (uint32_t)imin(prow, last);
                const uint32_t c = (uint32_t)((P % CPR) ^ hswz<DQK>(prow));
                src = tile == 0 ? qrow + (row * ldq_b + 16u * c) : grow + (row * lddo_b + 16u * c);
            } else if ((TCH % NT == 0) ? (i * NT < TCH) : (P < TCH)) {
                // Q or dO: whole rounds when TCH is a multiple of NT, else
                // uniform per wave (TCH is a multiple of 64)
                const int prow = P / CPR;
                const uint32_t row = (uint32_t)imin(prow, last);
                const uint32_t c = (uint32_t)((P % CPR) ^ hswz<DQK>(prow));
                src = qrow + (row * ldq_b + 16u * c);
            } else if (P >= TCH + TCHV) {
                src = qrow;  // padding: Q's first chunk into the stage's spare slots
            } else {
                const int Pg = P - TCH;
                const int prow = Pg / CPRV;
                const uint32_t row = (uint32_t)imin(prow, last);
                const uint32_t c = (uint32_t)((Pg % CPRV) ^ hswz<DV>(prow));
                src = grow + (row * lddo_b + 16u * c);
            }
            gl_lds16_at(src, sb + 16u * (uint32_t)(i * NT));
        }
    };

    // Per-lane LDS byte offsets, computed once.  Row operands: row
    // 32*rh + l32 of a staged tile and key row 32*kw + l32 of K / V, logical
    // chunk 2c + hl.  Transposing reads (quarter q = lane/16, j = lane%16):
    // rows 32*rh + 16*h2 + 8*rr + 4*(q/2) + j/4, columns 32*db + 16*(q%2) +
    // 4*(j%4): the row order of the S accumulator (8*(r/4) + 4*hl + r%4) as
    // the k order of the dV / dK products.  The swizzle of a row does not
    // change when a multiple of 16 is added to it, so h2 (and the dO tile)
    // are immediate offsets; a step adds its stage's base once.
    const int q4 = lane >> 4, j16 = lane & 15;
    typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8_t;
    auto lds_row = [](uint32_t addr) __attribute__((always_inline)) {
        return *reinterpret_cast<lds_bf16x8_t *>(addr);
    };
    auto lds_tr = [](uint32_t addr) __attribute__((always_inline)) {
        shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_shortx4_t *>(addr));
        return __builtin_bit_cast(uint2, v);
    };
    const uint32_t lds_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
    // bytes: the [K | V] region (BN DW bf16), one [Q | dO] stage (BM DW
    // bf16), the staged Q tile (the dO tile follows it), the K tile (V
    // follows it)
    constexpr uint32_t KV_BYTES = 2u * BN * DW, STAGE_BYTES = 16u * SLOTS;
    constexpr uint32_t TILE_BYTES = 2u * BM * DQK, K_BYTES = 2u * BN * DQK;
    static_assert(KV_BYTES == BN * DW * sizeof(uint16_t), "ring starts after [K | V]");
    constexpr uint32_t H2_BYTES = 2u * 16u * DQK, H2V_BYTES = 2u * 16u * DV;
    // row operands: Q and K (width DQK), dO and V (width DV); transposing
    // reads: Q (dK products) and dO (dV products)
    uint32_t aoffs[NC], koffs[NC], goffs[NCV], voffs[NCV], toffs[2][NDB], tgoffs[2][NDBV];
    const int ar = 32 * rh + l32, br = 32 * kw + l32;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        aoffs[c] = 2u * (uint32_t)(ar * DQK + 8 * ((2 * c + hl) ^ hswz<DQK>(ar)));
        koffs[c] = lds_base + 2u * (uint32_t)(br * DQK + 8 * ((2 * c + hl) ^ hswz<DQK>(br)));
    }
#pragma unroll
    for (int c = 0; c < NCV; ++c) {
        if constexpr (DV == DQK) {  // the same per-lane offsets, one tile further
            goffs[c] = aoffs[c] + TILE_BYTES;
            voffs[c] = koffs[c] + K_BYTES;
        } else {
            goffs[c] = TILE_BYTES + 2u * (uint32_t)(ar * DV + 8 * ((2 * c + hl) ^ hswz<DV>(ar)));
            voffs[c] = lds_base + K_BYTES +
                       2u * (uint32_t)(br * DV + 8 * ((2 * c + hl) ^ hswz<DV>(br)));
        }
    }
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int row = 32 * rh + 8 * rr + 4 * (q4 >> 1) + (j16 >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = 32 * db + 16 * (q4 & 1) + 4 * (j16 & 3);
            toffs[rr][db] = 2u * (uint32_t)(row * DQK + 8 * ((col >> 3) ^ hswz<DQK>(row)) + (col & 7));
        }
#pragma unroll
        for (int db = 0; db < NDBV; ++db) {
            const int col = 32 * db + 16 * (q4 & 1) + 4 * (j16 & 3);
            if constexpr (DV == DQK) tgoffs[rr][db] = toffs[rr][db] + TILE_BYTES;
            else
                tgoffs[rr][db] = TILE_BYTES + 2u * (uint32_t)(row * DV + 8 * ((col >> 3) ^ hswz<DV>(row)) +
                                                             (col & 7));
        }
    }

    floatx16 dkacc[NDB], dvacc[NDBV];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dkacc[i] = zero16();
#pragma unroll
    for (int i = 0; i < NDBV; ++i) dvacc[i] = zero16();

    // One step of this wave's 32 rows x 32 keys: S = Q K^T and dP = dO V^T,
    // then P = s sigma (= SiLU(t) / alpha) and dS = g sigma (1 + t (1 -
    // sigma)) = g (sigma + a (alpha - alpha sigma)) in fp32 (exp(-t)
    // overflowing to inf gives sigma = 0, a = 0 and dS = 0, its limit, with
    // no NaN), masked on partial steps, rounded to bf16 (with the low parts
    // when split), and the dV, dK products.  Mask: in terms of x = i - kj
    // (register r has x = x0 + 8*(r/4) + r%4), rows before m1 of a history
    // step see the key iff 0 <= x < W, W = m1 - kj, capped at K1 unless kj is
    // a prefix key; rows of a target step iff x < m1 - kj and (x == 0 or kj
    // lies in row U's view).  No branch inside a step.
    auto step = [&](int t, auto FULL, auto SPLIT) __attribute__((always_inline)) {
        constexpr bool full = decltype(FULL)::value, split = decltype(SPLIT)::value;
        // wait for this step's DMA (the newest (NST - 2) SPS loads, those of
        // the following steps, may still be in flight), publish it with a
        // barrier that also frees stage (t + NST - 1) % NST (read by step
        // t - 1), and start the DMA of step t + NST - 1 into it.  With the dS
        // stores, which the vector memory counter tracks in issue order with
        // the loads, the two stores of each of steps t - 2 and t - 1 are
        // newer than this step's DMA too (from step 2 on).
        if constexpr (STORE_DS) {
            static_assert(NST == 3, "the store-aware wait counts assume a ring of three");
            if (t >= 2) vm_wait<SPS + 4>();
            else vm_wait<SPS>();
        } else {
            vm_wait<(NST - 2) * SPS>();
        }
        barrier_lds();
        issue(t + NST - 1);
        const uint32_t sb = lds_base + KV_BYTES + (uint32_t)uniform(t % NST) * STAGE_BYTES;
        int m0, m1;
        step_rows(t, m0, m1);
        m0 = uniform(m0);
        m1 = uniform(m1);

        floatx16 sacc = zero16(), pacc = zero16();
#pragma unroll
        for (int c = 0; c < (NC > NCV ? NC : NCV); ++c) {
            if (c < NC) sacc = mfma32(lds_row(aoffs[c] + sb), lds_row(koffs[c]), sacc);
            if (c < NCV) pacc = mfma32(lds_row(goffs[c] + sb), lds_row(voffs[c]), pacc);
        }
        float pv[16], dv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float sv = sacc[r];
            const float sgm = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sv * nal2e));
            const float a = sv * sgm;
            pv[r] = a;
            dv[r] = pacc[r] * fmaf(a, fmaf(-alpha, sgm, alpha), sgm);
        }
        if constexpr (!full) {
            const int x0 = m0 + 32 * rh + 4 * hl - kj;
            const bool tstep = m0 >= sd.U;
            const int Wh = (!tstep && kj >= p.k2e) ? imin(m1 - kj, p.k1) : m1 - kj;
            const uint32_t Wu = (uint32_t)imax(Wh, 0);
            const bool tv = !tstep || ((kj < sd.U) & ((sd.U - kj < p.k1) | (kj < p.k2e)));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int x = x0 + 8 * (r >> 2) + (r & 3);
                const bool vis = ((uint32_t)x < Wu) & (tv | (x == 0));
                pv[r] = vis ? pv[r] : 0.0f;
                dv[r] = vis ? dv[r] : 0.0f;
            }
        }
        uint32_t taddr[2][NDB], tgaddr[2][NDBV];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) taddr[rr][db] = toffs[rr][db] + sb;
#pragma unroll
            for (int db = 0; db < NDBV; ++db) tgaddr[rr][db] = tgoffs[rr][db] + sb;
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int o = 8 * h2;
            const bf16x8 pa = cvt8(pv[o], pv[o + 1], pv[o + 2], pv[o + 3], pv[o + 4], pv[o + 5],
                                   pv[o + 6], pv[o + 7]);
            const bf16x8 da = cvt8(dv[o], dv[o + 1], dv[o + 2], dv[o + 3], dv[o + 4], dv[o + 5],
                                   dv[o + 6], dv[o + 7]);
            if constexpr (STORE_DS) {
                const int blk = t + (t < nh ? ds_dh : ds_dt);
                uint8_t *dst = ds_wave + (int64_t)blk * DS_BLOCK_BYTES + 1024 * h2 + 16 * lane;
                st16_global_stream(dst, as_u4(da));
            }
            bf16x8 pl, dl;
            if constexpr (split) {
                pl = lo_part(pv + o, pa);
                dl = lo_part(dv + o, da);
            }
            // dV block db then dK block db, as far as both exist
#pragma unroll
            for (int db = 0; db < (NDB > NDBV ? NDB : NDBV); ++db) {
                if (db < NDBV) {
                    const uint32_t ho = h2 * H2V_BYTES;
                    const uint2 g0 = lds_tr(tgaddr[0][db] + ho);
                    const uint2 g1 = lds_tr(tgaddr[1][db] + ho);
                    const bf16x8 gfr = __builtin_bit_cast(bf16x8, make_uint4(g0.x, g0.y, g1.x, g1.y));
                    dvacc[db] = mfma32(pa, gfr, dvacc[db]);
                    if constexpr (split) dvacc[db] = mfma32(pl, gfr, dvacc[db]);
                }
                if (db < NDB) {
                    const uint32_t ho = h2 * H2_BYTES;
                    const uint2 q0 = lds_tr(taddr[0][db] + ho);
                    const uint2 q1 = lds_tr(taddr[1][db] + ho);
                    const bf16x8 qfr = __builtin_bit_cast(bf16x8, make_uint4(q0.x, q0.y, q1.x, q1.y));
                    dkacc[db] = mfma32(da, qfr, dkacc[db]);
                    if constexpr (split) dkacc[db] = mfma32(dl, qfr, dkacc[db]);
                }
            }
        }
    };
    // the key tile, then masked steps [0, s_lo), full steps [s_lo, s_hi) and
    // masked steps [s_hi, nsteps); split (two-term P and dS) for key tiles
    // that hold global-prefix keys
    auto run = [&](auto SPLIT) __attribute__((always_inline)) {
        if (nsteps == 0) return;
        issue_kv();
#pragma unroll
        for (int i = 0; i < NST - 1; ++i) issue(i);
        for (int t = 0; t < s_lo; ++t) step(t, std::false_type{}, SPLIT);
        for (int t = s_lo; t < s_hi; ++t) step(t, std::true_type{}, SPLIT);
        for (int t = s_hi; t < nsteps; ++t) step(t, std::false_type{}, SPLIT);
        vm_wait<0>();  // no DMA (of the clamped steps past the end) left in flight
    };
    if (it.c0 < p.k2e) run(std::true_type{});
    else run(std::false_type{});

    // the two row halves of key block kw: the rh = 1 wave hands its dK sum to
    // the rh = 0 wave and takes the rh = 0 wave's dV sum, through LDS (free
    // after the barrier): 32 keys x DQK floats of dK and 32 x DV of dV per
    // key block, 32 KB at d = 128.  Accumulator: lane holds column
    // d = 32*db + l32, register r holds key 32*kw + 8*(r/4) + 4*hl + r%4 of
    // the tile; rh = 0 writes dK, rh = 1 dV, both scaled by alpha / N (P
    // carries 1/alpha).
    __syncthreads();
    const float sc = p.out_scale;
    if constexpr (DQK == DV) {
        // region 2 kw holds the dK hand-over, 2 kw + 1 the dV one
        float *const xr = reinterpret_cast<float *>(lds);
        floatx16 *mine = rh == 0 ? dkacc : dvacc;   // the sum this wave writes out
        floatx16 *other = rh == 0 ? dvacc : dkacc;  // the sum it hands over
        {
            float *xo = xr + (2 * kw + (1 - rh)) * (32 * DQK);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64 + lane] = other[db][r];
        }
        __syncthreads();
        {
            const float *xi = xr + (2 * kw + rh) * (32 * DQK);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) mine[db][r] += xi[(db * 16 + r) * 64 + lane];
        }
        if (it.nchunk == 1) {
            void *dst = rh == 0 ? p.dk : p.dv;
            const int64_t ld = rh == 0 ? p.lddk : p.lddv;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = it.c0 + 32 * kw + 8 * (r >> 2) + 4 * hl + (r & 3);
                    if (j < it.c1) {
                        const int64_t o = (sd.base + j) * ld + h * DQK + 32 * db + l32;
                        if constexpr (OUTF32) reinterpret_cast<float *>(dst)[o] = mine[db][r] * sc;
                        else reinterpret_cast<__bf16 *>(dst)[o] = (__bf16)(mine[db][r] * sc);
                    }
                }
            }
        } else {
            // fp32 partials [key][dK | dV] of this chunk
            const int slot = p.s.part_base[b] + it.tile * nch + it.chunk;
            float *part = p.partials + ((int64_t)slot * p.H + h) * BN * DW + rh * DQK;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int jl = 32 * kw + 8 * (r >> 2) + 4 * hl + (r & 3);
                    part[jl * DW + 32 * db + l32] = mine[db][r];
                }
            }
        }
        return;
    }
    float *const xreg = reinterpret_cast<float *>(lds) + kw * (32 * DW);
    float *const xk = xreg, *const xv = xreg + 32 * DQK;
    if (rh == 0) {
#pragma unroll
        for (int db = 0; db < NDBV; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) xv[(db * 16 + r) * 64 + lane] = dvacc[db][r];
    } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) xk[(db * 16 + r) * 64 + lane] = dkacc[db][r];
    }
    __syncthreads();
    if (rh == 0) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) dkacc[db][r] += xk[(db * 16 + r) * 64 + lane];
    } else {
#pragma unroll
        for (int db = 0; db < NDBV; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) dvacc[db][r] += xv[(db * 16 + r) * 64 + lane];
    }

    auto write_out = [&](const floatx16 *acc, auto NB, void *dst, int64_t ld, int width, int pcol)
        __attribute__((always_inline)) {
        constexpr int nb = decltype(NB)::value;
        if (it.nchunk == 1) {
#pragma unroll
            for (int db = 0; db < nb; ++db) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = it.c0 + 32 * kw + 8 * (r >> 2) + 4 * hl + (r & 3);
                    if (j < it.c1) {
                        const int64_t o = (sd.base + j) * ld + h * width + 32 * db + l32;
                        if constexpr (OUTF32) reinterpret_cast<float *>(dst)[o] = acc[db][r] * sc;
                        else reinterpret_cast<__bf16 *>(dst)[o] = (__bf16)(acc[db][r] * sc);
                    }
                }
            }
        } else {
            // fp32 partials [key][dK | dV] of this chunk
            const int slot = p.s.part_base[b] + it.tile * nch + it.chunk;
            float *part = p.partials + ((int64_t)slot * p.H + h) * BN * DW + pcol;
#pragma unroll
            for (int db = 0; db < nb; ++db) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int jl = 32 * kw + 8 * (r >> 2) + 4 * hl + (r & 3);
                    part[jl * DW + 32 * db + l32] = acc[db][r];
                }
            }
        }
    };
    if (rh == 0) write_out(dkacc, std::integral_constant<int, NDB>{}, p.dk, p.lddk, DQK, 0);
    else write_out(dvacc, std::integral_constant<int, NDBV>{}, p.dv, p.lddv, DV, DQK);
}

// Sum the chunk partials of each split prefix key tile in chunk order.  Block
// (item, slab) handles 1024 consecutive values of the [BN][2D] tile.
constexpr int RED_SLAB = 1024;

template <int DQK, int DV, bool OUTF32>
__global__ __launch_bounds__(256) void sla_bwd_reduce_kernel(AttnParams p)
{
    constexpr int BN = BWD_BN, W = DQK + DV, SLABS = BN * W / RED_SLAB;
    static_assert((BN * W) % RED_SLAB == 0 && DQK % 4 == 0, "whole slabs; no float4 spans dK | dV");
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
    const float sc = p.out_scale;
    const int64_t off = col < DQK ? (sd.base + c0 + jl) * p.lddk + h * DQK + col
                                  : (sd.base + c0 + jl) * p.lddv + h * DV + (col - DQK);
    void *base = col < DQK ? p.dk : p.dv;
    if constexpr (OUTF32) {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(base) + off) =
            make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
    } else {
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(base) + off) =
            cvt4_u2(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
    }
}

template <bool OUTF32>
static hipError_t launch_dkdv_o(const AttnParams &p, hipStream_t st)
{
    return with_head_dims(p, [&](auto QK, auto V) {
        constexpr int DQK = decltype(QK)::value, DV = decltype(V)::value;
        if (p.ds)
            hipLaunchKernelGGL((sla_bwd_dkdv_bf16_kernel<DQK, DV, OUTF32, true>),
                               dim3(p.grid_bwd), dim3(DKDV_THREADS), 0, st, p);
        else
            hipLaunchKernelGGL((sla_bwd_dkdv_bf16_kernel<DQK, DV, OUTF32, false>),
                               dim3(p.grid_bwd), dim3(DKDV_THREADS), 0, st, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || p.grid_red == 0) return e;
        hipLaunchKernelGGL((sla_bwd_reduce_kernel<DQK, DV, OUTF32>),
                           dim3(p.grid_red * (BWD_BN * (DQK + DV) / RED_SLAB)), dim3(256), 0, st, p);
        return hipGetLastError();
    });
}

hipError_t launch_bwd_dkdv_bf16(const AttnParams &p, hipStream_t st)
{
    return p.out_f32 ? launch_dkdv_o<true>(p, st) : launch_dkdv_o<false>(p, st);
}

}  // namespace sla
