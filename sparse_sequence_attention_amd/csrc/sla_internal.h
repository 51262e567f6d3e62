// sla_internal.h -- types, tile constants and the on-device tile schedule shared
// by the HIP kernels of the SLA library and its host launcher.
//
// The schedule is the integer part of the semi-local attention hot path
// (ULTRA-HSTU paper, section 4.2.1, Eq.7: a row sees a local window of K1 keys
// and a global prefix of K2e keys, so only those tiles are visited; the
// torcheasyrec "ULTRA HSTU" page gives K2e = max(sla_k2, contextual_seq_len);
// target rows follow the M-FALCON mask of the HSTU notes, Q8).  It is built on
// the device from the jagged offsets, so no host synchronisation is needed:
//   1. sla_sched_kernel (one workgroup) writes per-sequence prefix sums of the
//      work items of each kernel;
//   2. every attention workgroup maps its block index to a work item, finds its
//      sequence by binary search over those prefix sums and derives its tile and
//      the ranges of the other operand with the functions below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sla {

// ---------------------------------------------------------------------------
// Tile geometry
// ---------------------------------------------------------------------------
constexpr int FWD_BM = 128;        // rows per forward / dQ work item (4 waves x 32)
constexpr int FWD_BN = 64;         // keys per forward / dQ step
constexpr int BWD_BN = 128;        // keys per dK/dV work item (4 waves x 32)
constexpr int BWD_BM = 64;         // rows per dK/dV step
constexpr int BWD_CHUNK_TILES = 18;  // target row tiles per chunk of a split prefix key tile
constexpr int BWD_MAX_CHUNKS = 16;   // at most this many chunks per prefix key tile
constexpr int BWD_MAX_SPLIT_TILES = 4;  // prefix key tiles per sequence that may be split
constexpr int NUM_XCD = 8;         // MI355X: 8 accelerator complex dies, own L2 each
// Per-sequence prefix sums written by the schedule kernel (device, int32).
struct Sched {
    int32_t *fwd_base;   // [B+1] row-tile items (forward, dQ); [B] = total
    int32_t *bwd_base;   // [B+1] key-tile items (dK/dV), split prefix tiles expanded
    int32_t *red_base;   // [B+1] split key tiles to reduce
    int32_t *part_base;  // [B+1] fp32 partial slots
    int32_t *nch;        // [B]   chunks per prefix key tile (1 = unsplit)
    // stored-dS backward only (null otherwise):
    int32_t *ktile_base; // [B+1] key tiles of BWD_BN keys per sequence
    int32_t *ds_base;    // [key tiles + 1] dS blocks (64-row steps) of each key tile
};

// One stored dS block: the 64-row step x 128-key tile of one head as the
// dK/dV kernel's eight waves hold it in registers (bf16 MFMA A fragments).
constexpr int DS_BLOCK_BYTES = 64 * 128 * 2;

struct SeqDims {
    int64_t base;  // first token of the sequence
    int L;         // length
    int U;         // first target row (L when there are no targets)
};

// Up to three half-open ranges of the other operand, in tokens of the sequence
// (scalar fields: an indexed array would be placed in scratch memory).
struct Ranges {
    int lo0, hi0, lo1, hi1, lo2, hi2;
    int n;
};

__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Visibility of key j from row i (both within one sequence): history rows are
// causal with a K1 local window or a K2e global prefix; a target row sees itself
// and the history keys of the first target slot's window.
__host__ __device__ inline bool visible(int i, int j, int U, int K1, int K2e)
{
    // branch-free: both cases evaluated with non-short-circuit logic, then a select
    const bool hist = (j <= i) & ((i - j < K1) | (j < K2e));
    const bool tgt = (j == i) | ((j < U) & ((U - j < K1) | (j < K2e)));
    return (i < U) ? hist : tgt;
}

// Number of row tiles (forward / dQ items) of a sequence: history rows from 0
// and target rows from U, each cut into bm-row tiles, so no tile mixes them.
__host__ __device__ inline int row_tiles(int L, int U, int bm)
{
    return cdiv(U, bm) + cdiv(L - U, bm);
}

__host__ __device__ inline void row_tile(int L, int U, int bm, int t, int &r0, int &r1)
{
    int nh = cdiv(U, bm);
    if (t < nh) {
        r0 = t * bm;
        r1 = imin(r0 + bm, U);
    } else {
        r0 = U + (t - nh) * bm;
        r1 = imin(r0 + bm, L);
    }
}

// Round the key interval [a, b) out to whole bn-key tiles (clipped at L).
__host__ __device__ inline void tile_round(int &a, int &b, int bn, int L)
{
    if (a >= b) {
        a = b = 0;
        return;
    }
    a = (a / bn) * bn;
    b = imin(cdiv(b, bn) * bn, L);
}

// Keys visited by the row tile [r0, r1): the union of the visible keys, rounded
// out to whole key tiles.  History tile: prefix [0, min(K2e, r1)) and band
// [r0-K1+1, r1).  Target tile: prefix [0, min(K2e, U)), window of row U over
// history keys [U-K1+1, U), and the diagonal [r0, r1).  The three candidate
// intervals start in increasing order; touching ones are merged.  (Scalars
// only: an indexed array here would live in scratch memory.)
__host__ __device__ inline Ranges fwd_key_ranges(int L, int U, int K1, int K2e, int r0, int r1,
                                                 int bn)
{
    Ranges r{0, 0, 0, 0, 0, 0, 0};
    if (r0 >= r1) return r;
    int aA, bA, aB, bB, aC, bC;
    if (r0 < U) {
        aA = 0; bA = imin(K2e, r1);
        aB = K1 >= 1 ? imax(0, r0 - K1 + 1) : 0; bB = K1 >= 1 ? r1 : 0;
        aC = bC = 0;
    } else {
        aA = 0; bA = imin(K2e, U);
        aB = K1 >= 2 ? imax(0, U - K1 + 1) : 0; bB = K1 >= 2 ? U : 0;
        aC = r0; bC = r1;
    }
    tile_round(aA, bA, bn, L);
    tile_round(aB, bB, bn, L);
    tile_round(aC, bC, bn, L);
    bool eA = aA < bA, eB = aB < bB, eC = aC < bC;
    if (eA && eB && aB <= bA) { bA = imax(bA, bB); eB = false; }
    if (eC && eB && aC <= bB) { bB = imax(bB, bC); eC = false; }
    if (eC && !eB && eA && aC <= bA) { bA = imax(bA, bC); eC = false; }
    // compact the non-empty ranges into slots 0..n-1
    if (!eA) { aA = aB; bA = bB; eA = eB; aB = aC; bB = bC; eB = eC; eC = false; }
    if (!eA) { aA = aB; bA = bB; eA = eB; eB = false; }
    if (!eB) { aB = aC; bB = bC; eB = eC; eC = false; }
    r.lo0 = aA; r.hi0 = bA; r.lo1 = aB; r.hi1 = bB; r.lo2 = aC; r.hi2 = bC;
    r.n = eA ? (eB ? (eC ? 3 : 2) : 1) : 0;
    if (r.n < 3) { r.lo2 = r.hi2 = 0; }
    if (r.n < 2) { r.lo1 = r.hi1 = 0; }
    if (r.n < 1) { r.lo0 = r.hi0 = 0; }
    return r;
}

// Tiles of up to three ranges, addressed by index with scalar state only (a
// dynamically indexed array would be placed in LDS by the compiler).
struct TileCursor {
    int lo0, lo1, lo2, n0, n01, total;
    __host__ __device__ TileCursor(const Ranges &r, int bn)
    {
        lo0 = r.n > 0 ? r.lo0 : 0;
        lo1 = r.n > 1 ? r.lo1 : 0;
        lo2 = r.n > 2 ? r.lo2 : 0;
        int c0 = r.n > 0 ? cdiv(r.hi0 - r.lo0, bn) : 0;
        int c1 = r.n > 1 ? cdiv(r.hi1 - r.lo1, bn) : 0;
        int c2 = r.n > 2 ? cdiv(r.hi2 - r.lo2, bn) : 0;
        n0 = c0;
        n01 = c0 + c1;
        total = c0 + c1 + c2;
    }
    // first key of tile t (0 <= t < total); selects rather than branches
    __host__ __device__ int start(int t, int bn) const
    {
        const bool in0 = t < n0, in1 = t < n01;
        const int lo = in0 ? lo0 : (in1 ? lo1 : lo2);
        const int first = in0 ? 0 : (in1 ? n0 : n01);
        return lo + (t - first) * bn;
    }
};

// dK/dV items.  Key tiles of bn keys from key 0.  The rows that see the key
// tile [c0, c1): history rows [c0, U) if the tile holds a global-prefix key,
// else [c0, min(last history key + K1, U)); all targets if a history key of the
// tile lies in row U's view, else the tile's own target rows (self).
struct BwdItem {
    int c0, c1;       // key tile
    int ha, hb;       // history rows of this chunk
    int ta, tb;       // target rows of this chunk
    int chunk, nchunk;
    int tile;         // key tile index within the sequence
};

__host__ __device__ inline int prefix_key_tiles(int L, int K2e, int bn)
{
    return cdiv(imin(K2e, L), bn);
}

__host__ __device__ inline void bwd_rows(int L, int U, int K1, int K2e, int c0, int c1, int &ha,
                                         int &hb, int &ta, int &tb)
{
    ha = hb = ta = tb = 0;
    int jhi = imin(c1, U) - 1;  // last history key of the tile
    if (c0 < U) {
        if (c0 < K2e) {
            ha = c0;
            hb = U;
        } else if (K1 >= 1) {
            ha = c0;
            hb = (int)((long long)jhi + K1 < (long long)U ? jhi + K1 : U);
        }
    }
    bool all_t = (c0 < U) && ((U - jhi < K1) || (c0 < K2e));
    if (U < L) {
        if (all_t) {
            ta = U;
            tb = L;
        } else if (c1 > U) {
            ta = imax(c0, U);
            tb = c1;
        }
    }
    if (ha >= hb) ha = hb = 0;
    if (ta >= tb) ta = tb = 0;
}

// The 64-row steps (bm rows, history steps counted from row 0, target steps
// from row U) of all rows that see the key tile [c0, c1): history steps
// h_first .. h_first + nh, then target steps t_first .. t_first + nt.  The
// chunks of a split key tile partition these steps; the stored-dS backward
// numbers a key tile's blocks in this order.
struct TileSteps {
    int h_first, nh, t_first, nt;
};

__host__ __device__ inline TileSteps tile_steps(int L, int U, int K1, int K2e, int c0, int c1,
                                                int bm)
{
    int ha, hb, ta, tb;
    bwd_rows(L, U, K1, K2e, c0, c1, ha, hb, ta, tb);
    TileSteps t{0, 0, 0, 0};
    if (ha < hb) {
        t.h_first = ha / bm;
        t.nh = cdiv(hb, bm) - t.h_first;
    }
    if (ta < tb) {
        t.t_first = (ta - U) / bm;
        t.nt = cdiv(tb - U, bm) - t.t_first;
    }
    return t;
}

// The index, within key tile [ct, ct + 128)'s blocks (tile_steps order, 64-row
// steps), of the step that starts at row m0 (history rows from 0, target rows
// from U, in 64-row steps), or -1 when no row of that step sees the tile: the
// same numbers as tile_steps, without its general case analysis.  K1c =
// min(K1, U).
__host__ __device__ inline int ds_block_in_tile(int L, int U, int K1, int K1c, int K2e, int ct,
                                                int m0)
{
    const int jhi = imin(ct + 128, U) - 1;  // last history key of the tile
    const bool hk = ct < U;
    const int hb = !hk ? 0 : (ct < K2e ? U : (K1 < 1 ? 0 : imin(jhi + K1c, U)));
    if (m0 < U) return (m0 >= ct && m0 < hb) ? (m0 - ct) >> 6 : -1;
    const int nh = hb > ct ? ((hb + 63) >> 6) - (ct >> 6) : 0;
    const bool all_t = hk && ((U - jhi < K1) || ct < K2e);
    const int c1 = imin(ct + 128, L);
    const int ta = all_t ? U : imax(ct, U);
    const int tb = all_t ? L : (c1 > U ? c1 : 0);
    const int tf = (ta - U) >> 6, g = (m0 - U) >> 6;
    return (ta < tb && g >= tf && m0 < tb) ? nh + g - tf : -1;
}

// Row tiles (of bm rows, aligned as the forward row tiles) overlapping [a, b),
// as tile indices [lo, hi) of the history (origin 0) or target (origin U) part.
__host__ __device__ inline void tile_span(int a, int b, int origin, int bm, int &lo, int &hi)
{
    if (a >= b) {
        lo = hi = 0;
        return;
    }
    lo = (a - origin) / bm;
    hi = cdiv(b - origin, bm);
}

// Number of chunks for the prefix key tiles of a sequence: enough to keep a
// chunk near BWD_CHUNK_TILES row tiles, at most BWD_MAX_CHUNKS, and 1 when the
// sequence is short.
__host__ __device__ inline int bwd_num_chunks(int L, int U, int bm)
{
    int rows = row_tiles(L, U, bm);
    int n = cdiv(rows, BWD_CHUNK_TILES);
    if (n > BWD_MAX_CHUNKS) n = BWD_MAX_CHUNKS;
    return n < 1 ? 1 : n;
}

__host__ __device__ inline int bwd_items(int L, int U, int K2e, int bn, int bm, int &np, int &nch)
{
    int nk = cdiv(L, bn);
    np = imin(prefix_key_tiles(L, K2e, bn), BWD_MAX_SPLIT_TILES);
    nch = bwd_num_chunks(L, U, bm);
    if (nch <= 1 || np == 0) {
        nch = 1;
        return nk;
    }
    return np * nch + (nk - np);
}

__host__ __device__ inline BwdItem bwd_item(int L, int U, int K1, int K2e, int bn, int bm,
                                            int li, int np, int nch)
{
    BwdItem it;
    if (nch > 1 && li < np * nch) {
        it.tile = li / nch;
        it.chunk = li - it.tile * nch;
        it.nchunk = nch;
    } else {
        it.tile = (nch > 1) ? np + (li - np * nch) : li;
        it.chunk = 0;
        it.nchunk = 1;
    }
    it.c0 = it.tile * bn;
    it.c1 = imin(it.c0 + bn, L);
    int ha, hb, ta, tb;
    bwd_rows(L, U, K1, K2e, it.c0, it.c1, ha, hb, ta, tb);
    if (it.nchunk == 1) {
        it.ha = ha; it.hb = hb; it.ta = ta; it.tb = tb;
        return it;
    }
    // split the row tiles of [ha,hb) then [ta,tb) into nchunk even pieces
    int hlo, hhi, tlo, thi;
    tile_span(ha, hb, 0, bm, hlo, hhi);
    tile_span(ta, tb, U, bm, tlo, thi);
    int nh = hhi - hlo, nt = thi - tlo, R = nh + nt;
    int p0 = (int)((long long)R * it.chunk / it.nchunk);
    int p1 = (int)((long long)R * (it.chunk + 1) / it.nchunk);
    // history part: tiles [p0, min(p1, nh))
    int a0 = imin(p0, nh), a1 = imin(p1, nh);
    if (a0 < a1) {
        it.ha = imax(ha, (hlo + a0) * bm);
        it.hb = imin(hb, (hlo + a1) * bm);
    } else {
        it.ha = it.hb = 0;
    }
    int b0 = imax(p0 - nh, 0), b1 = imax(p1 - nh, 0);
    if (b0 < b1) {
        it.ta = imax(ta, U + (tlo + b0) * bm);
        it.tb = imin(tb, U + (tlo + b1) * bm);
    } else {
        it.ta = it.tb = 0;
    }
    return it;
}

// One work-list record (layout documented with sla_schedule in sla.h) for
// local item li of a sequence of length L with first target U.
__host__ __device__ inline void fill_record(int op, int b, int L, int U, int K1, int K2e, int li,
                                            int32_t *rec)
{
    for (int i = 0; i < 12; ++i) rec[i] = 0;
    rec[0] = b;
    if (op == 0) {
        int r0, r1;
        row_tile(L, U, FWD_BM, li, r0, r1);
        Ranges kr = fwd_key_ranges(L, U, K1, K2e, r0, r1, FWD_BN);
        rec[1] = r0;
        rec[2] = r1;
        rec[3] = kr.n;
        rec[4] = kr.lo0; rec[5] = kr.hi0;
        rec[6] = kr.lo1; rec[7] = kr.hi1;
        rec[8] = kr.lo2; rec[9] = kr.hi2;
        rec[11] = 1;
    } else {
        int np, nch;
        bwd_items(L, U, K2e, BWD_BN, BWD_BM, np, nch);
        BwdItem it = bwd_item(L, U, K1, K2e, BWD_BN, BWD_BM, li, np, nch);
        rec[1] = it.c0;
        rec[2] = it.c1;
        rec[3] = 2;
        rec[4] = it.ha;
        rec[5] = it.hb;
        rec[6] = it.ta;
        rec[7] = it.tb;
        rec[10] = it.chunk;
        rec[11] = it.nchunk;
    }
}

// Work items of one sequence for op (0 = row tiles of the forward and dQ,
// 1 = key tiles of dK/dV).
__host__ __device__ inline int seq_items(int op, int L, int U, int K2e)
{
    if (op == 0) return row_tiles(L, U, FWD_BM);
    int np, nch;
    return bwd_items(L, U, K2e, BWD_BN, BWD_BM, np, nch);
}

// Workgroup-uniform value kept in a scalar register (the compiler cannot prove
// that values loaded through the kernel's pointers are uniform).  Only for
// values that are the same in every lane.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform64(int64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Largest b with base[b] <= item (base is non-decreasing, base[0] = 0).
// UNIFORM: the item is the same in every lane (one work item per workgroup).
template <bool UNIFORM = true>
__device__ inline int find_seq(const int32_t *base, int B, int item)
{
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        int v = base[mid];
        if (UNIFORM) v = uniform(v);
        if (v <= item) lo = mid;
        else hi = mid - 1;
    }
    return UNIFORM ? uniform(lo) : lo;
}

template <bool UNIFORM = true>
__device__ inline SeqDims seq_dims(const int64_t *offsets, const int32_t *num_targets, int b)
{
    SeqDims s;
    s.base = offsets[b];
    s.L = (int)(offsets[b + 1] - s.base);
    s.U = s.L - (num_targets ? num_targets[b] : 0);
    if (UNIFORM) {
        s.base = uniform64(s.base);
        s.L = uniform(s.L);
        s.U = uniform(s.U);
    }
    return s;
}

// Blocks are dispatched round-robin over the XCDs (block i on XCD i % 8).  Give
// each XCD a contiguous run of work items so that neighbouring row tiles, which
// share most of their key band, meet in the same L2.  Returns -1 past the end.
__device__ inline int xcd_remap(int i, int total)
{
    if (i >= total) return -1;
    int x = i % NUM_XCD, p = i / NUM_XCD;
    int q = total / NUM_XCD, r = total % NUM_XCD;
    return x * q + imin(x, r) + p;
}

}  // namespace sla
