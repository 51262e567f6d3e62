// sla_tiles.h -- staging of 64-row bf16 tiles from HBM through registers into
// LDS, row-major (operand rows read as 16-byte chunks) and/or transposed (the
// contraction index made contiguous for the second MFMA of a pair).
#pragma once

#include "sla_device.h"

namespace sla {

// A 64-row x D-column bf16 tile.  Thread t owns rows 4g..4g+3 (g = t / CPR) of
// 16-byte column chunk c = t % CPR, so the four rows can be written both as
// rows and, regrouped per column, as 4-key runs of the transposed tile.
template <int D>
struct Tile64 {
    static constexpr int CPR = D / 8;            // 16-byte chunks per row
    static constexpr int NG = 16;                // 4-row groups in 64 rows
    static constexpr int ACTIVE = NG * CPR;      // threads that carry data
    static constexpr int ELEMS = 64 * D;         // bf16 elements in the tile
    uint32_t w[4][4];                            // rows x 4 words (8 bf16)

    // every thread of a 256-thread workgroup carries data when D = 128
    __device__ __forceinline__ static bool active(int tid) { return ACTIVE >= 256 || tid < ACTIVE; }

    // Load rows [row0, row0 + 64) of a [tokens][ld] tensor (head offset
    // already applied to `base_ptr`); rows at or past `limit` (>= 1) read as zero.
    __device__ __forceinline__ void load(const uint16_t *base_ptr, int64_t ld, int row0, int limit,
                                         int tid)
    {
        if (!active(tid)) return;
        const int g = tid / CPR, c = tid % CPR;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 v = ld16_row(base_ptr, ld, row0 + 4 * g + i, limit, 8 * c);
            w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
        }
    }

    // As load, but rows at or past `limit` hold a copy of row limit - 1 and
    // must be masked by the consumer.  No select follows the loads, so they
    // stay in flight until the tile is stored (used for tiles streamed in a
    // loop, where a wait right after each load would expose its latency).
    __device__ __forceinline__ void load_clamped(const uint16_t *base_ptr, int64_t ld, int row0,
                                                 int limit, int tid)
    {
        if (!active(tid)) return;
        const int g = tid / CPR, c = tid % CPR;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 v = ld16_clamped(base_ptr, ld, row0 + 4 * g + i, limit, 8 * c);
            w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
        }
    }

    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) w[i][j] = 0u;
    }

    // Row-major [64][D], chunks swizzled by row.
    __device__ __forceinline__ void store_rows(uint16_t *lds, int tid) const
    {
        if (!active(tid)) return;
        const int g = tid / CPR, c = tid % CPR;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            uint4 v = {w[i][0], w[i][1], w[i][2], w[i][3]};
            *reinterpret_cast<uint4 *>(lds + r * D + 8 * swz_row<CPR>(r, c)) = v;
        }
    }

    // Transposed [D][64], rows of 64 positions (see tpos) with chunks swizzled
    // by swz_t.
    __device__ __forceinline__ void store_transposed(uint16_t *lds, int tid) const
    {
        if (!active(tid)) return;
        const int g = tid / CPR, c = tid % CPR;
        const int pos = tpos(4 * g);
        const int ch = pos >> 3, within = pos & 7;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = 8 * c + e;
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const int m = e >> 1;
            uint2 v;
            v.x = pack_halves(w[0][m], w[1][m], sel);
            v.y = pack_halves(w[2][m], w[3][m], sel);
            *reinterpret_cast<uint2 *>(lds + d * 64 + 8 * swz_t(d, ch) + within) = v;
        }
    }
};

// The transposed tile converted to fp16 (values multiplied by `scale`, a power
// of two, first): same layout as store_transposed.
template <int D>
__device__ __forceinline__ void store_transposed_f16(const Tile64<D> &t, uint16_t *lds, int tid,
                                                     float scale)
{
    if (!Tile64<D>::active(tid)) return;
    constexpr int CPR = Tile64<D>::CPR;
    const int g = tid / CPR, c = tid % CPR;
    const int pos = tpos(4 * g);
    const int ch = pos >> 3, within = pos & 7;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int d = 8 * c + e;
        const int m = e >> 1;
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = ((e & 1) ? bf16_hi(t.w[i][m]) : bf16_lo(t.w[i][m])) * scale;
        uint2 v;
        v.x = cvt2h_u32(f[0], f[1]);
        v.y = cvt2h_u32(f[2], f[3]);
        *reinterpret_cast<uint2 *>(lds + d * 64 + 8 * swz_t(d, ch) + within) = v;
    }
}

// 16-byte operand read from a row-major swizzled tile: row r, logical chunk c.
template <int D>
__device__ __forceinline__ bf16x8 lds_row_chunk(const uint16_t *lds, int r, int c)
{
    return as_bf16x8(*reinterpret_cast<const uint4 *>(lds + r * D + 8 * swz_row<D / 8>(r, c)));
}

// 16-byte fp16 operand read from a transposed tile: column d, position chunk c.
__device__ __forceinline__ halfx8 lds_t_chunk_h(const uint16_t *lds, int d, int c)
{
    return as_halfx8(*reinterpret_cast<const uint4 *>(lds + d * 64 + 8 * swz_t(d, c)));
}

}  // namespace sla
