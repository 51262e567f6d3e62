// stu_bwd.hip -- kernels of the STU layer backward (ULTRA-HSTU paper, section 3
// Eq.1-5 differentiated in the reverse of the Code Listing 1 order; selective
// rematerialisation as in section 4.2.2: the normalised input and the fused
// projection are recomputed, the attention output is kept, and y is formed
// inside the gated LayerNorm backward):
//   - a weight-gradient GEMM C[m][n] = sum_t A[t][m] B[t][n] over the token
//     dimension, split over token ranges into fp32 partials that a second
//     kernel adds in a fixed order (no atomics);
//   - LayerNorm and gated-LayerNorm backward, one wave per row, with per-block
//     column partial sums for the norm parameters;
//   - SiLU' applied to the gradient of the projection output, column sums of
//     a [T][C] tensor, and a bf16 matrix transpose.
#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

__device__ __forceinline__ void unpack8(const uint4 &r, float *f)
{
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_lo(w[e]);
        f[2 * e + 1] = bf16_hi(w[e]);
    }
}

// ---------------------------------------------------------------------------
// C_part[s][m][n] = sum_{t in split s} A[t][m] * B[t][n]   (bf16 in, fp32 out)
// ---------------------------------------------------------------------------
// Tile TB x TB (TB = 256: 8 waves of 64 x 128; TB = 128: 8 waves of 64 x 32)
// per token range.  The A and B columns of 32 tokens stream HBM -> LDS by
// DMA through a four-stage ring (three stages ahead), row-major
// ([token][column]); the MFMA operands, 8 consecutive tokens of one column per
// lane, come from transposing LDS reads, with the same token order for A and
// B.  Tokens past the range read a zero row (`zero`, >= TB * 2 bytes), so the
// tail needs no masking.  16-byte chunk c of token row r sits at
// c ^ (4 (r & 3)): the four rows of a transposing read pass land in four
// different quarters of the banks.
constexpr int TN_T = 32;  // tokens per stage

template <int TB>
__global__ __launch_bounds__(512, (TB == 256 ? 1 : 2)) void gemm_tn_kernel(
    const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, const uint16_t *zero,
    float *part, int64_t T, int M, int N, int64_t rows_per_split)
{
    constexpr int RB = TB * 2;                  // bytes per token row of one operand
    constexpr int STAGE = 2 * TN_T * RB;        // A rows then B rows
    constexpr int PER = STAGE / 1024 / 8;       // DMA instructions per thread and stage
    constexpr int WMR = 64;                     // m per wave
    constexpr int WNC = TB == 256 ? 128 : 32;   // n per wave
    constexpr int NFM = WMR / 32, NFN = WNC / 32;
    constexpr int NWM = TB / WMR;               // waves along m
    static_assert(NWM * (TB / WNC) == 8, "8 waves");
    __shared__ __align__(16) uint8_t st0[STAGE], st1[STAGE], st2[STAGE], st3[STAGE];

    const int ntm = M / TB, ntn = N / TB;
    const int item = blockIdx.x;
    const int s = item / (ntm * ntn), rem = item - s * (ntm * ntn);
    const int m0 = (rem / ntn) * TB, n0 = (rem % ntn) * TB;
    const int64_t t0 = (int64_t)s * rows_per_split;
    int64_t t1 = t0 + rows_per_split < T ? t0 + rows_per_split : T;
    if (t1 < t0) t1 = t0;  // a range past the last token writes zeros

    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int wm = wv % NWM, wn = wv / NWM;
    const int q4 = lane >> 4, j16 = lane & 15;

    auto stage = [&](auto S) -> uint8_t * {
        constexpr int sidx = decltype(S)::value;
        if constexpr (sidx == 0) return st0;
        else if constexpr (sidx == 1) return st1;
        else if constexpr (sidx == 2) return st2;
        else return st3;
    };
    // wave-chunk q (1 KB) = stage rows [q * 1024 / RB, ...): lane -> row
    // (q * 1024 + 16 lane) / RB, physical chunk ((16 lane) % RB) / 16
    auto issue = [&](int64_t step, auto S) {
        uint8_t *sb = stage(S);
        const int64_t tb = t0 + step * TN_T;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = i * 8 + wv;
            const int byte = q * 1024 + 16 * lane;
            const int row = byte / RB;              // 0 .. 2 TN_T - 1 (A rows, then B rows)
            const int pc = (byte % RB) / 16;
            const int r = row % TN_T;               // token within the stage
            const int lc = pc ^ (4 * (r & 3));
            const int64_t t = tb + r;
            const uint16_t *src;
            if (t < t1) src = row < TN_T ? A + t * lda + m0 + 8 * lc : B + t * ldb + n0 + 8 * lc;
            else src = zero + 8 * lc;
            gl_lds16(src, reinterpret_cast<uint16_t *>(sb + q * 1024));
        }
    };
    // transposing read: tokens 16 kc + 8 rr + 4 (q4 / 2) + j16 / 4, columns
    // c0 + 16 (q4 % 2) + 4 (j16 % 4) of the operand region at `base`
    auto tr = [&](const uint8_t *base, int kc, int c0) {
        uint2 v[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int row = 16 * kc + 8 * rr + 4 * (q4 >> 1) + (j16 >> 2);
            const int col = c0 + 16 * (q4 & 1) + 4 * (j16 & 3);
            const int pc = (col >> 3) ^ (4 * (row & 3));
            v[rr] = tr_read_b64(reinterpret_cast<const uint16_t *>(base + row * RB + 16 * pc) +
                                (col & 7));
        }
        return __builtin_bit_cast(bf16x8, make_uint4(v[0].x, v[0].y, v[1].x, v[1].y));
    };

    floatx16 acc[NFM][NFN];
#pragma unroll
    for (int i = 0; i < NFM; ++i)
#pragma unroll
        for (int j = 0; j < NFN; ++j) acc[i][j] = zero16();

    auto compute = [&](auto S) {
        const uint8_t *sa = stage(S), *sbb = stage(S) + TN_T * RB;
#pragma unroll
        for (int kc = 0; kc < TN_T / 16; ++kc) {
            bf16x8 a[NFM], b[NFN];
#pragma unroll
            for (int i = 0; i < NFM; ++i) a[i] = tr(sa, kc, WMR * wm + 32 * i);
#pragma unroll
            for (int j = 0; j < NFN; ++j) b[j] = tr(sbb, kc, WNC * wn + 32 * j);
#pragma unroll
            for (int i = 0; i < NFM; ++i)
#pragma unroll
                for (int j = 0; j < NFN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
        }
    };

    // the ring as in the projection GEMM: unconditional DMAs (clamped past the
    // last step), branch-free groups of four steps, then the remainder
    const int64_t nk = (t1 - t0 + TN_T - 1) / TN_T;
    auto step = [&](int64_t k, auto S) {
        constexpr int sidx = decltype(S)::value;
        vm_wait<2 * PER>();
        barrier_lds();
        issue(k + 3 < nk ? k + 3 : (nk > 0 ? nk - 1 : 0), std::integral_constant<int, (sidx + 3) % 4>{});
        compute(S);
    };
    issue(0, std::integral_constant<int, 0>{});
    issue(nk > 1 ? 1 : 0, std::integral_constant<int, 1>{});
    issue(nk > 2 ? 2 : 0, std::integral_constant<int, 2>{});
    const int64_t ng = nk / 4;
    for (int64_t g = 0; g < ng; ++g) {
        step(4 * g, std::integral_constant<int, 0>{});
        step(4 * g + 1, std::integral_constant<int, 1>{});
        step(4 * g + 2, std::integral_constant<int, 2>{});
        step(4 * g + 3, std::integral_constant<int, 3>{});
    }
    const int rem4 = uniform((int)(nk - 4 * ng));
    if (rem4 > 0) step(4 * ng, std::integral_constant<int, 0>{});
    if (rem4 > 1) step(4 * ng + 1, std::integral_constant<int, 1>{});
    if (rem4 > 2) step(4 * ng + 2, std::integral_constant<int, 2>{});
    vm_wait<0>();

    // register r of acc[i][j]: m = 8 (r / 4) + 4 hl + r % 4, n = l32
    const int l32 = lane & 31, hl = lane >> 5;
    float *ps = part + (int64_t)s * M * N;
#pragma unroll
    for (int i = 0; i < NFM; ++i)
#pragma unroll
        for (int j = 0; j < NFN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + WMR * wm + 32 * i + 8 * (r >> 2) + 4 * hl + (r & 3);
                const int n = n0 + WNC * wn + 32 * j + l32;
                ps[(int64_t)m * N + n] = acc[i][j][r];
            }
}

// 256-wide tiles when there are at least 8 of them, else 128; token ranges
// for about one (256) or two (128) workgroups per CU, at least 256 tokens each
TnPlan tn_plan(int64_t T, int M, int N)
{
    TnPlan p{};
    p.tile = (M % 256 == 0 && N % 256 == 0 && (M / 256) * (N / 256) >= 8) ? 256 : 128;
    const int64_t tiles = (int64_t)(M / p.tile) * (N / p.tile);
    const int64_t target = p.tile == 256 ? 256 : 512;
    int64_t splits = tiles > 0 ? (target + tiles - 1) / tiles : 1;
    const int64_t cap = (T + 255) / 256;
    if (splits > cap) splits = cap;
    p.splits = (int)(splits < 1 ? 1 : splits);
    int64_t rows = (T + p.splits - 1) / p.splits;
    p.rows = (rows + TN_T - 1) / TN_T * TN_T;
    return p;
}

// ---------------------------------------------------------------------------
// out[i] = sum over s < splits of part[s][i], i < count (count % 4 == 0), in a
// fixed order: block (x, y) covers floats [256 x, 256 x + 256) (a float4 per
// lane) and the splits of group y; wave w adds splits s0 + w, s0 + w + 4, ...
// in increasing order and the four waves' sums are added in wave order.  A
// short float range with many splits is spread over G groups whose sums go
// to `mid` [G][count], then a second launch adds the G group sums.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sum_splits_kernel(const float *part, int64_t count,
                                                         int splits, int per, float *out)
{
    __shared__ floatx4 red[4][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t i = (int64_t)blockIdx.x * 256 + 4 * lane;
    const int s0 = (int)blockIdx.y * per;
    const int s1 = s0 + per < splits ? s0 + per : splits;
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (i < count) {
        const floatx4 *p = reinterpret_cast<const floatx4 *>(part + i);
        const int64_t step = count / 4;  // one split, in float4
        int s = s0 + wv;
        for (; s + 12 < s1; s += 16) {
            const floatx4 a = p[(int64_t)s * step], b = p[(int64_t)(s + 4) * step];
            const floatx4 c = p[(int64_t)(s + 8) * step], d = p[(int64_t)(s + 12) * step];
            acc += a;
            acc += b;
            acc += c;
            acc += d;
        }
        for (; s < s1; s += 4) acc += p[(int64_t)s * step];
    }
    red[wv][lane] = acc;
    __syncthreads();
    if (wv == 0 && i < count) {
        floatx4 r = red[0][lane];
        r += red[1][lane];
        r += red[2][lane];
        r += red[3][lane];
        *reinterpret_cast<floatx4 *>(out + (int64_t)blockIdx.y * count + i) = r;
    }
}

hipError_t sum_splits(const float *part, int64_t count, int splits, float *out, float *mid,
                      hipStream_t st)
{
    if (count <= 0) return hipSuccess;
    if (count % 4 != 0 || splits < 1) return hipErrorInvalidValue;
    const int64_t gx = (count + 255) / 256;
    int groups = 1;
    if (mid && gx < 256 && splits >= 32) {
        const int64_t want = (256 + gx - 1) / gx;
        groups = (int)(splits / 16 < want ? splits / 16 : want);
    }
    const int per = (splits + groups - 1) / groups;
    groups = (splits + per - 1) / per;
    if (groups == 1) {
        hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)gx, 1), dim3(256), 0, st, part, count,
                           splits, splits, out);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)gx, (unsigned)groups), dim3(256), 0, st,
                       part, count, splits, per, mid);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)gx, 1), dim3(256), 0, st,
                       (const float *)mid, count, groups, groups, out);
    return hipGetLastError();
}

hipError_t launch_gemm_tn_bf16(const void *A, int64_t lda, const void *B, int64_t ldb, int64_t T,
                               int M, int N, const void *zero, float *part, float *out,
                               hipStream_t st)
{
    if (M % 128 != 0 || N % 128 != 0 || lda % 8 != 0 || ldb % 8 != 0 || !zero)
        return hipErrorInvalidValue;
    const TnPlan pl = tn_plan(T, M, N);
    const int tiles = (M / pl.tile) * (N / pl.tile);
    if (pl.tile == 256)
        hipLaunchKernelGGL(gemm_tn_kernel<256>, dim3((unsigned)(tiles * pl.splits)), dim3(512), 0,
                           st, (const uint16_t *)A, lda, (const uint16_t *)B, ldb,
                           (const uint16_t *)zero, part, T, M, N, pl.rows);
    else
        hipLaunchKernelGGL(gemm_tn_kernel<128>, dim3((unsigned)(tiles * pl.splits)), dim3(512), 0,
                           st, (const uint16_t *)A, lda, (const uint16_t *)B, ldb,
                           (const uint16_t *)zero, part, T, M, N, pl.rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return sum_splits(part, (int64_t)M * N, pl.splits, out, nullptr, st);
}

// ---------------------------------------------------------------------------
// Column sums of a [T][C] bf16 tensor (token stride ld, C % 8 == 0): block
// (x, y) covers columns [512 x, 512 x + 512) (8 per lane) of rows
// [COLSUM_ROWS y, ...); wave w adds rows r0 + w, r0 + w + 4, ... in order and
// the waves' sums are added in wave order into part[y][c]; then the
// fixed-order sum over the row blocks.
// ---------------------------------------------------------------------------
constexpr int COLSUM_ROWS = 128;

__global__ __launch_bounds__(256) void colsum_kernel(const uint16_t *X, int64_t ld, int64_t T,
                                                     int C, float *part)
{
    __shared__ float red[4][64 * 8];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = (int)blockIdx.x * 512 + 8 * lane;
    const int64_t r0 = (int64_t)blockIdx.y * COLSUM_ROWS;
    const int64_t r1 = r0 + COLSUM_ROWS < T ? r0 + COLSUM_ROWS : T;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (c < C) {
        for (int64_t r = r0 + wv; r < r1; r += 4) {
            float v[8];
            unpack8(ld16(X + r * ld + c), v);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += v[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wv][8 * lane + e] = acc[e];
    __syncthreads();
    if (wv == 0 && c < C) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            part[(int64_t)blockIdx.y * C + c + e] =
                ((red[0][8 * lane + e] + red[1][8 * lane + e]) + red[2][8 * lane + e]) +
                red[3][8 * lane + e];
    }
}

int colsum_blocks(int64_t T) { return (int)((T + COLSUM_ROWS - 1) / COLSUM_ROWS); }

hipError_t launch_colsum_bf16(const void *X, int64_t ld, int64_t T, int C, float *part, float *out,
                              float *mid, hipStream_t st)
{
    const int nb = colsum_blocks(T);
    if (nb == 0) return hipSuccess;
    if (C % 8 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((C + 511) / 512), (unsigned)nb), dim3(256), 0,
                       st, (const uint16_t *)X, ld, T, C, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return sum_splits(part, (int64_t)C, nb, out, mid, st);
}

// ---------------------------------------------------------------------------
// LayerNorm backward, one wave per row, LN_ROWS rows per workgroup (4 waves
// taking every fourth row).  With xh = (x - mean) * rstd of the row:
//   plain:  g = dy * w;                  dx = rstd (g - mean g - xh mean(g xh)) + res
//           partial_w += dy * xh,        partial_b += dy
//   gated (y = (xh * w + b) (.) u, also written when y is non-NULL: the
//   output projection's weight gradient needs it):
//                                    dyh = dy * u, du = dy * (xh * w + b),
//           g = dyh * w;                 dx = rstd (g - mean g - xh mean(g xh))
//           partial_w += dyh * xh,       partial_b += dyh
// Rows of up to 64 x 8 x 4 = 2048 columns; each lane owns 8-column chunks.
// A wave issues all loads of its next row before the arithmetic of the
// current one, and reads the weight (and bias) chunks once.
// ---------------------------------------------------------------------------
constexpr int LN_ROWS = 16;

__device__ __forceinline__ float wave_sum_b(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}


__device__ __forceinline__ uint4 pack8(const float *f)
{
    const uint2 lo = cvt4_u2(f[0], f[1], f[2], f[3]);
    const uint2 hi = cvt4_u2(f[4], f[5], f[6], f[7]);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

template <bool GATED, int NCH>
__global__ __launch_bounds__(256) void ln_bwd_kernel(
    const uint16_t *x, int64_t ldx, const uint16_t *dy, int64_t lddy, const uint16_t *u,
    int64_t ldu, const float *w, const float *b, const uint16_t *res, int64_t ldres, uint16_t *dx,
    int64_t lddx, uint16_t *du, int64_t lddu, uint16_t *y, int64_t ldy, float *part_w,
    float *part_b, int64_t rows, int cols, float eps)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int nchunk = cols / 8;
    float pw[NCH][8], pb[NCH][8], wf[NCH][8], bf[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = lane + 64 * c;
#pragma unroll
        for (int e = 0; e < 8; ++e) pw[c][e] = pb[c][e] = wf[c][e] = bf[c][e] = 0.0f;
        if (ch < nchunk) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                wf[c][e] = w[8 * ch + e];
                if (GATED && b) bf[c][e] = b[8 * ch + e];
            }
        }
    }
    // the loads of a row, issued together; the next row's are issued before
    // this row's arithmetic
    struct RowIn {
        uint4 x[NCH], dy[NCH], u[NCH], res[NCH];
    };
    auto load = [&](int64_t row, RowIn &in) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = lane + 64 * c;
            if (ch < nchunk) {
                in.x[c] = ld16(x + row * ldx + 8 * ch);
                in.dy[c] = ld16(dy + row * lddy + 8 * ch);
                if (GATED) in.u[c] = ld16(u + row * ldu + 8 * ch);
                if (!GATED && res) in.res[c] = ld16(res + row * ldres + 8 * ch);
            }
        }
    };

    const int64_t r0 = (int64_t)blockIdx.x * LN_ROWS;
    const int64_t rend = r0 + LN_ROWS < rows ? r0 + LN_ROWS : rows;
    int64_t row = r0 + wv;
    RowIn cur, nxt;
    if (row < rend) load(row, cur);
    for (; row < rend; row += 4) {
        if (row + 4 < rend) load(row + 4, nxt);
        float xv[NCH][8], gv[NCH][8];
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (lane + 64 * c < nchunk) {
                unpack8(cur.x[c], xv[c]);
#pragma unroll
                for (int e = 0; e < 8; ++e) s += xv[c][e];
            }
        }
        const float mean = wave_sum_b(s) / (float)cols;
        float q = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            if (lane + 64 * c < nchunk)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float d = xv[c][e] - mean;
                    q += d * d;
                }
        const float rstd = rsqrtf(wave_sum_b(q) / (float)cols + eps);
        // xh, the upstream gradient of the normalised affine output, g
        float m1 = 0.0f, m2 = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = lane + 64 * c;
            if (ch < nchunk) {
                float dv[8];
                unpack8(cur.dy[c], dv);
                float uv[8];
                if (GATED) unpack8(cur.u[c], uv);
                float duv[8], yv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float xh = (xv[c][e] - mean) * rstd;
                    xv[c][e] = xh;
                    float dyh = dv[e];
                    if (GATED) {
                        // same expression as the forward's gated LayerNorm
                        const float yh = xh * wf[c][e] + bf[c][e];
                        yv[e] = yh * uv[e];
                        duv[e] = dv[e] * yh;
                        dyh = dv[e] * uv[e];
                    }
                    pw[c][e] += dyh * xh;
                    pb[c][e] += dyh;
                    const float g = dyh * wf[c][e];
                    gv[c][e] = g;
                    m1 += g;
                    m2 += g * xh;
                }
                if (GATED) {
                    *reinterpret_cast<uint4 *>(du + row * lddu + 8 * ch) = pack8(duv);
                    if (y) *reinterpret_cast<uint4 *>(y + row * ldy + 8 * ch) = pack8(yv);
                }
            }
        }
        m1 = wave_sum_b(m1) / (float)cols;
        m2 = wave_sum_b(m2) / (float)cols;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = lane + 64 * c;
            if (ch < nchunk) {
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = rstd * (gv[c][e] - m1 - xv[c][e] * m2);
                if (!GATED && res) {
                    float rv[8];
                    unpack8(cur.res[c], rv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] += rv[e];
                }
                *reinterpret_cast<uint4 *>(dx + row * lddx + 8 * ch) = pack8(o);
            }
        }
        cur = nxt;
    }
    // column partials of this block: the four waves' sums added in wave order
    __shared__ float red[4][2][64 * 8];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = lane + 64 * c;
        if (c > 0) __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            red[wv][0][lane * 8 + e] = pw[c][e];
            red[wv][1][lane * 8 + e] = pb[c][e];
        }
        __syncthreads();
        if (wv == 0 && ch < nchunk) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int col = 8 * ch + e;
                float sw = 0.0f, sb = 0.0f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    sw += red[k][0][lane * 8 + e];
                    sb += red[k][1][lane * 8 + e];
                }
                part_w[(int64_t)blockIdx.x * cols + col] = sw;
                part_b[(int64_t)blockIdx.x * cols + col] = sb;
            }
        }
    }
}

int ln_bwd_blocks(int64_t rows) { return (int)((rows + LN_ROWS - 1) / LN_ROWS); }

hipError_t launch_ln_bwd_bf16(bool gated, const void *x, int64_t ldx, const void *dy, int64_t lddy,
                              const void *u, int64_t ldu, const float *w, const float *b,
                              const void *res, int64_t ldres, void *dx, int64_t lddx, void *du,
                              int64_t lddu, void *y, int64_t ldy, float *part_w, float *part_b,
                              float *mid, float *dw, float *db,
                              int64_t rows, int cols, float eps, hipStream_t st)
{
    const int nb = ln_bwd_blocks(rows);
    if (nb == 0) return hipSuccess;
    if (cols % 8 != 0 || cols > 2048) return hipErrorInvalidValue;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)nb), dim3(256), 0, st, (const uint16_t *)x, ldx,
                           (const uint16_t *)dy, lddy, (const uint16_t *)u, ldu, w, b,
                           (const uint16_t *)res, ldres, (uint16_t *)dx, lddx, (uint16_t *)du,
                           lddu, (uint16_t *)y, ldy, part_w, part_b, rows, cols, eps);
    };
    if (gated) {
        if (cols <= 512) go(ln_bwd_kernel<true, 1>);
        else if (cols <= 1024) go(ln_bwd_kernel<true, 2>);
        else go(ln_bwd_kernel<true, 4>);
    } else {
        if (cols <= 512) go(ln_bwd_kernel<false, 1>);
        else if (cols <= 1024) go(ln_bwd_kernel<false, 2>);
        else go(ln_bwd_kernel<false, 4>);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = sum_splits(part_w, (int64_t)cols, nb, dw, mid, st);
    if (e != hipSuccess || !db) return e;
    return sum_splits(part_b, (int64_t)cols, nb, db, mid, st);
}

// ---------------------------------------------------------------------------
// dz = ds * SiLU'(z), in place on ds, over [T][C] (C a multiple of 8)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dsilu_kernel(uint16_t *ds, int64_t ldd, const uint16_t *z,
                                                    int64_t ldz, int64_t rows, int cols)
{
    const int cpr = cols / 8;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * cpr) return;
    const int64_t r = i / cpr;
    const int c = (int)(i % cpr);
    float dv[8], zv[8];
    unpack8(ld16(ds + r * ldd + 8 * c), dv);
    unpack8(ld16(z + r * ldz + 8 * c), zv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // sigma(z) (1 + z (1 - sigma(z))); exp(-z) overflowing to inf gives
        // sigma = 0 and a zero derivative, the limit
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * zv[e]));
        dv[e] *= sg * (1.0f + zv[e] * (1.0f - sg));
    }
    *reinterpret_cast<uint4 *>(ds + r * ldd + 8 * c) = pack8(dv);
}

hipError_t launch_dsilu_bf16(void *ds, int64_t ldd, const void *z, int64_t ldz, int64_t rows,
                             int cols, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    if (cols % 8 != 0) return hipErrorInvalidValue;
    const int64_t n = rows * (cols / 8);
    hipLaunchKernelGGL(dsilu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (uint16_t *)ds, ldd, (const uint16_t *)z, ldz, rows, cols);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dst[c][r] = src[r][c] for a [R][C] bf16 matrix (R, C multiples of 64)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *src, int R, int C,
                                                        uint16_t *dst)
{
    __shared__ uint16_t tile[64][66];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int r = i / 64, c = i % 64;
        tile[r][c] = src[(int64_t)(r0 + r) * C + c0 + c];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int c = i / 64, r = i % 64;
        dst[(int64_t)(c0 + c) * R + r0 + r] = tile[r][c];
    }
}

hipError_t launch_transpose_bf16(const void *src, int R, int C, void *dst, hipStream_t st)
{
    if (R % 64 != 0 || C % 64 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)(C / 64), (unsigned)(R / 64)), dim3(256), 0,
                       st, (const uint16_t *)src, R, C, (uint16_t *)dst);
    return hipGetLastError();
}

// dst[0 .. n) = v
__global__ __launch_bounds__(256) void fill_f32_kernel(float *dst, int64_t n, float v)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = v;
}

hipError_t launch_fill_f32(float *dst, size_t n, float v, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dst,
                       (int64_t)n, v);
    return hipGetLastError();
}

}  // namespace sla
