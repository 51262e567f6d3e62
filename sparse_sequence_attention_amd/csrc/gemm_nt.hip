// gemm_nt.hip -- the STU projections' GEMM, C[M][N] = epi(A[M][K] . W[N][K]^T),
// with bf16 or FP8 E4M3 operands (both K-contiguous, as a Linear layer's
// input and weight), fp32 accumulation and a bf16 output.
//
// Tile BMT (M) x BN (N) per workgroup of NWV waves, each 64 x BN / (NWV / (BMT
// / 64)): 256 x 128 with 8 waves (4 x 2), or 128 x 128 with 4 waves (2 x 2)
// for products whose 256-row tiles would leave the GPU's workgroup slots
// part empty.
// Operands stream HBM -> LDS by DMA (global_load_lds) through a ring of three
// or four stages of 64 bytes of K (32 bf16 or 64 fp8 values) per row, the
// next stages in flight while one is multiplied, one barrier per stage; stage rows
// are 64 bytes, chunk c of row r stored at c ^ f(r) so that the 16-lane
// passes of the operand reads hit distinct banks.
//
// The waves compute C^T blocks (W rows as the MFMA A operand, A rows as B).
// The W rows of a 32-row fragment are taken in the order that leaves each
// lane with 16 consecutive output columns of one row: the epilogue packs
// them into two 16-byte LDS writes, and the tile leaves LDS in whole
// 16-byte row chunks, so every global store is row-contiguous.
//
// Epilogues, with z = sa[m] sw[n] acc + bias[n] (sa, sw: FP8 row scales, 1
// for bf16): 0: SiLU(z); 1: z + R (residual, added in fp32 before the single
// rounding); 2: z; 3: SiLU(z), and z itself to Z.
#include <type_traits>

#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

namespace {

typedef int intx8_t __attribute__((ext_vector_type(8)));

constexpr int GB_RB = 64;   // bytes of K per stage row

// stage-row swizzle: 16-byte chunk c of row r sits at c ^ gswz(r)
__device__ __forceinline__ int gswz(int r)
{
    const int x = r >> 2;
    return (x ^ (((x >> 2) & 1) << 1)) & 3;
}

// W row of fragment row j (0..31) that leaves accumulator register r of
// lane half h with output column 16 h + r
__device__ __forceinline__ int wperm(int j)
{
    return 16 * ((j >> 2) & 1) + 4 * (j >> 3) + (j & 3);
}

// NS stages (3 or 4); MINB workgroups per CU (MINB x NS x STAGE bytes of
// LDS); BMT rows of A per tile with NWV waves
template <bool FP8, int BN, int EPI, int NS, int MINB, int BMT, int NWV>
__global__ __launch_bounds__(64 * NWV, MINB) void gemm_nt_kernel(
    const uint8_t *A, int64_t lda, const float *sa, const uint8_t *W, int64_t ldw,
    const float *sw, const float *bias, const uint16_t *R, int64_t ldr, uint16_t *C, int64_t ldc,
    uint16_t *Z, int64_t ldz, int64_t M, int N, int Kb)
{
    constexpr int GB_M = BMT;                 // rows of A per tile
    constexpr int WM = BMT / 64, WN = NWV / WM;  // wave grid: 64-row groups x column groups
    constexpr int WCOLS = BN / WN;            // columns per wave
    constexpr int ROWS = GB_M + BN;           // stage rows: A then W
    constexpr int STAGE = ROWS * GB_RB;       // bytes
    constexpr int PER = ROWS / 16 / NWV;      // DMA instructions per thread and stage
    constexpr int NBW = WCOLS / 32;           // 32-column fragments per wave
    static_assert(WM * WN == NWV && WCOLS == 64, "64 x 64 per wave");
    static_assert(ROWS % (16 * NWV) == 0, "whole DMA rounds");
    static_assert(NS == 3 || NS == 4, "three or four stages");
    __shared__ __align__(16) uint8_t st0[STAGE], st1[STAGE], st2[STAGE];
    __shared__ __align__(16) uint8_t st3[NS == 4 ? STAGE : 16];

    const int ntn = N / BN;
    const int64_t ntm = (M + GB_M - 1) / GB_M;
    const int item = xcd_remap(blockIdx.x, (int)(ntm * ntn));
    if (item < 0) return;
    const int64_t m0 = (int64_t)(item / ntn) * GB_M;
    const int n0 = (item % ntn) * BN;

    const int tid = threadIdx.x, lane = tid & 63, wv = uniform(tid >> 6);
    const int l32 = lane & 31, hl = lane >> 5;
    const int wm = wv % WM, wn = wv / WM;

    auto stage = [&](auto S) -> uint8_t * {
        constexpr int s = decltype(S)::value;
        if constexpr (s == 0) return st0;
        else if constexpr (s == 1) return st1;
        else if constexpr (s == 2) return st2;
        else return st3;
    };

    // DMA of K bytes [kb, kb + 64) of the tile's A and W rows into a stage:
    // wave-chunk q = i * NWV + wv holds stage rows 16 q .. +16, lane -> row
    // 16 q + lane / 4, physical chunk lane % 4 (logical chunk ^ gswz)
    const int64_t mlast = M - 1;
    auto issue = [&](int kstep, auto S) {
        uint8_t *sb = stage(S);
        const int kb = kstep * GB_RB;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = i * NWV + wv;
            const int row = 16 * q + (lane >> 2);
            const int lc = (lane & 3) ^ gswz(row);
            const uint8_t *src;
            if (16 * q < GB_M) {
                const int64_t m = m0 + row < mlast ? m0 + row : mlast;
                src = A + m * lda + kb + 16 * lc;
            } else {
                src = W + (int64_t)(n0 + row - GB_M) * ldw + kb + 16 * lc;
            }
            gl_lds16(src, reinterpret_cast<uint16_t *>(sb + q * 1024));
        }
    };

    // operand fragment (16 bytes: one bf16 k16 slice, or half an fp8 k64 slice)
    auto frag = [&](const uint8_t *sb, int row, int lc) {
        return *reinterpret_cast<const uint4 *>(sb + row * GB_RB + 16 * (lc ^ gswz(row)));
    };

    floatx16 acc[NBW][2];  // [n fragment][m fragment] of C^T
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

    const int wrow0 = GB_M + wn * WCOLS;     // this wave's first W stage row
    const int arow0 = 64 * wm;               // and first A stage row
    auto compute = [&](auto S) {
        const uint8_t *sb = stage(S);
        if constexpr (FP8) {
            intx8_t wa[NBW], xb[2];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int r = wrow0 + 32 * nb + wperm(l32);
                const uint4 lo = frag(sb, r, 2 * hl), hi = frag(sb, r, 2 * hl + 1);
                wa[nb] = intx8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int r = arow0 + 32 * mb + l32;
                const uint4 lo = frag(sb, r, 2 * hl), hi = frag(sb, r, 2 * hl + 1);
                xb[mb] = intx8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        wa[nb], xb[mb], acc[nb][mb], 0, 0, 0, 0, 0, 0);
        } else {
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                bf16x8 wa[NBW], xb[2];
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                    wa[nb] = as_bf16x8(frag(sb, wrow0 + 32 * nb + wperm(l32), 2 * kc + hl));
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    xb[mb] = as_bf16x8(frag(sb, arow0 + 32 * mb + l32, 2 * kc + hl));
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = mfma32(wa[nb], xb[mb], acc[nb][mb]);
            }
        }
    };

    // main loop: stage k % NS holds K step k; the next NS - 2 steps (and,
    // after this step's issue, NS - 1) are in flight.  The DMAs are issued
    // unconditionally (past the last step they reload it into a stage nobody
    // reads any more): a DMA under a branch makes the compiler wait for all
    // of them at the merge, which would serialise the ring.
    const int nk = Kb / GB_RB;
    auto step = [&](int k, auto S) {
        constexpr int s = decltype(S)::value;
        vm_wait<(NS - 2) * PER>();  // this thread's stage-k DMAs have landed
        barrier_lds();              // everyone's have; stage k - 1 is free
        issue(imin(k + NS - 1, nk - 1), std::integral_constant<int, (s + NS - 1) % NS>{});
        compute(S);
    };
    issue(0, std::integral_constant<int, 0>{});
    issue(imin(1, nk - 1), std::integral_constant<int, 1>{});
    if constexpr (NS == 4) issue(imin(2, nk - 1), std::integral_constant<int, 2>{});
    // whole groups of NS steps without branches (a branch between steps
    // costs the same conservative wait), then the remainder
    const int ng = nk / NS;
    for (int g = 0; g < ng; ++g) {
        step(NS * g, std::integral_constant<int, 0>{});
        step(NS * g + 1, std::integral_constant<int, 1>{});
        step(NS * g + 2, std::integral_constant<int, 2>{});
        if constexpr (NS == 4) step(NS * g + 3, std::integral_constant<int, 3 % NS>{});
    }
    const int rem = uniform(nk - NS * ng);
    if (rem > 0) step(NS * ng, std::integral_constant<int, 0>{});
    if (rem > 1) step(NS * ng + 1, std::integral_constant<int, 1>{});
    if constexpr (NS == 4)
        if (rem > 2) step(NS * ng + 2, std::integral_constant<int, 2>{});

    // epilogue: lane holds row m = 64 wm + 32 mb + l32 and, per n fragment,
    // columns 16 hl + 0..15 of its 32.  Every wave stages its own 64 x BN/2
    // block in a private slice of the (now idle) stages, 16-byte chunk c of
    // block row r at c ^ eswz(r), and stores it back out in row chunks; no
    // barrier after the first (within a wave, LDS accesses complete in
    // order).  EPI 3 does it twice (SiLU(z) to C, then z to Z).
    constexpr int CPW = WCOLS / 8;        // 16-byte chunks per block row
    constexpr int SLICE = 64 * CPW * 16;  // bytes per wave
    constexpr int SPS = STAGE / SLICE;  // wave slices per stage
    static_assert(SPS * NS >= NWV, "every wave has a slice");
    uint8_t *slice;
    switch (wv / SPS) {
    case 0: slice = st0; break;
    case 1: slice = st1; break;
    case 2: slice = st2; break;
    default: slice = st3; break;
    }
    slice += (wv % SPS) * SLICE;
    auto eswz = [](int r) { return CPW == 16 ? (r & 15) : ((r >> 1) & (CPW - 1)); };
    auto spos = [&](int r, int c) { return slice + r * (CPW * 16) + 16 * (c ^ eswz(r)); };
    vm_wait<0>();
    __syncthreads();  // every wave is done with the stages
    constexpr int PASSES = EPI == 3 ? 2 : 1;
#pragma unroll
    for (int out = 0; out < PASSES; ++out) {
        uint16_t *dst = out == 0 ? C : Z;
        const int64_t ldd = out == 0 ? ldc : ldz;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int rl = 32 * mb + l32;  // block row
            const int64_t m = m0 + 64 * wm + rl;
            const float am = FP8 ? (m < M ? sa[m] : 0.0f) : 1.0f;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int cl = 32 * nb + 16 * hl;  // first column in the block
                const int n = n0 + wn * WCOLS + cl;
                float o[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float v = acc[nb][mb][r];
                    if (FP8) v *= am * sw[n + r];
                    o[r] = v + (bias ? bias[n + r] : 0.0f);
                }
                if ((EPI == 0) || (EPI == 3 && out == 0)) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        o[r] = o[r] * sigmoid_fast(o[r], -1.4426950408889634f);
                }
                if (EPI == 1 && m < M) {
                    const uint4 r0 = *reinterpret_cast<const uint4 *>(R + m * ldr + n);
                    const uint4 r1 = *reinterpret_cast<const uint4 *>(R + m * ldr + n + 8);
                    const uint32_t rw[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        o[2 * e] += bf16_lo(rw[e]);
                        o[2 * e + 1] += bf16_hi(rw[e]);
                    }
                }
                uint2 p[4];
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    p[g] = cvt4_u2(o[4 * g], o[4 * g + 1], o[4 * g + 2], o[4 * g + 3]);
                *reinterpret_cast<uint4 *>(spos(rl, cl / 8)) = make_uint4(p[0].x, p[0].y, p[1].x, p[1].y);
                *reinterpret_cast<uint4 *>(spos(rl, cl / 8 + 1)) =
                    make_uint4(p[2].x, p[2].y, p[3].x, p[3].y);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's staging writes done
        // the block leaves in 16-byte row chunks: 64 lanes cover 64 / CPW rows per pass
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int c = i * 64 + lane;
            const int rl = c / CPW, ch = c % CPW;
            const int64_t m = m0 + 64 * wm + rl;
            const uint4 v = *reinterpret_cast<const uint4 *>(spos(rl, ch));
            if (m < M) *reinterpret_cast<uint4 *>(dst + m * ldd + n0 + wn * WCOLS + 8 * ch) = v;
        }
        if (EPI == 3 && out == 0) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next writes
        }
    }
}

template <bool FP8, int BN, int NS, int MINB, int BMT, int NWV>
hipError_t launch_nt(const void *A, int64_t lda, const float *sa, const void *W, int64_t ldw,
                     const float *sw, const float *bias, const void *R, int64_t ldr, void *C,
                     int64_t ldc, void *Z, int64_t ldz, int64_t M, int N, int Kb, int epi,
                     hipStream_t st)
{
    const int64_t tiles = ((M + BMT - 1) / BMT) * (N / BN);
    dim3 grid((unsigned)tiles), block(64 * NWV);
#define GNT_ARGS                                                                               \
    (const uint8_t *)A, lda, sa, (const uint8_t *)W, ldw, sw, bias, (const uint16_t *)R, ldr, \
        (uint16_t *)C, ldc, (uint16_t *)Z, ldz, M, N, Kb
    switch (epi) {
    case 0: hipLaunchKernelGGL((gemm_nt_kernel<FP8, BN, 0, NS, MINB, BMT, NWV>), grid, block, 0, st, GNT_ARGS); break;
    case 1: hipLaunchKernelGGL((gemm_nt_kernel<FP8, BN, 1, NS, MINB, BMT, NWV>), grid, block, 0, st, GNT_ARGS); break;
    case 2: hipLaunchKernelGGL((gemm_nt_kernel<FP8, BN, 2, NS, MINB, BMT, NWV>), grid, block, 0, st, GNT_ARGS); break;
    default: hipLaunchKernelGGL((gemm_nt_kernel<FP8, BN, 3, NS, MINB, BMT, NWV>), grid, block, 0, st, GNT_ARGS); break;
    }
#undef GNT_ARGS
    return hipGetLastError();
}

// whether a bf16 product takes the 128-row tiles: when its 256-row tiles
// would number fewer than 1024 (two rounds of 512 workgroup slots on 256
// CUs).  Measured on the STU layer's products (one box): 128-row tiles take
// the truncated layers' UVQK (M = 8832, N = 2048) from 37.2 to 35.2 us, the
// output projection (M = 21,930, N = 512) from 27.0 to 25.8 us and the
// backward's dn (K = 2048) from 67.2 to 65.4 us; the full-length UVQK (1376
// tiles of 256 rows) is faster with 256-row tiles (78-80 against 83 us).
static bool gemm_small_tiles(int64_t M, int N)
{
    return ((M + 255) / 256) * (N / 128) < 1024;
}

// bf16: 256 x 128 tiles in a three-stage ring, two workgroups per CU (one
// workgroup's epilogue runs under the other's products; measured faster than
// 256 x 256 tiles with one workgroup per CU on every projection shape of the
// layer), or 128 x 128 tiles of four waves, three workgroups per CU, for the
// smaller products (gemm_small_tiles).  FP8: the operand fragments take twice the registers, so 256 x 128
// tiles with four stages and one workgroup per CU.
template <bool FP8>
hipError_t launch_nt_any(const void *A, int64_t lda, const float *sa, const void *W, int64_t ldw,
                         const float *sw, const float *bias, const void *R, int64_t ldr, void *C,
                         int64_t ldc, void *Z, int64_t ldz, int64_t M, int N, int Kb, int epi,
                         hipStream_t st)
{
    if constexpr (!FP8) {
        if (gemm_small_tiles(M, N))
            return launch_nt<FP8, 128, 3, 3, 128, 4>(A, lda, sa, W, ldw, sw, bias, R,
                                                                   ldr, C, ldc, Z, ldz, M, N, Kb,
                                                                   epi, st);
        return launch_nt<FP8, 128, 3, 2, 256, 8>(A, lda, sa, W, ldw, sw, bias, R, ldr, C, ldc, Z,
                                                 ldz, M, N, Kb, epi, st);
    } else {
        return launch_nt<FP8, 128, 4, 1, 256, 8>(A, lda, sa, W, ldw, sw, bias, R, ldr, C, ldc, Z,
                                                 ldz, M, N, Kb, epi, st);
    }
}

}  // namespace

hipError_t launch_gemm_nt_bf16(const void *A, int64_t lda, const void *W, int64_t ldw,
                               const float *bias, const void *R, int64_t ldr, void *C, int64_t ldc,
                               void *Z, int64_t ldz, int64_t M, int N, int K, int epi,
                               hipStream_t st)
{
    if (M <= 0) return hipSuccess;
    if (N % 128 != 0 || K % 32 != 0 || epi < 0 || epi > 3) return hipErrorInvalidValue;
    if ((epi == 1 && !R) || (epi == 3 && !Z)) return hipErrorInvalidValue;
    if ((lda % 8) || (ldw % 8) || (ldc % 8) || (epi == 1 && ldr % 8) || (epi == 3 && ldz % 8))
        return hipErrorInvalidValue;
    return launch_nt_any<false>(A, lda * 2, nullptr, W, ldw * 2, nullptr, bias, R, ldr, C, ldc, Z,
                                ldz, M, N, K * 2, epi, st);
}

hipError_t launch_gemm_nt_fp8(const void *A, const float *sa, const void *W, const float *sw,
                              const float *bias, const void *R, int64_t ldr, void *C, int64_t ldc,
                              int64_t M, int N, int K, int epi, hipStream_t st)
{
    if (M <= 0) return hipSuccess;
    if (N % 128 != 0 || K % 64 != 0 || epi < 0 || epi > 3 || epi == 3) return hipErrorInvalidValue;
    if (epi == 1 && (!R || ldr % 8)) return hipErrorInvalidValue;
    if (ldc % 8) return hipErrorInvalidValue;
    return launch_nt_any<true>(A, K, sa, W, K, sw, bias, R, ldr, C, ldc, nullptr, 0, M, N, K, epi,
                               st);
}

}  // namespace sla
