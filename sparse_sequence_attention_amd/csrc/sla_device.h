// sla_device.h -- CDNA4 (gfx950) device helpers for the SLA kernels: bf16
// vectors, the 32x32x16 bf16 MFMA, LDS swizzles, the pointwise SiLU and its
// derivative in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sla_internal.h"

namespace sla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef uint16_t bf16_t;  // bf16 storage as raw bits on the host-visible side

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l holds A[m = l%32][k-slot 8*(l/32) .. +8], B[k-slot ..][n = l%32];
// the accumulator register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
// The k slots only have to agree between A and B; kernels choose which logical
// index each slot carries.
__device__ __forceinline__ floatx16 mfma32(const bf16x8 &a, const bf16x8 &b, const floatx16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Same shape with fp16 operands.  The second product of each attention pair
// (P.V, P^T.dO, dS^T.Q, dS.K) runs in fp16: its computed operand (P or dS) is
// rounded to 11 significant bits instead of bf16's 8, which keeps the bf16
// outputs within their error budget; the partner input is converted to fp16
// when it is staged into LDS.
__device__ __forceinline__ floatx16 mfma32h(const halfx8 &a, const halfx8 &b, const floatx16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 zero16()
{
    floatx16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 as_u4(const bf16x8 &b) { return __builtin_bit_cast(uint4, b); }

// 8 fp32 -> 8 bf16 (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x8 cvt8(float a0, float a1, float a2, float a3, float a4, float a5,
                                       float a6, float a7)
{
    floatx2 p0 = {a0, a1}, p1 = {a2, a3}, p2 = {a4, a5}, p3 = {a6, a7};
    bf16x2 b0 = __builtin_convertvector(p0, bf16x2);
    bf16x2 b1 = __builtin_convertvector(p1, bf16x2);
    bf16x2 b2 = __builtin_convertvector(p2, bf16x2);
    bf16x2 b3 = __builtin_convertvector(p3, bf16x2);
    bf16x8 r;
    r[0] = b0[0]; r[1] = b0[1]; r[2] = b1[0]; r[3] = b1[1];
    r[4] = b2[0]; r[5] = b2[1]; r[6] = b3[0]; r[7] = b3[1];
    return r;
}

__device__ __forceinline__ halfx8 as_halfx8(const uint4 &u) { return __builtin_bit_cast(halfx8, u); }

// 8 fp32 -> 8 fp16 (round to nearest even; v_cvt_pk_f16_f32).
__device__ __forceinline__ halfx8 cvt8h(float a0, float a1, float a2, float a3, float a4, float a5,
                                        float a6, float a7)
{
    floatx2 p0 = {a0, a1}, p1 = {a2, a3}, p2 = {a4, a5}, p3 = {a6, a7};
    halfx2 b0 = __builtin_convertvector(p0, halfx2);
    halfx2 b1 = __builtin_convertvector(p1, halfx2);
    halfx2 b2 = __builtin_convertvector(p2, halfx2);
    halfx2 b3 = __builtin_convertvector(p3, halfx2);
    halfx8 r;
    r[0] = b0[0]; r[1] = b0[1]; r[2] = b1[0]; r[3] = b1[1];
    r[4] = b2[0]; r[5] = b2[1]; r[6] = b3[0]; r[7] = b3[1];
    return r;
}

__device__ __forceinline__ uint32_t cvt2h_u32(float a, float b)
{
    floatx2 p = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, halfx2));
}

__device__ __forceinline__ uint2 cvt4_u2(float a0, float a1, float a2, float a3)
{
    floatx2 p0 = {a0, a1}, p1 = {a2, a3};
    bf16x2 b0 = __builtin_convertvector(p0, bf16x2);
    bf16x2 b1 = __builtin_convertvector(p1, bf16x2);
    uint2 r;
    r.x = __builtin_bit_cast(uint32_t, b0);
    r.y = __builtin_bit_cast(uint32_t, b1);
    return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// Pointwise activation in registers.  With t = alpha*s and
// e = 2^(t * -log2(e)) = exp(-t):  sigma = 1 / (1 + e),  SiLU(t) = t * sigma.
// The forward keeps s * sigma and applies alpha once, with 1/N, to the output.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigmoid_fast(float s, float neg_alpha_log2e)
{
    float e = __builtin_amdgcn_exp2f(s * neg_alpha_log2e);
    return __builtin_amdgcn_rcpf(1.0f + e);
}

// sigma and e = exp(-alpha s); 1 - sigma = e * sigma without cancellation.
// The exponent is capped at 2^100 so that e * sigma stays finite for very
// negative alpha s (where sigma and SiLU' are 0 to fp32 precision anyway);
// uncapped, e = inf and sigma = 0 would make e * sigma a NaN.
__device__ __forceinline__ float sigmoid_e(float s, float neg_alpha_log2e, float &e)
{
    e = __builtin_amdgcn_exp2f(fminf(s * neg_alpha_log2e, 100.0f));
    return __builtin_amdgcn_rcpf(1.0f + e);
}

// Multiply 8 bf16 values by a power of two (exact unless out of range).
__device__ __forceinline__ bf16x8 scale_bf16x8(const bf16x8 &x, float sc)
{
    uint4 u = as_u4(x);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(w[i]) * sc;
        f[2 * i + 1] = bf16_hi(w[i]) * sc;
    }
    return cvt8(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
}

// 8 bf16 -> 8 fp16 (exact for |x| in fp16's normal range).
__device__ __forceinline__ halfx8 bf16x8_to_halfx8(const bf16x8 &x)
{
    uint4 u = as_u4(x);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
    return cvt8h(bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1]), bf16_lo(w[2]),
                 bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3]));
}

// ---------------------------------------------------------------------------
// Memory helpers
// ---------------------------------------------------------------------------
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4_t;

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane
// l's 16 bytes from `src` land at lds_wave_base + 16 * l.  lds_wave_base must
// be the same in every lane of the wave.  Completion is tracked by vmcnt only:
// wait with vm_wait before the barrier that publishes the data.
__device__ __forceinline__ void gl_lds16(const void *src, uint16_t *lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)lds_wave_base, 16, 0, 0);
}

// As gl_lds16, for data read exactly once: the non-temporal hint keeps it
// from displacing reused data in the caches.
__device__ __forceinline__ void gl_lds16_nt(const void *src, uint16_t *lds_wave_base)
{
    constexpr int kNonTemporal = 2;  // cache-policy bit NT
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)lds_wave_base, 16, 0, kNonTemporal);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
// The s_waitcnt builtin (rather than inline asm) lets the compiler's own wait
// tracking see the wait, so it adds no conservative vmcnt(0) later; the empty
// asm statements with a memory clobber keep every memory access on its side.
// gfx9 encoding: vmcnt[3:0] and [15:14], expcnt[6:4] and lgkmcnt[11:8] (the
// latter two left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// Workgroup barrier for LDS filled by DMA only, without the memory fence of
// __syncthreads: the fence would make every wave also wait for the DMA of
// later stages in flight.  The caller waits (vm_wait) for the DMA it
// publishes; the memory clobber keeps the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void barrier_lds_dma()
{
    asm volatile("s_barrier" ::: "memory");
}

// Instruction classes of __builtin_amdgcn_sched_group_barrier (LLVM AMDGPU
// IGroupLP masks): a sequence of (class, count) groups in one basic block
// asks the scheduler to emit that many instructions of each class in that
// order, which interleaves independent MFMA and VALU work of one wave.
constexpr int SG_VALU = 0x002 | 0x400;  // vector ALU, transcendentals included
constexpr int SG_MFMA = 0x008;
constexpr int SG_VMEM_READ = 0x020;     // global loads, DMA into LDS included
constexpr int SG_DS_READ = 0x100;

// Workgroup barrier that publishes this wave's LDS writes (and waits for its
// LDS reads) but leaves global loads and stores, including DMA into other
// LDS buffers, in flight; __syncthreads' fence would wait for those too.
__device__ __forceinline__ void barrier_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j points at 4 consecutive 16-bit values (an 8-byte run) and lane i
// receives value i % 4 of the runs of lanes i / 4, 4 + i / 4, 8 + i / 4 and
// 12 + i / 4.  With lane j pointing at run (row r0 + j / 4, columns
// c0 + 4 * (j % 4) .. + 3) of a row-major [row][col] tile, lane i receives
// column c0 + i of rows r0 .. r0 + 3: a 4-deep slice of an MFMA operand whose
// contraction index runs along the tile's rows.
__device__ __forceinline__ uint2 tr_read_b64(const uint16_t *lds_run)
{
    shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)lds_run);
    return __builtin_bit_cast(uint2, v);
}

// Chunk (16 bytes) of a stored 64-row x 128-key dS block holding lane (kl, hl)'s
// 8 values of row group qc for the keys of wave wv of the dK/dV kernel: the
// fp16 operand that kernel feeds its dK product, stored as it is held.  Key
// kl of the wave, rows 32*(qc/2) + 16*(qc%2) + 4*hl + {0..3, 8..11}.  The
// lane pairs are interleaved and odd row groups shifted by 128 bytes so that
// the transposing reads of the dQ kernel hit distinct banks.
__host__ __device__ inline int ds_frag_chunk(int wv, int qc, int kl, int hl)
{
    return (wv * 4 + qc) * 64 + ((2 * kl + hl) ^ (8 * (qc & 1)));
}
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// 16-byte store marked non-temporal (streamed out, not kept in the caches):
// for data written once and read back only by a later kernel.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st16_nt(void *p, const halfx8 &v)
{
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t *>(p));
}
__device__ __forceinline__ uint4 ld16_or_zero(const void *p, bool ok)
{
    uint4 z = {0u, 0u, 0u, 0u};
    return ok ? *reinterpret_cast<const uint4 *>(p) : z;
}

// 16 bytes at column `col` of row r of a [rows][ld] bf16 tensor, zero when
// r >= limit.  The load itself is unconditional (row clamped to limit-1, which
// the caller guarantees is >= 0) so it stays one 16-byte load; the zeroing is
// a select.
__device__ __forceinline__ uint4 ld16_row(const uint16_t *base, int64_t ld, int r, int limit,
                                          int col)
{
    const int rr = r < limit ? r : limit - 1;
    uint4 v = *reinterpret_cast<const uint4 *>(base + (int64_t)rr * ld + col);
    const bool ok = r < limit;
    v.x = ok ? v.x : 0u;
    v.y = ok ? v.y : 0u;
    v.z = ok ? v.z : 0u;
    v.w = ok ? v.w : 0u;
    return v;
}

// Row r of a [tokens][ld] bf16 tensor, clamped to row limit - 1 (limit >= 1):
// a plain 16-byte load with no use of its value until the caller consumes it,
// so it stays in flight; rows at or past `limit` hold a copy of the last valid
// row, which the caller masks out.
__device__ __forceinline__ uint4 ld16_clamped(const uint16_t *base, int64_t ld, int r, int limit,
                                              int col)
{
    const int rr = r < limit ? r : limit - 1;
    return *reinterpret_cast<const uint4 *>(base + (int64_t)rr * ld + col);
}

// 16-byte chunk swizzle for a row-major tile whose rows hold `cpr` chunks: the
// chunk index is XORed with the low bits of the row so that 8 consecutive rows
// read at the same logical chunk hit 8 different bank groups.
template <int CPR>
__device__ __forceinline__ int swz_row(int row, int chunk)
{
    constexpr int m = (CPR >= 8 ? 8 : CPR) - 1;
    return chunk ^ (row & m);
}

// Swizzle for the transposed tiles ([d][key] with 64-key rows = 8 chunks):
// consecutive d of one aligned group of 8 land in distinct bank groups, and
// rows 8 apart also differ.
__device__ __forceinline__ int swz_t(int d, int chunk) { return chunk ^ ((d ^ (d >> 3)) & 7); }

// Position of key k (0..63) inside a transposed 64-key row.  Within every 16-key
// group the 4-key blocks are stored in the order 0, 2, 1, 3, which is the order
// in which the 32x32 MFMA accumulator hands a lane its keys (rows
// 8*(r/4) + 4*half + r%4): a lane's 8 operand slots then read one 16-byte chunk.
__device__ __forceinline__ int tpos(int k)
{
    int kb4 = (k >> 2) & 3;
    int pb = ((kb4 & 1) << 1) | (kb4 >> 1);
    return (k & ~15) | (pb << 2) | (k & 3);
}

// Select the low (sel = 0x05040100) or high (0x07060302) bf16 halves of two
// words: result = lo-word half | hi-word half << 16.
__device__ __forceinline__ uint32_t pack_halves(uint32_t lo_word, uint32_t hi_word, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi_word, lo_word, sel);
}

}  // namespace sla
