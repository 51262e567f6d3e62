// sla_device.h -- CDNA4 (gfx950) device helpers for the SLA kernels: bf16
// vectors, the 32x32x16 bf16 MFMA, LDS swizzles, the pointwise SiLU and its
// derivative in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sla_internal.h"

namespace sla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l holds A[m = l%32][k-slot 8*(l/32) .. +8], B[k-slot ..][n = l%32];
// the accumulator register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
// The k slots only have to agree between A and B; kernels choose which logical
// index each slot carries.
__device__ __forceinline__ floatx16 mfma32(const bf16x8 &a, const bf16x8 &b, const floatx16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// ---------------------------------------------------------------------------
// Memory helpers
// ---------------------------------------------------------------------------
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4_t;


// Direct HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane
// l's 16 bytes from `src` land at lds_wave_base + 16 * l.  lds_wave_base must
// be the same in every lane of the wave.  Completion is tracked by vmcnt only:
// wait with vm_wait before the barrier that publishes the data.
__device__ __forceinline__ void gl_lds16(const void *src, uint16_t *lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_wave_base, 16, 0, 0);
}

// As gl_lds16, issued through inline assembly so that the compiler does not
// see an LDS write: it then adds no wait counts of its own between this DMA
// and later LDS reads (its alias tracking of DMA targets is lost at branch
// joins, after which it waits for every DMA in flight before any LDS read).
// The caller orders the data itself: vm_wait for its own DMAs, then a
// barrier, before any wave reads the destination.  M0 carries the LDS byte
// address of the wave's destination (wave-uniform; the kernels form these
// addresses once: the address-space cast of a generic pointer costs scalar
// instructions per call); lane l's 16 bytes from `src` land at that address
// + 16 * l.  No register is written, so nothing of the load's result is left
// for the compiler to reuse early.  The _stream form is non-temporal, for
// data read once (kept from displacing the L2 working set).
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

__device__ __forceinline__ void gl_lds16_at(const void *src, uint32_t lds_byte_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_byte_addr)
                 : "memory", "m0");
}

__device__ __forceinline__ void gl_lds16_at_stream(const void *src, uint32_t lds_byte_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(src), "s"(lds_byte_addr)
                 : "memory", "m0");
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

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// 16-byte streaming store through a global-address-space pointer
// (global_store_dwordx4 nt: data read once, by a later kernel, so it should
// not displace the working set of this one from the L2; a generic pointer
// would give a flat store, which the LDS wait counter tracks too).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st16_global_stream(void *p, const uint4 &v)
{
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (__attribute__((address_space(1))) u32x4 *)p);
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

}  // namespace sla
