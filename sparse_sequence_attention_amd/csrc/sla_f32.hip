// sla_f32.hip -- fp32 SLA forward and backward (plain FMA kernels).
//
// The fp32 path exists for small parity workloads that ask for single
// precision; it uses the same on-device schedule as the bf16 MFMA kernels but
// plain vector FMAs: four threads share one row (or key), each holding a
// quarter of the head dimension, and combine dot products with two lane
// shuffles.  Key/row tiles are staged in LDS.
//
// Semantics as in sla_fwd_bf16.hip / sla_bwd_bf16.hip (ULTRA-HSTU paper,
// section 3 Eq.3 and section 4.2.1 Eq.6-7): O_i = (1/N) sum_j SiLU(alpha
// q_i.k_j) v_j over visible pairs, and its gradients.
#include "sla_device.h"
#include "sla_kernels.h"

namespace sla {

constexpr int F32_TPR = 4;  // threads per row / key

__device__ __forceinline__ float quad_sum(float x)
{
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    return x;
}

__device__ __forceinline__ float silu_f32(float t) { return t / (1.0f + expf(-t)); }

// SiLU'(t) = sigma (1 + t (1 - sigma)) with 1 - sigma = e sigma, e = exp(-t), so
// that no cancellation occurs when sigma is close to 1.
__device__ __forceinline__ float dsilu_f32(float t)
{
    // e capped at exp(80): for t < -80, SiLU'(t) is 0 to fp32 precision, and
    // an infinite e would turn e * sg into a NaN
    const float e = expf(fminf(-t, 80.0f));
    const float sg = 1.0f / (1.0f + e);
    return sg * (1.0f + t * (e * sg));
}

// cooperative copy of rows [r0, r0+nrows) (zero past `limit`) of a [T][ld]
// fp32 tensor into a dense [nrows][D] LDS tile
template <int D>
__device__ __forceinline__ void stage_rows_f32(float *lds, const float *g, int64_t ld, int r0,
                                               int nrows, int limit)
{
    for (int e = threadIdx.x * 4; e < nrows * D; e += blockDim.x * 4) {
        const int r = e / D, c = e % D;
        float4 v = {0.f, 0.f, 0.f, 0.f};
        if (r0 + r < limit) v = *reinterpret_cast<const float4 *>(g + (int64_t)(r0 + r) * ld + c);
        *reinterpret_cast<float4 *>(lds + e) = v;
    }
}

// DQK: the Q / K head width, DV: the V width (DQ, DW: their shares per thread)
template <int DQK, int DV>
__global__ __launch_bounds__(FWD_BM *F32_TPR) void sla_fwd_f32_kernel(AttnParams p)
{
    constexpr int BM = FWD_BM, BN = FWD_BN, DQ = DQK / F32_TPR, DW = DV / F32_TPR;
    __shared__ __align__(16) float sk[BN * DQK];
    __shared__ __align__(16) float sv[BN * DV];
    const int nrec = p.s.fwd_base[p.B];
    const int item = xcd_remap(blockIdx.x, nrec * p.H);
    if (item < 0) return;
    const int h = item / nrec, rec = item - h * nrec;
    const int b = find_seq(p.s.fwd_base, p.B, rec);
    const SeqDims sd = seq_dims(p.offsets, p.num_targets, b);
    int r0, r1;
    row_tile(sd.L, sd.U, BM, rec - p.s.fwd_base[b], r0, r1);
    const TileCursor cur(fwd_key_ranges(sd.L, sd.U, p.k1, p.k2e, r0, r1, BN), BN);

    const float *qg = reinterpret_cast<const float *>(p.q) + sd.base * p.ldq + h * DQK;
    const float *kg = reinterpret_cast<const float *>(p.k) + sd.base * p.ldk + h * DQK;
    const float *vg = reinterpret_cast<const float *>(p.v) + sd.base * p.ldv + h * DV;
    const int row = threadIdx.x / F32_TPR, qt = threadIdx.x % F32_TPR;
    const int i = r0 + row;
    float q[DQ], acc[DW];
#pragma unroll
    for (int c = 0; c < DQ; ++c) q[c] = i < r1 ? qg[(int64_t)i * p.ldq + qt * DQ + c] : 0.0f;
#pragma unroll
    for (int c = 0; c < DW; ++c) acc[c] = 0.0f;
    for (int t = 0; t < cur.total; ++t) {
        const int c0 = cur.start(t, BN);
        __syncthreads();
        stage_rows_f32<DQK>(sk, kg, p.ldk, c0, BN, sd.L);
        stage_rows_f32<DV>(sv, vg, p.ldv, c0, BN, sd.L);
        __syncthreads();
        float part[DW];  // per-tile partial sums keep the rounding error growth short
#pragma unroll
        for (int c = 0; c < DW; ++c) part[c] = 0.0f;
        for (int jj = 0; jj < BN; ++jj) {
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < DQ; ++c) s += q[c] * sk[jj * DQK + qt * DQ + c];
            s = quad_sum(s);
            const bool vis = i < r1 && c0 + jj < sd.L && visible(i, c0 + jj, sd.U, p.k1, p.k2e);
            const float a = vis ? silu_f32(p.alpha * s) : 0.0f;
#pragma unroll
            for (int c = 0; c < DW; ++c) part[c] += a * sv[jj * DV + qt * DW + c];
        }
#pragma unroll
        for (int c = 0; c < DW; ++c) acc[c] += part[c];
    }
    if (i < r1) {
        float *o = reinterpret_cast<float *>(p.o) + (sd.base + i) * p.ldo + h * DV + qt * DW;
#pragma unroll
        for (int c = 0; c < DW; ++c) o[c] = acc[c] * p.inv_n;
    }
}

template <int DQK, int DV>
__global__ __launch_bounds__(FWD_BM *F32_TPR) void sla_bwd_dq_f32_kernel(AttnParams p)
{
    constexpr int BM = FWD_BM, BN = FWD_BN, DQ = DQK / F32_TPR, DW = DV / F32_TPR;
    __shared__ __align__(16) float sk[BN * DQK];
    __shared__ __align__(16) float sv[BN * DV];
    const int nrec = p.s.fwd_base[p.B];
    const int item = xcd_remap(blockIdx.x, nrec * p.H);
    if (item < 0) return;
    const int h = item / nrec, rec = item - h * nrec;
    const int b = find_seq(p.s.fwd_base, p.B, rec);
    const SeqDims sd = seq_dims(p.offsets, p.num_targets, b);
    int r0, r1;
    row_tile(sd.L, sd.U, BM, rec - p.s.fwd_base[b], r0, r1);
    const TileCursor cur(fwd_key_ranges(sd.L, sd.U, p.k1, p.k2e, r0, r1, BN), BN);

    const float *qg = reinterpret_cast<const float *>(p.q) + sd.base * p.ldq + h * DQK;
    const float *kg = reinterpret_cast<const float *>(p.k) + sd.base * p.ldk + h * DQK;
    const float *vg = reinterpret_cast<const float *>(p.v) + sd.base * p.ldv + h * DV;
    const float *gg = reinterpret_cast<const float *>(p.dout) + sd.base * p.lddo + h * DV;
    const int row = threadIdx.x / F32_TPR, qt = threadIdx.x % F32_TPR;
    const int i = r0 + row;
    float q[DQ], go[DW], acc[DQ];
#pragma unroll
    for (int c = 0; c < DQ; ++c) {
        q[c] = i < r1 ? qg[(int64_t)i * p.ldq + qt * DQ + c] : 0.0f;
        acc[c] = 0.0f;
    }
#pragma unroll
    for (int c = 0; c < DW; ++c) go[c] = i < r1 ? gg[(int64_t)i * p.lddo + qt * DW + c] : 0.0f;
    for (int t = 0; t < cur.total; ++t) {
        const int c0 = cur.start(t, BN);
        __syncthreads();
        stage_rows_f32<DQK>(sk, kg, p.ldk, c0, BN, sd.L);
        stage_rows_f32<DV>(sv, vg, p.ldv, c0, BN, sd.L);
        __syncthreads();
        float part[DQ];
#pragma unroll
        for (int c = 0; c < DQ; ++c) part[c] = 0.0f;
        for (int jj = 0; jj < BN; ++jj) {
            float s = 0.0f, g = 0.0f;
#pragma unroll
            for (int c = 0; c < DQ; ++c) s += q[c] * sk[jj * DQK + qt * DQ + c];
#pragma unroll
            for (int c = 0; c < DW; ++c) g += go[c] * sv[jj * DV + qt * DW + c];
            s = quad_sum(s);
            g = quad_sum(g);
            const bool vis = i < r1 && c0 + jj < sd.L && visible(i, c0 + jj, sd.U, p.k1, p.k2e);
            const float ds = vis ? g * dsilu_f32(p.alpha * s) : 0.0f;
#pragma unroll
            for (int c = 0; c < DQ; ++c) part[c] += ds * sk[jj * DQK + qt * DQ + c];
        }
#pragma unroll
        for (int c = 0; c < DQ; ++c) acc[c] += part[c];
    }
    if (i < r1) {
        float *o = reinterpret_cast<float *>(p.dq) + (sd.base + i) * p.lddq + h * DQK + qt * DQ;
#pragma unroll
        for (int c = 0; c < DQ; ++c) o[c] = acc[c] * p.out_scale;
    }
}

template <int DQK, int DV>
__global__ __launch_bounds__(BWD_BN *F32_TPR) void sla_bwd_dkdv_f32_kernel(AttnParams p)
{
    constexpr int BN = BWD_BN, BM = BWD_BM, DQ = DQK / F32_TPR, DW = DV / F32_TPR;
    constexpr int W = DQK + DV;  // a partial row: [dK | dV]
    __shared__ __align__(16) float sq[BM * DQK];
    __shared__ __align__(16) float sg_[BM * DV];
    const int nrec = p.s.bwd_base[p.B];
    const int item = xcd_remap(blockIdx.x, nrec * p.H);
    if (item < 0) return;
    const int h = item / nrec, rec = item - h * nrec;
    const int b = find_seq(p.s.bwd_base, p.B, rec);
    const SeqDims sd = seq_dims(p.offsets, p.num_targets, b);
    int np, nch;
    bwd_items(sd.L, sd.U, p.k2e, BN, BM, np, nch);
    const BwdItem it = bwd_item(sd.L, sd.U, p.k1, p.k2e, BN, BM, rec - p.s.bwd_base[b], np, nch);

    const float *qg = reinterpret_cast<const float *>(p.q) + sd.base * p.ldq + h * DQK;
    const float *kg = reinterpret_cast<const float *>(p.k) + sd.base * p.ldk + h * DQK;
    const float *vg = reinterpret_cast<const float *>(p.v) + sd.base * p.ldv + h * DV;
    const float *gg = reinterpret_cast<const float *>(p.dout) + sd.base * p.lddo + h * DV;
    const int kl = threadIdx.x / F32_TPR, qt = threadIdx.x % F32_TPR;
    const int j = it.c0 + kl;
    const bool jok = j < it.c1;
    float kr[DQ], vr[DW], dk[DQ], dv[DW];
#pragma unroll
    for (int c = 0; c < DQ; ++c) {
        kr[c] = jok ? kg[(int64_t)j * p.ldk + qt * DQ + c] : 0.0f;
        dk[c] = 0.0f;
    }
#pragma unroll
    for (int c = 0; c < DW; ++c) {
        vr[c] = jok ? vg[(int64_t)j * p.ldv + qt * DW + c] : 0.0f;
        dv[c] = 0.0f;
    }
    int h_first = 0, nh = 0, t_first = 0, nt = 0;
    if (it.ha < it.hb) {
        h_first = it.ha / BM;
        nh = cdiv(it.hb, BM) - h_first;
    }
    if (it.ta < it.tb) {
        t_first = (it.ta - sd.U) / BM;
        nt = cdiv(it.tb - sd.U, BM) - t_first;
    }
    for (int s = 0; s < nh + nt; ++s) {
        int m0, m1;
        if (s < nh) {
            m0 = (h_first + s) * BM;
            m1 = imin(m0 + BM, sd.U);
        } else {
            m0 = sd.U + (t_first + s - nh) * BM;
            m1 = imin(m0 + BM, sd.L);
        }
        __syncthreads();
        stage_rows_f32<DQK>(sq, qg, p.ldq, m0, BM, m1);
        stage_rows_f32<DV>(sg_, gg, p.lddo, m0, BM, m1);
        __syncthreads();
        float pk[DQ], pv[DW];
#pragma unroll
        for (int c = 0; c < DQ; ++c) pk[c] = 0.0f;
#pragma unroll
        for (int c = 0; c < DW; ++c) pv[c] = 0.0f;
        for (int ii = 0; ii < BM; ++ii) {
            float sv = 0.0f, g = 0.0f;
#pragma unroll
            for (int c = 0; c < DQ; ++c) sv += sq[ii * DQK + qt * DQ + c] * kr[c];
#pragma unroll
            for (int c = 0; c < DW; ++c) g += sg_[ii * DV + qt * DW + c] * vr[c];
            sv = quad_sum(sv);
            g = quad_sum(g);
            const int i = m0 + ii;
            const bool vis = jok && i < m1 && visible(i, j, sd.U, p.k1, p.k2e);
            const float tt = p.alpha * sv;
            const float a = vis ? sv / (1.0f + expf(-tt)) : 0.0f;  // SiLU(alpha s) / alpha
            const float ds = vis ? g * dsilu_f32(tt) : 0.0f;
#pragma unroll
            for (int c = 0; c < DW; ++c) pv[c] += a * sg_[ii * DV + qt * DW + c];
#pragma unroll
            for (int c = 0; c < DQ; ++c) pk[c] += ds * sq[ii * DQK + qt * DQ + c];
        }
#pragma unroll
        for (int c = 0; c < DQ; ++c) dk[c] += pk[c];
#pragma unroll
        for (int c = 0; c < DW; ++c) dv[c] += pv[c];
    }
    if (it.nchunk == 1) {
        if (jok) {
            float *ok = reinterpret_cast<float *>(p.dk) + (sd.base + j) * p.lddk + h * DQK + qt * DQ;
            float *ov = reinterpret_cast<float *>(p.dv) + (sd.base + j) * p.lddv + h * DV + qt * DW;
#pragma unroll
            for (int c = 0; c < DQ; ++c) ok[c] = dk[c] * p.out_scale;
#pragma unroll
            for (int c = 0; c < DW; ++c) ov[c] = dv[c] * p.out_scale;
        }
    } else {
        const int slot = p.s.part_base[b] + it.tile * nch + it.chunk;
        float *part = p.partials + ((int64_t)slot * p.H + h) * BN * W + kl * W;
#pragma unroll
        for (int c = 0; c < DQ; ++c) part[qt * DQ + c] = dk[c];
#pragma unroll
        for (int c = 0; c < DW; ++c) part[DQK + qt * DW + c] = dv[c];
    }
}

// fp32 reduce of split prefix key tiles, in chunk order; dK and dV partials
// both take the alpha/N scale.
template <int DQK, int DV>
__global__ __launch_bounds__(256) void sla_bwd_reduce_f32_kernel(AttnParams p)
{
    constexpr int BN = BWD_BN, W = DQK + DV;
    const int nrec = p.s.red_base[p.B];
    const int item = blockIdx.x;
    if (item >= nrec * p.H) return;
    const int h = item / nrec, rec = item - h * nrec;
    const int b = find_seq(p.s.red_base, p.B, rec);
    const SeqDims sd = seq_dims(p.offsets, p.num_targets, b);
    const int tile = rec - p.s.red_base[b];
    const int nch = p.s.nch[b];
    const int slot0 = p.s.part_base[b] + tile * nch;
    const int c0 = tile * BN, c1 = imin(c0 + BN, sd.L);
    float *dkg = reinterpret_cast<float *>(p.dk) + sd.base * p.lddk + h * DQK;
    float *dvg = reinterpret_cast<float *>(p.dv) + sd.base * p.lddv + h * DV;
    for (int e = threadIdx.x; e < BN * W; e += blockDim.x) {
        const int jl = e / W, col = e % W;
        if (c0 + jl >= c1) continue;
        float acc = 0.0f;
        for (int c = 0; c < nch; ++c) acc += p.partials[((int64_t)(slot0 + c) * p.H + h) * BN * W + e];
        if (col < DQK) dkg[(int64_t)(c0 + jl) * p.lddk + col] = acc * p.out_scale;
        else dvg[(int64_t)(c0 + jl) * p.lddv + (col - DQK)] = acc * p.out_scale;
    }
}

hipError_t launch_fwd_f32(const AttnParams &p, hipStream_t st)
{
    return with_head_dims(p, [&](auto QK, auto V) {
        hipLaunchKernelGGL((sla_fwd_f32_kernel<decltype(QK)::value, decltype(V)::value>),
                           dim3(p.grid_fwd), dim3(FWD_BM * F32_TPR), 0, st, p);
        return hipGetLastError();
    });
}

hipError_t launch_bwd_dkdv_f32(const AttnParams &p, hipStream_t st)
{
    return with_head_dims(p, [&](auto QK, auto V) {
        constexpr int DQK = decltype(QK)::value, DV = decltype(V)::value;
        hipLaunchKernelGGL((sla_bwd_dkdv_f32_kernel<DQK, DV>), dim3(p.grid_bwd),
                           dim3(BWD_BN * F32_TPR), 0, st, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || p.grid_red == 0) return e;
        hipLaunchKernelGGL((sla_bwd_reduce_f32_kernel<DQK, DV>), dim3(p.grid_red), dim3(256), 0,
                           st, p);
        return hipGetLastError();
    });
}

hipError_t launch_bwd_dq_f32(const AttnParams &p, hipStream_t st)
{
    return with_head_dims(p, [&](auto QK, auto V) {
        hipLaunchKernelGGL((sla_bwd_dq_f32_kernel<decltype(QK)::value, decltype(V)::value>),
                           dim3(p.grid_fwd), dim3(FWD_BM * F32_TPR), 0, st, p);
        return hipGetLastError();
    });
}

}  // namespace sla
