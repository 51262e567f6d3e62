// sla_noalloc.hip -- sla_bwd_noalloc: the SLA backward with its workspace
// (tile schedule and fp32 prefix partials) in a static device array instead of
// a caller buffer, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable: each device the library runs
// on holds its own copy, at its own address, from module load until the
// process ends.  In host code its name is only a host-side stand-in, so the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept; only that address is ever passed to kernels.
// Nothing in the array has to start at zero: the schedule kernel writes every
// schedule entry and the dK/dV kernel writes every partial slot it uses before
// the reduce kernel reads it, in the same call on the same stream.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sla.h"
#include "sla_kernels.h"

namespace {

static_assert(SLA_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");

static __device__ __align__(256) unsigned char scratch[SLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device, once known

// Device address of this device's copy of `scratch` (looked up on the first
// call on each device).
sla_status_t scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return (sla_status_t)sla::set_last_error(SLA_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices)
        return (sla_status_t)sla::set_last_error(SLA_ERR_DEVICE, "device index out of range");
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return (sla_status_t)sla::set_last_error(
                SLA_ERR_HIP, "hipGetSymbolAddress of the static workspace failed");
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return SLA_OK;
}

}  // namespace

extern "C" sla_status_t sla_bwd_noalloc(const sla_problem_t *p, const void *q, int64_t ldq,
                                        const void *k, int64_t ldk, const void *v, int64_t ldv,
                                        const void *dout, int64_t lddo, void *dq, int64_t lddq,
                                        void *dk, int64_t lddk, void *dv, int64_t lddv,
                                        void *stream)
{
    const size_t need = sla_workspace_size(p, SLA_OP_BWD_RECOMPUTE);
    if (need == 0)  // an invalid problem: sla_bwd reports which check failed
        return sla_bwd(p, q, ldq, k, ldk, v, ldv, dout, lddo, dq, lddq, dk, lddk, dv, lddv,
                       nullptr, 0, stream);
    if (need > SLA_NOALLOC_SCRATCH_BYTES) {
        char msg[160];
        snprintf(msg, sizeof(msg),
                 "the problem needs %zu bytes of workspace; sla_bwd_noalloc holds at most %zu",
                 need, (size_t)SLA_NOALLOC_SCRATCH_BYTES);
        return (sla_status_t)sla::set_last_error(SLA_ERR_WORKSPACE, msg);
    }
    if (p->batch == 0 || p->total_tokens == 0)  // nothing is read or written
        return sla_bwd(p, q, ldq, k, ldk, v, ldv, dout, lddo, dq, lddq, dk, lddk, dv, lddv,
                       nullptr, 0, stream);
    void *ws = nullptr;
    const sla_status_t st = scratch_address(&ws);
    if (st != SLA_OK) return st;
    return sla_bwd(p, q, ldq, k, ldk, v, ldv, dout, lddo, dq, lddq, dk, lddk, dv, lddv, ws,
                   SLA_NOALLOC_SCRATCH_BYTES, stream);
}
