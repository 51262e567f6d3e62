// sla_api.cpp -- host side of the C ABI declared in include/sla.h: argument
// validation (before any HIP call), workspace sizing from host-known sizes,
// and kernel launches on the caller's stream.  No host synchronisation, no
// device allocation.
#include "sla.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

#include "sla_kernels.h"

using namespace sla;

namespace {

thread_local std::string g_last_error;

sla_status_t fail(sla_status_t s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

sla_status_t hip_fail(hipError_t e, const char *what)
{
    return fail(SLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// gfx950 check, cached per device
sla_status_t check_device()
{
    static std::mutex mu;
    static std::unordered_map<int, bool> cache;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = cache.find(dev);
        if (it != cache.end())
            return it->second ? SLA_OK : fail(SLA_ERR_DEVICE, "device %d is not gfx950", dev);
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    {
        std::lock_guard<std::mutex> lk(mu);
        cache[dev] = ok;
    }
    return ok ? SLA_OK : fail(SLA_ERR_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
}

int k2_eff(const sla_problem_t *p) { return p->k2 > p->contextual_len ? p->k2 : p->contextual_len; }

sla_status_t validate_problem(const sla_problem_t *p)
{
    if (!p) return fail(SLA_ERR_NULL, "problem is NULL");
    if (p->dtype != SLA_F32 && p->dtype != SLA_BF16)
        return fail(SLA_ERR_UNSUPPORTED, "dtype %d unsupported", p->dtype);
    if (p->batch < 0 || p->total_tokens < 0)
        return fail(SLA_ERR_INVALID, "negative batch (%d) or total_tokens (%lld)", p->batch,
                    (long long)p->total_tokens);
    if (p->total_tokens >= (int64_t)1 << 30)
        return fail(SLA_ERR_UNSUPPORTED, "total_tokens %lld too large", (long long)p->total_tokens);
    if (p->batch > 0 && !p->offsets) return fail(SLA_ERR_NULL, "offsets is NULL");
    if (p->num_heads < 1) return fail(SLA_ERR_INVALID, "num_heads must be >= 1");
    if (!attn_dims_supported(p->d_qk, p->d_v))
        return fail(SLA_ERR_UNSUPPORTED, "head widths d_qk = %d, d_v = %d not in {32, 64, 128}",
                    p->d_qk, p->d_v);
    if (p->k1 < 0 || p->k2 < 0 || p->contextual_len < 0)
        return fail(SLA_ERR_INVALID, "k1, k2 and contextual_len must be >= 0");
    if (p->max_seq_len < 1) return fail(SLA_ERR_INVALID, "max_seq_len must be >= 1");
    if (!std::isfinite(p->alpha)) return fail(SLA_ERR_INVALID, "alpha must be finite");
    if (p->out_f32 != 0 && p->out_f32 != 1) return fail(SLA_ERR_INVALID, "out_f32 must be 0 or 1");
    return SLA_OK;
}

// elem_f32: the tensor holds fp32 elements (the f32 path, or an output of
// the bf16 path with out_f32 set), else bf16
sla_status_t validate_tensor(const char *name, const void *ptr, int64_t ld, const sla_problem_t *p,
                             int d, bool output = false)
{
    if (!ptr) return fail(SLA_ERR_NULL, "%s is NULL", name);
    if (ld < (int64_t)p->num_heads * d)
        return fail(SLA_ERR_INVALID, "%s: token stride %lld < H*d = %d", name, (long long)ld,
                    p->num_heads * d);
    const bool f32 = p->dtype == SLA_F32 || (output && p->out_f32);
    const int elems16 = f32 ? 4 : 8;
    if (ld % elems16 != 0)
        return fail(SLA_ERR_UNSUPPORTED, "%s: token stride %lld is not a multiple of 16 bytes",
                    name, (long long)ld);
    if (!aligned16(ptr)) return fail(SLA_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
    return SLA_OK;
}

// Optional validation mode (environment SLA_VALIDATE, read at every call):
// check the device-resident layout facts, synchronising the stream, before
// any other kernel of the call.  scratch: 8 bytes of device memory the call
// owns and overwrites later anyway.
bool validate_mode()
{
    const char *e = std::getenv("SLA_VALIDATE");
    return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

sla_status_t validate_layout(int B, int64_t T, const int64_t *offsets, const int32_t *num_targets,
                             int ctx, void *scratch, hipStream_t s)
{
    if (!validate_mode() || B == 0) return SLA_OK;
    if (!scratch) return fail(SLA_ERR_NULL, "validation needs the workspace");
    int32_t *res = static_cast<int32_t *>(scratch);
    hipError_t e = launch_validate(offsets, num_targets, B, T, ctx, res, s);
    if (e != hipSuccess) return hip_fail(e, "validation kernel");
    int32_t host[2] = {0, -1};
    e = hipMemcpyAsync(host, res, sizeof(host), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "validation copy");
    switch (host[0]) {
    case 0: return SLA_OK;
    case 1: return fail(SLA_ERR_INVALID, "offsets[0] != 0");
    case 2: return fail(SLA_ERR_INVALID, "offsets decrease at sequence %d", host[1]);
    case 3: return fail(SLA_ERR_INVALID, "offsets[B] != total_tokens (%lld)", (long long)T);
    case 4: return fail(SLA_ERR_INVALID, "num_targets[%d] outside [0, L_b]", host[1]);
    case 5: return fail(SLA_ERR_INVALID, "contextual_len + num_targets[%d] > L_b", host[1]);
    default: return fail(SLA_ERR_INVALID, "layout check failed (code %d)", host[0]);
    }
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

WsLayout layout(const sla_problem_t *p, int op)
{
    WsLayout w{};
    const int64_t T = p->total_tokens, B = p->batch;
    const int K2e = k2_eff(p);
    w.fwd_items = T / FWD_BM + 2 * B + 1;
    int64_t np_max = (K2e + BWD_BN - 1) / BWD_BN;
    if (np_max > BWD_MAX_SPLIT_TILES) np_max = BWD_MAX_SPLIT_TILES;
    int64_t chunk_sum = T / ((int64_t)BWD_BM * BWD_CHUNK_TILES) + 2 * B + 1;
    if (chunk_sum > B * BWD_MAX_CHUNKS) chunk_sum = B * BWD_MAX_CHUNKS;
    w.part_slots = np_max * chunk_sum;
    w.bwd_items = T / BWD_BN + B + 1 + w.part_slots;
    w.red_items = np_max * B;
    w.sched_off = 0;
    const size_t sched_bytes = sizeof(int32_t) * (4 * (size_t)(B + 1) + (size_t)B);
    w.part_off = round_up(sched_bytes, 256);
    size_t part_bytes = 0;
    if (op == SLA_OP_BWD || op == SLA_OP_BWD_RECOMPUTE)
        part_bytes = (size_t)w.part_slots * p->num_heads * BWD_BN * (size_t)(p->d_qk + p->d_v) *
                     sizeof(float);
    w.total = w.part_off + round_up(part_bytes, 256);
    if (op != SLA_OP_BWD || p->dtype != SLA_BF16 || p->d_qk < 64) return w;
    // Stored dS: an upper bound of the 64-row steps over all key tiles, per
    // head, from host-known sizes only.  Key tiles: sum ceil(L/128) <= T/128 +
    // B; a window tile is seen by at most ceil((127 + K1) / 64) steps, a
    // global-prefix tile by every history step (sum ceil(L/64) <= T/64 + B);
    // with targets, a tile in the window of the first target slot or the
    // prefix is seen by every target step, any other by at most 3 steps of
    // its own targets.
    const int64_t tiles = T / BWD_BN + B, rsteps = T / BWD_BM + B;
    int64_t win = ((int64_t)p->k1 + BWD_BN - 1 + BWD_BM - 1) / BWD_BM;
    if (win > rsteps) win = rsteps;
    const int64_t npre = (K2e + BWD_BN - 1) / BWD_BN;
    int64_t blocks = tiles * win + npre * rsteps;
    if (p->num_targets) {
        int64_t kt = ((int64_t)p->k1 + BWD_BN - 1) / BWD_BN + 1;
        if (kt > tiles) kt = tiles;
        blocks += (npre + kt) * rsteps + 3 * tiles;
    }
    // only where dS costs at most 16 times the bytes of Q, K, V and dO
    const double in_bytes = 4.0 * (double)T * p->num_heads * (p->d_qk + p->d_v);
    const double ds_bytes = (double)blocks * p->num_heads * DS_BLOCK_BYTES;
    if (T == 0 || ds_bytes > 16.0 * in_bytes || blocks > INT32_MAX / 2) return w;
    w.ds_blocks = blocks;
    w.ktile_off = w.total;
    w.dsb_off = w.ktile_off + round_up(sizeof(int32_t) * (size_t)(B + 1), 256);
    w.ds_off = w.dsb_off + round_up(sizeof(int32_t) * (size_t)(tiles + 1), 256);
    w.total = w.ds_off + (size_t)blocks * p->num_heads * DS_BLOCK_BYTES;
    return w;
}

sla_status_t make_params(const sla_problem_t *p, int op, void *ws, size_t ws_bytes, AttnParams &a)
{
    // the backward stores dS when the workspace holds it, else dQ recomputes
    WsLayout w = layout(p, op);
    if (op == SLA_OP_BWD && ws_bytes < w.total) w = layout(p, SLA_OP_BWD_RECOMPUTE);
    if (!ws) return fail(SLA_ERR_WORKSPACE, "workspace is NULL");
    if (ws_bytes < w.total)
        return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", ws_bytes, w.total);
    if (!aligned16(ws)) return fail(SLA_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
    const int64_t H = p->num_heads;
    if (w.fwd_items * H > INT32_MAX || w.bwd_items * H > INT32_MAX)
        return fail(SLA_ERR_UNSUPPORTED, "problem too large for one launch");
    std::memset(&a, 0, sizeof(a));
    a.offsets = p->offsets;
    a.num_targets = p->num_targets;
    a.B = p->batch;
    a.H = p->num_heads;
    a.d = p->d_qk;
    a.d_v = p->d_v;
    a.k1 = p->k1;
    a.k2e = k2_eff(p);
    a.alpha = p->alpha;
    a.inv_n = 1.0f / (float)p->max_seq_len;
    a.out_scale = p->alpha / (float)p->max_seq_len;
    a.neg_alpha_log2e = -p->alpha * 1.4426950408889634f;
    a.out_f32 = p->dtype == SLA_BF16 && p->out_f32;
    int32_t *s = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + w.sched_off);
    const int B1 = p->batch + 1;
    a.s.fwd_base = s;
    a.s.bwd_base = s + B1;
    a.s.red_base = s + 2 * B1;
    a.s.part_base = s + 3 * B1;
    a.s.nch = s + 4 * B1;
    a.T = p->total_tokens;
    a.partials = reinterpret_cast<float *>(static_cast<char *>(ws) + w.part_off);
    if (w.ds_blocks > 0) {
        char *base = static_cast<char *>(ws);
        a.s.ktile_base = reinterpret_cast<int32_t *>(base + w.ktile_off);
        a.s.ds_base = reinterpret_cast<int32_t *>(base + w.dsb_off);
        a.ds = reinterpret_cast<uint8_t *>(base + w.ds_off);
        a.ds_head_blocks = w.ds_blocks;
    }
    a.grid_fwd = (int)(w.fwd_items * H);
    a.grid_bwd = (int)(w.bwd_items * H);
    a.grid_red = (int)(w.red_items * H);
    return SLA_OK;
}

// STU layer backward workspace: recomputed activations, their gradients, a
// transposed weight, fp32 partial sums, and the attention workspace last.
struct StuBwdLayout {
    size_t n, z, uvqk, A, y, dy, dA, dz, dn, wt, part, vec, mid, zero, attn, total;
};

StuBwdLayout stu_bwd_layout(const stu_layer_desc_t *d)
{
    const sla_problem_t *p = &d->attn;
    const size_t T = (size_t)p->total_tokens, D = (size_t)d->hidden;
    const size_t NU = (size_t)p->num_heads * p->d_v;
    const size_t NW = 2 * NU + 2 * (size_t)p->num_heads * p->d_qk;
    StuBwdLayout L{};
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t o = at;
        at += round_up(bytes, 256);
        return o;
    };
    L.n = take(T * D * 2);
    L.z = take(T * NW * 2);
    L.uvqk = take(T * NW * 2);
    L.A = take(T * NU * 2);
    L.y = take(T * NU * 2);
    L.dy = take(T * NU * 2);
    L.dA = take(T * NU * 2);
    L.dz = take(T * NW * 2);
    L.dn = take(T * D * 2);
    L.wt = take(NW * D * 2);
    size_t part = (size_t)tn_plan((int64_t)T, (int)D, (int)NU).splits * D * NU;
    const size_t pu = (size_t)tn_plan((int64_t)T, (int)NW, (int)D).splits * NW * D;
    if (pu > part) part = pu;
    const size_t cs = (size_t)colsum_blocks((int64_t)T) * (NW > D ? NW : D);
    if (cs > part) part = cs;
    const size_t ln = 2 * (size_t)ln_bwd_blocks((int64_t)T) * (NU > D ? NU : D);
    if (ln > part) part = ln;
    L.part = take(part * 4);
    L.vec = take((NW > D ? NW : D) * 4);
    L.mid = take((size_t)SUM_MID_FLOATS * 4);
    L.zero = take(1024);  // a zero token row for the weight-gradient products
    L.attn = at;
    L.total = at + layout(p, SLA_OP_BWD).total;
    return L;
}

}  // namespace

int sla::set_last_error(int status, const char *msg)
{
    return fail(static_cast<sla_status_t>(status), "%s", msg);
}

namespace {
sla_status_t fwd_impl(const sla_problem_t *p, const void *q, int64_t ldq, const void *k,
                      int64_t ldk, const void *v, int64_t ldv, void *o, int64_t ldo,
                      void *workspace, size_t ws_bytes, void *stream, bool build_schedule);
}

extern "C" {

size_t sla_probe_scratch_size(void)
{
    int dev = -1, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 0;
    // the sink (one float per thread of 4 workgroups of 256 per CU), then the
    // two clock counters; the issue-rate probe's sink (one workgroup of 512
    // per CU) fits in the same
    return round_up(sizeof(float) * (size_t)4 * cus * 256, 256) + 2 * sizeof(unsigned long long);
}

sla_status_t sla_probe_mfma_peak(int32_t iters, void *scratch, size_t scratch_bytes,
                                 double *tflops, double *sclk_ghz, void *stream)
{
    if (!tflops || !sclk_ghz || !scratch) return fail(SLA_ERR_NULL, "tflops, sclk_ghz or scratch is NULL");
    if (iters < 1 || iters > (1 << 20)) return fail(SLA_ERR_INVALID, "iters %d outside [1, 2^20]", iters);
    sla_status_t st = check_device();
    if (st != SLA_OK) return st;
    int dev = -1, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "device attributes");
    const int blocks = 4 * cus;
    const size_t sink_bytes = round_up(sizeof(float) * (size_t)blocks * 256, 256);
    if (scratch_bytes < sink_bytes + 2 * sizeof(unsigned long long))
        return fail(SLA_ERR_WORKSPACE, "probe scratch of %zu bytes < %zu required", scratch_bytes,
                    sink_bytes + 2 * sizeof(unsigned long long));
    if (!aligned16(scratch)) return fail(SLA_ERR_UNSUPPORTED, "probe scratch is not 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *sink = static_cast<float *>(scratch);
    unsigned long long *clk =
        reinterpret_cast<unsigned long long *>(static_cast<char *>(scratch) + sink_bytes);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    unsigned long long hclk[2] = {0, 0};
    float ms = 0.0f;
    e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) e = launch_mfma_peak(blocks, iters, sink, clk, s);  // warm-up
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    if (e == hipSuccess) e = launch_mfma_peak(blocks, iters, sink, clk, s);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess) e = hipMemcpy(hclk, clk, sizeof(hclk), hipMemcpyDeviceToHost);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (e != hipSuccess) return hip_fail(e, "MFMA probe");
    if (!(ms > 0.0f)) return fail(SLA_ERR_DEVICE, "MFMA probe: no elapsed time");
    *tflops = mfma_peak_flops(blocks, iters) / ((double)ms * 1e-3) / 1e12;
    // the constant clock counts at 100 MHz: GHz = cycles / (ticks * 10)
    *sclk_ghz = hclk[1] > 0 ? (double)hclk[0] / ((double)hclk[1] * 10.0) : 0.0;
    return SLA_OK;
}

sla_status_t sla_probe_issue_rates(int32_t iters, void *scratch, size_t scratch_bytes, double *ms,
                                   int32_t n_ms, void *stream)
{
    if (!ms || !scratch) return fail(SLA_ERR_NULL, "ms or scratch is NULL");
    if (n_ms < ISSUE_MODES) return fail(SLA_ERR_INVALID, "ms holds %d entries < %d modes", n_ms, (int)ISSUE_MODES);
    if (iters < 1 || iters > (1 << 20)) return fail(SLA_ERR_INVALID, "iters %d outside [1, 2^20]", iters);
    sla_status_t st = check_device();
    if (st != SLA_OK) return st;
    int dev = -1, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "device attributes");
    const int blocks = cus;  // one 512-thread workgroup per CU
    const size_t sink_bytes = sizeof(float) * (size_t)blocks * 512;
    if (scratch_bytes < sink_bytes)
        return fail(SLA_ERR_WORKSPACE, "probe scratch of %zu bytes < %zu required", scratch_bytes, sink_bytes);
    if (!aligned16(scratch)) return fail(SLA_ERR_UNSUPPORTED, "probe scratch is not 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *sink = static_cast<float *>(scratch);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    for (int m = 0; m < ISSUE_MODES && e == hipSuccess; ++m) {
        float t = 0.0f;
        e = launch_issue_probe(m, blocks, iters, sink, s);  // warm-up
        if (e == hipSuccess) e = hipEventRecord(e0, s);
        if (e == hipSuccess) e = launch_issue_probe(m, blocks, iters, sink, s);
        if (e == hipSuccess) e = hipEventRecord(e1, s);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        if (e == hipSuccess) e = hipEventElapsedTime(&t, e0, e1);
        ms[m] = (double)t;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (e != hipSuccess) return hip_fail(e, "issue-rate probe");
    return SLA_OK;
}

const char *sla_status_string(sla_status_t s)
{
    switch (s) {
    case SLA_OK: return "SLA_OK";
    case SLA_ERR_NULL: return "SLA_ERR_NULL";
    case SLA_ERR_INVALID: return "SLA_ERR_INVALID";
    case SLA_ERR_UNSUPPORTED: return "SLA_ERR_UNSUPPORTED";
    case SLA_ERR_WORKSPACE: return "SLA_ERR_WORKSPACE";
    case SLA_ERR_HIP: return "SLA_ERR_HIP";
    case SLA_ERR_DEVICE: return "SLA_ERR_DEVICE";
    }
    return "SLA_ERR_UNKNOWN";
}

const char *sla_last_error(void) { return g_last_error.c_str(); }

size_t sla_workspace_size(const sla_problem_t *p, int op)
{
    if (validate_problem(p) != SLA_OK) return 0;
    if (op != SLA_OP_FWD && op != SLA_OP_BWD && op != SLA_OP_BWD_RECOMPUTE) return 0;
    return layout(p, op).total;
}

int64_t sla_schedule_capacity(const sla_problem_t *p, int op)
{
    if (validate_problem(p) != SLA_OK) return -1;
    if (op != SLA_OP_FWD && op != SLA_OP_BWD) return -1;
    const WsLayout w = layout(p, SLA_OP_FWD);
    return op == SLA_OP_FWD ? w.fwd_items : w.bwd_items;
}

int32_t sla_schedule_tile(int op, int which)
{
    if (op == SLA_OP_FWD) return which == 0 ? FWD_BM : FWD_BN;
    if (op == SLA_OP_BWD) return which == 0 ? BWD_BN : BWD_BM;
    return -1;
}

sla_status_t sla_schedule(const sla_problem_t *p, int op, int32_t *records, int64_t capacity,
                          int32_t *count, void *workspace, size_t ws_bytes, void *stream)
{
    sla_status_t st = validate_problem(p);
    if (st != SLA_OK) return st;
    if (op != SLA_OP_FWD && op != SLA_OP_BWD) return fail(SLA_ERR_INVALID, "bad op %d", op);
    if (!records || !count) return fail(SLA_ERR_NULL, "records or count is NULL");
    if (capacity < sla_schedule_capacity(p, op))
        return fail(SLA_ERR_INVALID, "capacity below sla_schedule_capacity");
    AttnParams a;
    if ((st = make_params(p, SLA_OP_FWD, workspace, ws_bytes, a)) != SLA_OK) return st;
    if ((st = check_device()) != SLA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = validate_layout(p->batch, p->total_tokens, p->offsets, p->num_targets, -1, workspace,
                              s)) != SLA_OK)
        return st;
    hipError_t e = launch_sched(a, s);
    if (e != hipSuccess) return hip_fail(e, "schedule kernel");
    e = launch_sched_dump(a, op, records, capacity, count, s);
    if (e != hipSuccess) return hip_fail(e, "schedule dump kernel");
    return SLA_OK;
}

int64_t sla_schedule_host(const sla_problem_t *p, int op, const int64_t *offsets_host,
                          const int32_t *num_targets_host, int32_t *records, int64_t capacity)
{
    if (!p) return fail(SLA_ERR_NULL, "problem is NULL"), -1;
    sla_problem_t hp = *p;  // the device pointers are not used here
    hp.offsets = offsets_host;
    hp.num_targets = num_targets_host;
    p = &hp;
    if (validate_problem(p) != SLA_OK) return -1;
    if (op != SLA_OP_FWD && op != SLA_OP_BWD) {
        fail(SLA_ERR_INVALID, "bad op %d", op);
        return -1;
    }
    if (p->batch > 0 && !offsets_host) {
        fail(SLA_ERR_NULL, "offsets_host is NULL");
        return -1;
    }
    const int K2e = k2_eff(p);
    int64_t n = 0;
    for (int b = 0; b < p->batch; ++b) {
        const int64_t L64 = offsets_host[b + 1] - offsets_host[b];
        const int64_t nt = num_targets_host ? num_targets_host[b] : 0;
        if (L64 < 0 || L64 >= ((int64_t)1 << 30) || nt < 0 || nt > L64) {
            fail(SLA_ERR_INVALID, "sequence %d: bad length or target count", b);
            return -1;
        }
        const int L = (int)L64, U = (int)(L64 - nt);
        const int items = seq_items(op, L, U, K2e);
        for (int li = 0; li < items; ++li, ++n) {
            if (records && n < capacity)
                fill_record(op, b, L, U, p->k1, K2e, li, records + n * SLA_SCHED_RECORD_INTS);
        }
    }
    return n;
}

int64_t sla_ds_blocks_host(const sla_problem_t *p, const int64_t *offsets_host,
                           const int32_t *num_targets_host, int64_t *blocks, int64_t capacity)
{
    if (!p) return fail(SLA_ERR_NULL, "problem is NULL"), -1;
    sla_problem_t hp = *p;  // the device pointers are not used here
    hp.offsets = offsets_host;
    hp.num_targets = num_targets_host;
    p = &hp;
    if (validate_problem(p) != SLA_OK) return -1;
    if (p->batch > 0 && !offsets_host) {
        fail(SLA_ERR_NULL, "offsets_host is NULL");
        return -1;
    }
    const int K2e = k2_eff(p);
    int64_t n = 0;
    for (int b = 0; b < p->batch; ++b) {
        const int64_t L64 = offsets_host[b + 1] - offsets_host[b];
        const int64_t nt = num_targets_host ? num_targets_host[b] : 0;
        if (L64 < 0 || L64 >= ((int64_t)1 << 30) || nt < 0 || nt > L64) {
            fail(SLA_ERR_INVALID, "sequence %d: bad length or target count", b);
            return -1;
        }
        const int L = (int)L64, U = (int)(L64 - nt);
        for (int c0 = 0; c0 < L; c0 += BWD_BN) {
            const TileSteps ts = tile_steps(L, U, p->k1, K2e, c0, std::min(c0 + BWD_BN, L), BWD_BM);
            for (int s = 0; s < ts.nh + ts.nt; ++s, ++n) {
                if (!blocks || n >= capacity) continue;
                const int64_t m0 = s < ts.nh ? (int64_t)(ts.h_first + s) * BWD_BM
                                             : U + (int64_t)(ts.t_first + s - ts.nh) * BWD_BM;
                blocks[3 * n] = b;
                blocks[3 * n + 1] = m0;
                blocks[3 * n + 2] = c0;
            }
        }
    }
    return n;
}

sla_status_t sla_fwd(const sla_problem_t *p, const void *q, int64_t ldq, const void *k, int64_t ldk,
                     const void *v, int64_t ldv, void *o, int64_t ldo, void *workspace,
                     size_t ws_bytes, void *stream)
{
    return fwd_impl(p, q, ldq, k, ldk, v, ldv, o, ldo, workspace, ws_bytes, stream, true);
}

}  // extern "C"

namespace {
// sla_fwd; build_schedule false: the workspace already holds this layout's
// schedule (a stack's later layers)
sla_status_t fwd_impl(const sla_problem_t *p, const void *q, int64_t ldq, const void *k,
                      int64_t ldk, const void *v, int64_t ldv, void *o, int64_t ldo,
                      void *workspace, size_t ws_bytes, void *stream, bool build_schedule)
{
    sla_status_t st = validate_problem(p);
    if (st != SLA_OK) return st;
    if (p->batch == 0 || p->total_tokens == 0) return SLA_OK;  // nothing is read or written
    if ((st = validate_tensor("q", q, ldq, p, p->d_qk)) != SLA_OK) return st;
    if ((st = validate_tensor("k", k, ldk, p, p->d_qk)) != SLA_OK) return st;
    if ((st = validate_tensor("v", v, ldv, p, p->d_v)) != SLA_OK) return st;
    if ((st = validate_tensor("o", o, ldo, p, p->d_v, true)) != SLA_OK) return st;
    AttnParams a;
    if ((st = make_params(p, SLA_OP_FWD, workspace, ws_bytes, a)) != SLA_OK) return st;
    if ((st = check_device()) != SLA_OK) return st;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.ldq = ldq; a.ldk = ldk; a.ldv = ldv; a.ldo = ldo;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = validate_layout(p->batch, p->total_tokens, p->offsets, p->num_targets, -1, workspace,
                              s)) != SLA_OK)
        return st;
    hipError_t e = hipSuccess;
    if (build_schedule) {
        e = launch_sched(a, s);
        if (e != hipSuccess) return hip_fail(e, "schedule kernel");
    }
    e = p->dtype == SLA_BF16 ? launch_fwd_bf16(a, s) : launch_fwd_f32(a, s);
    if (e != hipSuccess) return hip_fail(e, "forward kernel");
    return SLA_OK;
}
}  // namespace

extern "C" {

size_t sla_fwd_candidates_workspace_size(const sla_problem_t *p, int64_t total_candidates)
{
    if (validate_problem(p) != SLA_OK || total_candidates < 0 ||
        total_candidates >= (int64_t)1 << 30)
        return 0;
    sla_problem_t pw = *p;
    if (total_candidates > pw.total_tokens) pw.total_tokens = total_candidates;
    return layout(&pw, SLA_OP_FWD).total;
}

sla_status_t sla_fwd_candidates(const sla_problem_t *p, const int64_t *cand_offsets,
                                int64_t total_candidates, const void *k_hist, int64_t ldk,
                                const void *v_hist, int64_t ldv, const void *q_c, int64_t ldq,
                                const void *k_c, int64_t ldkc, const void *v_c, int64_t ldvc,
                                void *o_c, int64_t ldo, void *workspace, size_t ws_bytes,
                                void *stream)
{
    sla_status_t st = validate_problem(p);
    if (st != SLA_OK) return st;
    if (p->dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "candidate scoring is bf16 only");
    if (p->num_targets)
        return fail(SLA_ERR_INVALID, "the history problem has no targets (num_targets must be NULL)");
    if (total_candidates < 0) return fail(SLA_ERR_INVALID, "negative total_candidates");
    if (total_candidates >= (int64_t)1 << 30)
        return fail(SLA_ERR_UNSUPPORTED, "total_candidates too large");
    if (p->batch > 0 && !cand_offsets) return fail(SLA_ERR_NULL, "cand_offsets is NULL");
    if (p->batch == 0 || total_candidates == 0) return SLA_OK;  // nothing is read or written
    sla_problem_t pc = *p;
    pc.total_tokens = total_candidates;
    if (p->total_tokens > 0) {
        if ((st = validate_tensor("k_hist", k_hist, ldk, p, p->d_qk)) != SLA_OK) return st;
        if ((st = validate_tensor("v_hist", v_hist, ldv, p, p->d_v)) != SLA_OK) return st;
    }
    if ((st = validate_tensor("q_c", q_c, ldq, &pc, p->d_qk)) != SLA_OK) return st;
    if ((st = validate_tensor("k_c", k_c, ldkc, &pc, p->d_qk)) != SLA_OK) return st;
    if ((st = validate_tensor("v_c", v_c, ldvc, &pc, p->d_v)) != SLA_OK) return st;
    if ((st = validate_tensor("o_c", o_c, ldo, &pc, p->d_v, true)) != SLA_OK) return st;
    sla_problem_t pw = *p;  // workspace and grid bound: the larger row count
    if (total_candidates > pw.total_tokens) pw.total_tokens = total_candidates;
    AttnParams a;
    if ((st = make_params(&pw, SLA_OP_FWD, workspace, ws_bytes, a)) != SLA_OK) return st;
    if ((st = check_device()) != SLA_OK) return st;
    a.q = q_c; a.k = k_hist; a.v = v_hist; a.o = o_c; a.kc = k_c; a.vc = v_c;
    a.ldq = ldq; a.ldk = ldk; a.ldv = ldv; a.ldo = ldo; a.ldkc = ldkc; a.ldvc = ldvc;
    a.cand_offsets = cand_offsets;
    a.num_targets = nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = validate_layout(p->batch, p->total_tokens, p->offsets, nullptr, -1, workspace, s)) !=
        SLA_OK)
        return st;
    if ((st = validate_layout(p->batch, total_candidates, cand_offsets, nullptr, -1, workspace,
                              s)) != SLA_OK)
        return st;
    hipError_t e = launch_sched(a, s);
    if (e != hipSuccess) return hip_fail(e, "schedule kernel");
    e = launch_fwd_candidates_bf16(a, s);
    if (e != hipSuccess) return hip_fail(e, "candidate forward kernel");
    return SLA_OK;
}

sla_status_t sla_bwd_stage(const sla_problem_t *p, int stage, const void *q, int64_t ldq,
                           const void *k, int64_t ldk, const void *v, int64_t ldv,
                           const void *dout, int64_t lddo, void *dq, int64_t lddq, void *dk,
                           int64_t lddk, void *dv, int64_t lddv, void *workspace,
                           size_t ws_bytes, void *stream)
{
    sla_status_t st = validate_problem(p);
    if (st != SLA_OK) return st;
    if (stage < SLA_BWD_ALL || stage > SLA_BWD_DQ) return fail(SLA_ERR_INVALID, "bad stage %d", stage);
    if (p->batch == 0 || p->total_tokens == 0) return SLA_OK;  // nothing is read or written
    if ((st = validate_tensor("q", q, ldq, p, p->d_qk)) != SLA_OK) return st;
    if ((st = validate_tensor("k", k, ldk, p, p->d_qk)) != SLA_OK) return st;
    if ((st = validate_tensor("v", v, ldv, p, p->d_v)) != SLA_OK) return st;
    if ((st = validate_tensor("dout", dout, lddo, p, p->d_v)) != SLA_OK) return st;
    if (stage == SLA_BWD_ALL || stage == SLA_BWD_DQ)
        if ((st = validate_tensor("dq", dq, lddq, p, p->d_qk, true)) != SLA_OK) return st;
    if (stage == SLA_BWD_ALL || stage == SLA_BWD_DKDV) {
        if ((st = validate_tensor("dk", dk, lddk, p, p->d_qk, true)) != SLA_OK) return st;
        if ((st = validate_tensor("dv", dv, lddv, p, p->d_v, true)) != SLA_OK) return st;
    }
    AttnParams a;
    if ((st = make_params(p, SLA_OP_BWD, workspace, ws_bytes, a)) != SLA_OK) return st;
    if ((st = check_device()) != SLA_OK) return st;
    a.q = q; a.k = k; a.v = v; a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
    a.ldq = ldq; a.ldk = ldk; a.ldv = ldv; a.lddo = lddo; a.lddq = lddq; a.lddk = lddk;
    a.lddv = lddv;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = validate_layout(p->batch, p->total_tokens, p->offsets, p->num_targets, -1, workspace,
                              s)) != SLA_OK)
        return st;
    hipError_t e = hipSuccess;
    if (stage == SLA_BWD_ALL || stage == SLA_BWD_PREPARE) {
        e = launch_sched(a, s);
        if (e != hipSuccess) return hip_fail(e, "schedule kernel");
    }
    const bool bf = p->dtype == SLA_BF16;
    if (stage == SLA_BWD_ALL || stage == SLA_BWD_DKDV) {
        e = bf ? launch_bwd_dkdv_bf16(a, s) : launch_bwd_dkdv_f32(a, s);
        if (e != hipSuccess) return hip_fail(e, "dK/dV kernels");
    }
    if (stage == SLA_BWD_ALL || stage == SLA_BWD_DQ) {
        e = bf ? launch_bwd_dq_bf16(a, s) : launch_bwd_dq_f32(a, s);
        if (e != hipSuccess) return hip_fail(e, "dQ kernel");
    }
    return SLA_OK;
}

sla_status_t sla_bwd(const sla_problem_t *p, const void *q, int64_t ldq, const void *k, int64_t ldk,
                     const void *v, int64_t ldv, const void *dout, int64_t lddo, void *dq,
                     int64_t lddq, void *dk, int64_t lddk, void *dv, int64_t lddv, void *workspace,
                     size_t ws_bytes, void *stream)
{
    return sla_bwd_stage(p, SLA_BWD_ALL, q, ldq, k, ldk, v, ldv, dout, lddo, dq, lddq, dk, lddk, dv,
                         lddv, workspace, ws_bytes, stream);
}

int64_t sla_count_pairs_host(int32_t batch, const int64_t *offsets_host,
                             const int32_t *num_targets_host, int32_t k1, int32_t k2,
                             int32_t contextual_len)
{
    if (batch < 0 || k1 < 0 || k2 < 0 || contextual_len < 0) return -1;
    if (batch > 0 && !offsets_host) return -1;
    const int64_t K1 = k1, K2e = k2 > contextual_len ? k2 : contextual_len;
    int64_t total = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t L = offsets_host[b + 1] - offsets_host[b];
        const int64_t nt = num_targets_host ? num_targets_host[b] : 0;
        if (L < 0 || nt < 0 || nt > L) return -1;
        const int64_t U = L - nt;
        // history row i: window [i-K1+1, i] clipped at 0, plus prefix keys below it
        for (int64_t i = 0; i < U; ++i) {
            const int64_t w0 = i - K1 + 1 > 0 ? i - K1 + 1 : 0;
            const int64_t win = i + 1 - w0;
            int64_t pre = K2e < w0 ? K2e : w0;
            total += win + pre;
        }
        // each target: history keys of row U's window, the prefix below it, itself
        if (nt > 0) {
            const int64_t w0 = U - K1 + 1 > 0 ? U - K1 + 1 : 0;
            const int64_t win = U > w0 ? U - w0 : 0;
            const int64_t pre = K2e < w0 ? K2e : w0;
            total += nt * (win + (pre < U ? pre : U) + 1);
        }
    }
    return total;
}

size_t stu_layer_workspace_size(const stu_layer_desc_t *d)
{
    if (!d || validate_problem(&d->attn) != SLA_OK || d->hidden <= 0) return 0;
    const sla_problem_t *p = &d->attn;
    const size_t T = (size_t)p->total_tokens, H = (size_t)p->num_heads;
    const size_t nw = 2 * H * p->d_v + 2 * H * p->d_qk;
    size_t bytes = 0;
    bytes += round_up(T * d->hidden * 2, 256);      // n
    bytes += round_up(T * nw * 2, 256);             // uvqk
    bytes += round_up(T * H * p->d_v * 2, 256);     // A
    bytes += round_up(T * H * p->d_v * 2, 256);     // y
    bytes += layout(p, SLA_OP_FWD).total;           // attention schedule
    return bytes;
}

sla_status_t stu_layer_fwd(const stu_layer_desc_t *d, const void *x, const float *ln1_w,
                           const float *ln1_b, const void *w_uvqk, const float *b_uvqk,
                           const float *ln2_w, const float *ln2_b, const void *w_out,
                           const float *b_out, void *out, void *uvqk_out, void *attn_out,
                           void *workspace, size_t ws_bytes, void *stream)
{
    if (!d) return fail(SLA_ERR_NULL, "layer descriptor is NULL");
    const sla_problem_t *p = &d->attn;
    if (d->flags & ~STU_REUSE_SCHEDULE) return fail(SLA_ERR_INVALID, "unknown layer flags");
    sla_status_t st = validate_problem(p);
    if (st != SLA_OK) return st;
    if (p->dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "the STU layer is bf16 only");
    if (p->out_f32) return fail(SLA_ERR_UNSUPPORTED, "the STU layer stores bf16 (out_f32 must be 0)");
    if (!x || !ln1_w || !w_uvqk || !ln2_w || !w_out || !out)
        return fail(SLA_ERR_NULL, "a required layer pointer is NULL");
    const int D = d->hidden, H = p->num_heads, dv = p->d_v, dqk = p->d_qk;
    const int NU = H * dv, NW = 2 * H * dv + 2 * H * dqk;
    if (D <= 0 || D % 128 != 0 || D > 2048)
        return fail(SLA_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 128, <= 2048", D);
    if (NU % 64 != 0 || NU > 2048)
        return fail(SLA_ERR_UNSUPPORTED, "H*d_v = %d must be a multiple of 64, <= 2048", NU);
    if (!(d->ln_eps > 0.0f) || !std::isfinite(d->ln_eps))
        return fail(SLA_ERR_INVALID, "ln_eps must be positive");
    if (out == x) return fail(SLA_ERR_INVALID, "out must not alias x");
    const void *ptrs[] = {x, w_uvqk, w_out, out, uvqk_out, attn_out, workspace,
                          ln1_w, ln1_b, ln2_w, ln2_b};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return fail(SLA_ERR_UNSUPPORTED, "a layer buffer is not 16-byte aligned");
    const size_t need = stu_layer_workspace_size(d);
    if (!workspace || ws_bytes < need)
        return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", ws_bytes, need);
    if ((st = check_device()) != SLA_OK) return st;
    const int64_t T = p->total_tokens;
    if (T == 0 || p->batch == 0) return SLA_OK;

    char *w = static_cast<char *>(workspace);
    void *n = w;
    w += round_up((size_t)T * D * 2, 256);
    void *uvqk_ws = w;
    w += round_up((size_t)T * NW * 2, 256);
    void *A = attn_out ? attn_out : w;
    w += round_up((size_t)T * NU * 2, 256);
    void *y = w;
    w += round_up((size_t)T * NU * 2, 256);
    void *attn_ws = w;
    const size_t attn_bytes = layout(p, SLA_OP_FWD).total;
    void *uvqk = uvqk_out ? uvqk_out : uvqk_ws;
    uint16_t *u16 = static_cast<uint16_t *>(uvqk);

    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = validate_layout(p->batch, T, p->offsets, p->num_targets, -1, workspace, s)) != SLA_OK)
        return st;
    hipError_t e = launch_layernorm_bf16(x, ln1_w, ln1_b, n, T, D, d->ln_eps, s);
    if (e != hipSuccess) return hip_fail(e, "layernorm");
    e = launch_gemm_bf16(n, D, w_uvqk, D, b_uvqk, nullptr, 0, uvqk, NW, nullptr, 0, T, NW, D, 0, s);
    if (e != hipSuccess) return hip_fail(e, "uvqk projection");
    // U | V | Q | K column blocks of the fused projection
    st = fwd_impl(p, u16 + 2 * NU, NW, u16 + 2 * NU + H * dqk, NW, u16 + NU, NW, A, NU, attn_ws,
                 attn_bytes, stream,
                  !(d->flags & STU_REUSE_SCHEDULE));
    if (st != SLA_OK) return st;
    e = launch_gated_layernorm_bf16(A, NU, u16, NW, ln2_w, ln2_b, y, T, NU, d->ln_eps, s);
    if (e != hipSuccess) return hip_fail(e, "gated layernorm");
    e = launch_gemm_bf16(y, NU, w_out, NU, b_out, x, D, out, D, nullptr, 0, T, D, NU, 1, s);
    if (e != hipSuccess) return hip_fail(e, "output projection");
    return SLA_OK;
}

size_t stu_layer_bwd_workspace_size(const stu_layer_desc_t *d)
{
    if (!d || validate_problem(&d->attn) != SLA_OK || d->hidden <= 0) return 0;
    return stu_bwd_layout(d).total;
}

sla_status_t stu_layer_bwd(const stu_layer_desc_t *d, const void *x, const void *attn,
                           const float *ln1_w, const float *ln1_b, const void *w_uvqk,
                           const float *b_uvqk, const float *ln2_w, const float *ln2_b,
                           const void *w_out, const float *b_out, const void *dout, void *dx,
                           float *dln1_w, float *dln1_b, float *dw_uvqk, float *db_uvqk,
                           float *dln2_w, float *dln2_b, float *dw_out, float *db_out,
                           void *workspace, size_t ws_bytes, void *stream)
{
    if (!d) return fail(SLA_ERR_NULL, "layer descriptor is NULL");
    const sla_problem_t *p = &d->attn;
    if (d->flags) return fail(SLA_ERR_INVALID, "stu_layer_bwd takes no layer flags");
    sla_status_t st = validate_problem(p);
    if (st != SLA_OK) return st;
    if (p->dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "the STU layer is bf16 only");
    if (p->out_f32) return fail(SLA_ERR_UNSUPPORTED, "the STU layer stores bf16 (out_f32 must be 0)");
    if (!ln1_w || !w_uvqk || !ln2_w || !w_out)
        return fail(SLA_ERR_NULL, "a required layer pointer is NULL");
    if (p->total_tokens > 0 && (!x || !dout || !dx))
        return fail(SLA_ERR_NULL, "x, dout or dx is NULL");
    const int D = d->hidden, H = p->num_heads, dv = p->d_v, dqk = p->d_qk;
    const int NU = H * dv, NQK = H * dqk, NW = 2 * NU + 2 * NQK;
    if (D <= 0 || D % 128 != 0 || D > 2048)
        return fail(SLA_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 128, <= 2048", D);
    if (NU % 128 != 0 || NU > 2048)
        return fail(SLA_ERR_UNSUPPORTED, "H*d_v = %d must be a multiple of 128, <= 2048", NU);
    if ((2 * NQK) % 128 != 0)
        return fail(SLA_ERR_UNSUPPORTED, "2*H*d_qk = %d must be a multiple of 128", 2 * NQK);
    if (!(d->ln_eps > 0.0f) || !std::isfinite(d->ln_eps))
        return fail(SLA_ERR_INVALID, "ln_eps must be positive");
    if (dx && (dx == x || dx == dout || dx == attn))
        return fail(SLA_ERR_INVALID, "dx must not alias an input");
    const void *ptrs[] = {x, attn, w_uvqk, w_out, dout, dx, workspace, ln1_w, ln1_b, ln2_w, ln2_b};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return fail(SLA_ERR_UNSUPPORTED, "a layer buffer is not 16-byte aligned");
    const StuBwdLayout L = stu_bwd_layout(d);
    if (!workspace || ws_bytes < L.total)
        return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", ws_bytes, L.total);
    if ((st = check_device()) != SLA_OK) return st;
    const int64_t T = p->total_tokens;
    if (T == 0 || p->batch == 0) {
        // no tokens: every parameter gradient is zero
        hipStream_t s0 = static_cast<hipStream_t>(stream);
        const struct { float *ptr; size_t n; } z[] = {
            {dln1_w, (size_t)D}, {dln1_b, (size_t)D}, {dw_uvqk, (size_t)NW * D},
            {db_uvqk, (size_t)NW}, {dln2_w, (size_t)NU}, {dln2_b, (size_t)NU},
            {dw_out, (size_t)D * NU}, {db_out, (size_t)D}};
        for (const auto &g : z)
            if (g.ptr) {
                hipError_t e = launch_fill_f32(g.ptr, g.n, 0.0f, s0);
                if (e != hipSuccess) return hip_fail(e, "gradient fill");
            }
        return SLA_OK;
    }

    char *base = static_cast<char *>(workspace);
    uint16_t *n = reinterpret_cast<uint16_t *>(base + L.n);
    uint16_t *z = reinterpret_cast<uint16_t *>(base + L.z);
    uint16_t *uvqk = reinterpret_cast<uint16_t *>(base + L.uvqk);
    uint16_t *A = attn ? static_cast<uint16_t *>(const_cast<void *>(attn))
                       : reinterpret_cast<uint16_t *>(base + L.A);
    uint16_t *y = reinterpret_cast<uint16_t *>(base + L.y);
    uint16_t *dy = reinterpret_cast<uint16_t *>(base + L.dy);
    uint16_t *dA = reinterpret_cast<uint16_t *>(base + L.dA);
    uint16_t *dz = reinterpret_cast<uint16_t *>(base + L.dz);
    uint16_t *dn = reinterpret_cast<uint16_t *>(base + L.dn);
    uint16_t *wt = reinterpret_cast<uint16_t *>(base + L.wt);
    float *part = reinterpret_cast<float *>(base + L.part);
    float *scratch_w = reinterpret_cast<float *>(base + L.vec);  // sums of unwanted gradients
    float *mid = reinterpret_cast<float *>(base + L.mid);
    float *zero = reinterpret_cast<float *>(base + L.zero);
    void *attn_ws = base + L.attn;
    const size_t attn_bytes = L.total - L.attn;
    auto or_scratch = [&](float *g) { return g ? g : scratch_w; };

    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = validate_layout(p->batch, T, p->offsets, p->num_targets, -1, workspace, s)) != SLA_OK)
        return st;
    hipError_t e;
#define STU_TRY(call, what)                      \
    do {                                         \
        e = (call);                              \
        if (e != hipSuccess) return hip_fail(e, what); \
    } while (0)
    STU_TRY(launch_fill_f32(zero, 256, 0.0f, s), "zero row");
    // recomputed activations: n, z, uvqk = SiLU(z), A (unless saved)
    STU_TRY(launch_layernorm_bf16(x, ln1_w, ln1_b, n, T, D, d->ln_eps, s), "layernorm");
    STU_TRY(launch_gemm_bf16(n, D, w_uvqk, D, b_uvqk, nullptr, 0, uvqk, NW, z, NW, T, NW, D, 3, s),
            "uvqk projection");
    if (!attn) {
        st = sla_fwd(p, uvqk + 2 * NU, NW, uvqk + 2 * NU + NQK, NW, uvqk + NU, NW, A, NU, attn_ws,
                     attn_bytes, stream);
        if (st != SLA_OK) return st;
    }
    // output projection input gradient: dy = dout W2 (W2^T staged as [NU][D])
    STU_TRY(launch_transpose_bf16(w_out, D, NU, wt, s), "weight transpose");
    STU_TRY(launch_gemm_bf16(dout, D, wt, D, nullptr, nullptr, 0, dy, NU, nullptr, 0, T, NU, D, 2,
                             s),
            "dy product");
    // gated LayerNorm: dA, dU (into the U block of dz), dln2, and y itself
    STU_TRY(launch_ln_bwd_bf16(true, A, NU, dy, NU, uvqk, NW, ln2_w, ln2_b, nullptr, 0, dA, NU, dz,
                               NW, dw_out ? y : nullptr, NU, part,
                               part + (size_t)ln_bwd_blocks(T) * NU, mid, or_scratch(dln2_w),
                               dln2_b, T, NU, d->ln_eps, s),
            "gated layernorm backward");
    // output projection weights: dW2 = dout^T y, db_out
    if (dw_out)
        STU_TRY(launch_gemm_tn_bf16(dout, D, y, NU, T, D, NU, zero, part, dw_out, s),
                "output weight gradient");
    if (db_out)
        STU_TRY(launch_colsum_bf16(dout, D, T, D, part, db_out, mid, s), "output bias gradient");
    // attention: dQ, dK, dV into their blocks of dz
    st = sla_bwd(p, uvqk + 2 * NU, NW, uvqk + 2 * NU + NQK, NW, uvqk + NU, NW, dA, NU, dz + 2 * NU,
                 NW, dz + 2 * NU + NQK, NW, dz + NU, NW, attn_ws, attn_bytes, stream);
    if (st != SLA_OK) return st;
    // SiLU: dz = d[U|V|Q|K] (.) SiLU'(z); dW1 = dz^T n, db_uvqk, dn = dz W1
    STU_TRY(launch_dsilu_bf16(dz, NW, z, NW, T, NW, s), "SiLU backward");
    if (dw_uvqk)
        STU_TRY(launch_gemm_tn_bf16(dz, NW, n, D, T, NW, D, zero, part, dw_uvqk, s),
                "projection weight gradient");
    if (db_uvqk)
        STU_TRY(launch_colsum_bf16(dz, NW, T, NW, part, db_uvqk, mid, s), "projection bias gradient");
    STU_TRY(launch_transpose_bf16(w_uvqk, NW, D, wt, s), "weight transpose");
    STU_TRY(launch_gemm_bf16(dz, NW, wt, NW, nullptr, nullptr, 0, dn, D, nullptr, 0, T, D, NW, 2, s),
            "dn product");
    // LayerNorm 1 with the residual: dx = LN backward + dout
    STU_TRY(launch_ln_bwd_bf16(false, x, D, dn, D, nullptr, 0, ln1_w, ln1_b, dout, D, dx, D,
                               nullptr, 0, nullptr, 0, part, part + (size_t)ln_bwd_blocks(T) * D,
                               mid, or_scratch(dln1_w), dln1_b, T, D, d->ln_eps, s),
            "layernorm backward");
#undef STU_TRY
    return SLA_OK;
}

sla_status_t stu_quantize_rows_fp8(const void *x, int64_t rows, int32_t cols, void *q,
                                   float *scale, void *stream)
{
    if (rows < 0) return fail(SLA_ERR_INVALID, "negative rows");
    if (rows == 0) return SLA_OK;
    if (!x || !q || !scale) return fail(SLA_ERR_NULL, "x, q or scale is NULL");
    if (cols <= 0 || cols % 16 != 0 || cols > 2048)
        return fail(SLA_ERR_UNSUPPORTED, "cols %d must be a positive multiple of 16, <= 2048",
                    cols);
    if (!aligned16(x) || !aligned16(q)) return fail(SLA_ERR_UNSUPPORTED, "x or q not 16-byte aligned");
    sla_status_t st = check_device();
    if (st != SLA_OK) return st;
    hipError_t e = launch_quant_rows_fp8(x, cols, rows, cols, q, scale,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "quantisation kernel");
    return SLA_OK;
}

size_t stu_layer_fp8_workspace_size(const stu_layer_desc_t *d)
{
    if (!d || validate_problem(&d->attn) != SLA_OK || d->hidden <= 0) return 0;
    const sla_problem_t *p = &d->attn;
    const size_t T = (size_t)p->total_tokens, H = (size_t)p->num_heads;
    const size_t NU = H * p->d_v, NW = 2 * H * p->d_v + 2 * H * p->d_qk;
    size_t bytes = 0;
    bytes += round_up(T * d->hidden, 256);  // n, e4m3
    bytes += round_up(T * 4, 256);          // its row scales
    bytes += round_up(T * NW * 2, 256);     // uvqk
    bytes += round_up(T * NU * 2, 256);     // A
    bytes += round_up(T * NU, 256);         // y, e4m3
    bytes += round_up(T * 4, 256);          // its row scales
    bytes += layout(p, SLA_OP_FWD).total;   // attention schedule
    return bytes;
}

sla_status_t stu_layer_fwd_fp8(const stu_layer_desc_t *d, const void *x, const float *ln1_w,
                               const float *ln1_b, const void *w_uvqk_q,
                               const float *w_uvqk_scale, const float *b_uvqk,
                               const float *ln2_w, const float *ln2_b, const void *w_out_q,
                               const float *w_out_scale, const float *b_out, void *out,
                               void *uvqk_out, void *attn_out, void *workspace, size_t ws_bytes,
                               void *stream)
{
    if (!d) return fail(SLA_ERR_NULL, "layer descriptor is NULL");
    const sla_problem_t *p = &d->attn;
    if (d->flags & ~STU_REUSE_SCHEDULE) return fail(SLA_ERR_INVALID, "unknown layer flags");
    sla_status_t st = validate_problem(p);
    if (st != SLA_OK) return st;
    if (p->dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "the STU layer is bf16 only");
    if (p->out_f32) return fail(SLA_ERR_UNSUPPORTED, "the STU layer stores bf16 (out_f32 must be 0)");
    if (!x || !ln1_w || !w_uvqk_q || !w_uvqk_scale || !ln2_w || !w_out_q || !w_out_scale || !out)
        return fail(SLA_ERR_NULL, "a required layer pointer is NULL");
    const int D = d->hidden, H = p->num_heads, dv = p->d_v, dqk = p->d_qk;
    const int NU = H * dv, NW = 2 * H * dv + 2 * H * dqk;
    if (D <= 0 || D % 128 != 0 || D > 2048)
        return fail(SLA_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 128, <= 2048", D);
    if (NU % 128 != 0 || NU > 2048)
        return fail(SLA_ERR_UNSUPPORTED, "H*d_v = %d must be a multiple of 128, <= 2048", NU);
    if (!(d->ln_eps > 0.0f) || !std::isfinite(d->ln_eps))
        return fail(SLA_ERR_INVALID, "ln_eps must be positive");
    if (out == x) return fail(SLA_ERR_INVALID, "out must not alias x");
    const void *ptrs[] = {x, w_uvqk_q, w_out_q, out, uvqk_out, attn_out, workspace,
                          ln1_w, ln1_b, ln2_w, ln2_b};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return fail(SLA_ERR_UNSUPPORTED, "a layer buffer is not 16-byte aligned");
    const size_t need = stu_layer_fp8_workspace_size(d);
    if (!workspace || ws_bytes < need)
        return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", ws_bytes, need);
    if ((st = check_device()) != SLA_OK) return st;
    const int64_t T = p->total_tokens;
    if (T == 0 || p->batch == 0) return SLA_OK;

    char *w = static_cast<char *>(workspace);
    void *nq = w;
    w += round_up((size_t)T * D, 256);
    float *sn = reinterpret_cast<float *>(w);
    w += round_up((size_t)T * 4, 256);
    void *uvqk_ws = w;
    w += round_up((size_t)T * NW * 2, 256);
    void *A = attn_out ? attn_out : w;
    w += round_up((size_t)T * NU * 2, 256);
    void *yq = w;
    w += round_up((size_t)T * NU, 256);
    float *sy = reinterpret_cast<float *>(w);
    w += round_up((size_t)T * 4, 256);
    void *attn_ws = w;
    const size_t attn_bytes = layout(p, SLA_OP_FWD).total;
    void *uvqk = uvqk_out ? uvqk_out : uvqk_ws;
    uint16_t *u16 = static_cast<uint16_t *>(uvqk);

    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = validate_layout(p->batch, T, p->offsets, p->num_targets, -1, workspace, s)) != SLA_OK)
        return st;
    hipError_t e = launch_ln_quant_fp8(false, x, D, nullptr, 0, ln1_w, ln1_b, nq, sn, T, D,
                                       d->ln_eps, s);
    if (e != hipSuccess) return hip_fail(e, "layernorm + quantisation");
    e = launch_gemm_fp8(nq, sn, w_uvqk_q, w_uvqk_scale, b_uvqk, nullptr, 0, uvqk, NW, T, NW, D, 0,
                        s);
    if (e != hipSuccess) return hip_fail(e, "uvqk projection (fp8)");
    st = fwd_impl(p, u16 + 2 * NU, NW, u16 + 2 * NU + H * dqk, NW, u16 + NU, NW, A, NU, attn_ws,
                 attn_bytes, stream,
                  !(d->flags & STU_REUSE_SCHEDULE));
    if (st != SLA_OK) return st;
    e = launch_ln_quant_fp8(true, A, NU, u16, NW, ln2_w, ln2_b, yq, sy, T, NU, d->ln_eps, s);
    if (e != hipSuccess) return hip_fail(e, "gated layernorm + quantisation");
    e = launch_gemm_fp8(yq, sy, w_out_q, w_out_scale, b_out, x, D, out, D, T, D, NU, 1, s);
    if (e != hipSuccess) return hip_fail(e, "output projection (fp8)");
    return SLA_OK;
}

sla_status_t stu_gather_targets(int32_t batch, int64_t total_tokens, const int64_t *offsets,
                                const int32_t *num_targets, const void *x, int32_t hidden,
                                int32_t dtype, int64_t *target_offsets, void *out, int64_t ld_out,
                                int64_t col_offset, int64_t capacity, void *stream)
{
    if (batch < 0 || total_tokens < 0) return fail(SLA_ERR_INVALID, "negative batch or total_tokens");
    if (!target_offsets) return fail(SLA_ERR_NULL, "target_offsets is NULL");
    if (batch > 0 && (!offsets || !num_targets))
        return fail(SLA_ERR_NULL, "offsets or num_targets is NULL");
    if (dtype != SLA_F32 && dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "bad dtype");
    const int eb = dtype == SLA_BF16 ? 2 : 4;
    if (capacity < 0) return fail(SLA_ERR_INVALID, "negative capacity");
    if (out) {
        if (!x) return fail(SLA_ERR_NULL, "x is NULL");
        if (hidden <= 0 || ((int64_t)hidden * eb) % 16 != 0)
            return fail(SLA_ERR_UNSUPPORTED, "hidden row must be a positive multiple of 16 bytes");
        if (col_offset < 0 || ld_out < col_offset + hidden)
            return fail(SLA_ERR_INVALID, "columns [col_offset, col_offset + hidden) exceed ld_out");
        if ((ld_out * eb) % 16 != 0 || (col_offset * eb) % 16 != 0)
            return fail(SLA_ERR_UNSUPPORTED, "ld_out and col_offset must be multiples of 16 bytes");
        if (!aligned16(x) || !aligned16(out))
            return fail(SLA_ERR_UNSUPPORTED, "x / out not 16-byte aligned");
    }
    sla_status_t st = check_device();
    if (st != SLA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = validate_layout(batch, total_tokens, offsets, num_targets, -1, target_offsets, s)) !=
        SLA_OK)
        return st;
    hipError_t e = launch_gather_targets(batch, offsets, num_targets, x, hidden * eb,
                                         target_offsets, out, ld_out * eb, col_offset * eb,
                                         capacity, s);
    if (e != hipSuccess) return hip_fail(e, "target gather kernels");
    return SLA_OK;
}

sla_status_t stu_truncate(int32_t batch, int64_t total_tokens, const int64_t *offsets,
                          const int32_t *num_targets, int32_t contextual_len, int32_t tail_len,
                          const void *x, int32_t hidden, int32_t dtype, int64_t *new_offsets,
                          int32_t *new_num_targets, int64_t *gather_idx, void *x_out,
                          int64_t capacity, void *stream)
{
    if (batch < 0 || total_tokens < 0 || contextual_len < 0)
        return fail(SLA_ERR_INVALID, "negative batch, total_tokens or contextual_len");
    if (tail_len < 1) return fail(SLA_ERR_INVALID, "tail_len must be >= 1");
    if (!new_offsets || (batch > 0 && !offsets)) return fail(SLA_ERR_NULL, "offsets is NULL");
    if (dtype != SLA_F32 && dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "bad dtype");
    const int eb = dtype == SLA_BF16 ? 2 : 4;
    if (x_out) {
        if (!x) return fail(SLA_ERR_NULL, "x is NULL");
        if (hidden <= 0 || ((int64_t)hidden * eb) % 16 != 0)
            return fail(SLA_ERR_UNSUPPORTED, "hidden row must be a positive multiple of 16 bytes");
        if (!aligned16(x) || !aligned16(x_out))
            return fail(SLA_ERR_UNSUPPORTED, "x / x_out not 16-byte aligned");
    }
    if (capacity < 0) return fail(SLA_ERR_INVALID, "negative capacity");
    if (batch > 0 && total_tokens >= (int64_t)1 << 30)
        return fail(SLA_ERR_UNSUPPORTED, "total_tokens too large");
    sla_status_t st = check_device();
    if (st != SLA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = validate_layout(batch, total_tokens, offsets, num_targets, contextual_len,
                              new_offsets, s)) != SLA_OK)
        return st;
    hipError_t e = launch_truncate(batch, total_tokens, offsets, num_targets, contextual_len,
                                   tail_len, x, hidden, eb, new_offsets, new_num_targets,
                                   gather_idx, x_out, capacity, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "truncation kernels");
    return SLA_OK;
}

sla_status_t stu_truncate_bwd(int32_t batch, int64_t total_tokens, const int64_t *offsets,
                              const int32_t *num_targets, int32_t contextual_len,
                              int32_t tail_len, const int64_t *new_offsets, const void *dy,
                              int32_t hidden, int32_t dtype, void *dx, void *stream)
{
    if (batch < 0 || total_tokens < 0 || contextual_len < 0)
        return fail(SLA_ERR_INVALID, "negative batch, total_tokens or contextual_len");
    if (tail_len < 1) return fail(SLA_ERR_INVALID, "tail_len must be >= 1");
    if (batch == 0 || total_tokens == 0) return SLA_OK;  // nothing is read or written
    if (!offsets || !new_offsets || !dy || !dx)
        return fail(SLA_ERR_NULL, "offsets, new_offsets, dy or dx is NULL");
    if (dtype != SLA_F32 && dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "bad dtype");
    const int eb = dtype == SLA_BF16 ? 2 : 4;
    if (hidden <= 0 || ((int64_t)hidden * eb) % 16 != 0)
        return fail(SLA_ERR_UNSUPPORTED, "hidden row must be a positive multiple of 16 bytes");
    if (!aligned16(dy) || !aligned16(dx))
        return fail(SLA_ERR_UNSUPPORTED, "dy / dx not 16-byte aligned");
    if (total_tokens >= (int64_t)1 << 30)
        return fail(SLA_ERR_UNSUPPORTED, "total_tokens too large");
    sla_status_t st = check_device();
    if (st != SLA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_truncate_bwd(batch, total_tokens, offsets, num_targets, contextual_len,
                                       tail_len, new_offsets, dy, hidden, eb, dx, s);
    if (e != hipSuccess) return hip_fail(e, "truncation backward kernel");
    return SLA_OK;
}

}  // extern "C"
