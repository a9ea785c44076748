// abi.hip -- host runtime behind the C ABI of libmoe_decode.so:
// argument validation, the context (workspace, streams, events), and the
// forward pass as an ordered list of kernel launches on the context stream.
//
// Nothing here waits on the device during a forward: the top-k / bucket
// kernels leave the routing plan in device memory and every later grid is sized for the
// worst case the request allows (B * k slots), so the host never learns how
// many experts were selected.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/moe_decode.h"
#include "moe_internal.h"

using namespace moe;

namespace {

thread_local std::string g_error;
thread_local moe_context* g_bound = nullptr;

moe_status fail(moe_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

moe_status ok() {
    g_error.clear();
    return MOE_OK;
}

size_t dtype_size(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Weight-row granularity: one wave-wide 16-byte-per-lane load covers
// 64 * (16 / sizeof(w)) elements.
int row_quantum(int wdt) { return 64 * 16 / (int)dtype_size(wdt); }

constexpr int kRouterChunk = 512;
constexpr int kTimingRing = 64;
// AUTO: batches up to this size use only GEMV kernels.  The pages' path uses
// GEMV-style kernels for one- and two-row batches; on MI355X the MFMA kernels
// already match them at two independent rows and beat them when rows share
// experts (whole layers at two rows: 429.7 against 430.0 us independent,
// 311.7 against 323.6 us correlated), so only one row stays on GEMV.
constexpr int kGemvMaxBatch = 1;

}  // namespace

struct moe_context {
    moe_config cfg;
    int device;
    hipStream_t stream;
    // workspace (one allocation)
    void* ws;
    size_t ws_bytes;
    double* logits;
    int* topk_idx;
    float* topk_w;
    DevPlan* plan;
    void* h;
    float* y;
    float* partial;        // split-K partial sums (own allocation, grown by set_path)
    size_t partial_bytes;
    int slot_cap;          // max_batch * max_topk
    // expert kernel choice
    int path;
    int mfma_min_rows;
    int split_k;
    int router;            // MOE_ROUTER_*
    int fused_combine;     // fold the combine into the down projection at batch 1
    int fused_select;      // at batch 1, the gate/up kernel takes the top-k selection
    int fused_next_router; // stacks: the combine folded into the next layer's router
    int last_router;       // router kernel of the last forward (ROUTER_GEMV / ROUTER_MFMA)
    int last_launches;     // kernels the last forward launched
    // prefetch ranges
    const void* pf_ptr[8];
    int64_t pf_bytes[8];
    int pf_n;
    int pf_start;          // 0: after the routing kernels; 1: with the forward's first launch
    int pf_grid;           // workgroups of the warm-up kernel
    hipStream_t side;
    hipEvent_t ev_fork;
    hipEvent_t ev_join;
    hipEvent_t ev_switch;  // orders a new context stream after the old one
    uint32_t* sink;        // prefetch kernel's (never written) result slot
    // timing: a ring of event sets, one per timed forward, read back lazily so
    // that timing never makes the host wait between forwards
    int timing;
    hipEvent_t ev[kTimingRing][MOE_STAGE_COUNT + 1];
    int ring_head;     // next set to record
    int ring_pending;  // recorded sets not yet read back (the oldest ones)
    double stage_ms[MOE_STAGE_COUNT];
    int64_t timed;
};

// ------------------------------------------------------------ validation

extern "C" moe_status moe_check_config(const moe_config* c) {
    if (!c) return fail(MOE_ERR_INVALID_ARG, "moe_check_config: cfg is NULL");
    if (c->weight_dtype < MOE_F32 || c->weight_dtype > MOE_FP8_E4M3)
        return fail(MOE_ERR_INVALID_ARG, "weight_dtype %d is not a moe_dtype", c->weight_dtype);
    if (c->act_dtype < MOE_F32 || c->act_dtype > MOE_FP8_E4M3)
        return fail(MOE_ERR_INVALID_ARG, "act_dtype %d is not a moe_dtype", c->act_dtype);
    const bool pair_ok = (c->weight_dtype == MOE_F32 && c->act_dtype == MOE_F32) ||
                         (c->weight_dtype == MOE_BF16 && c->act_dtype == MOE_BF16) ||
                         (c->weight_dtype == MOE_FP8_E4M3 && c->act_dtype == MOE_BF16);
    if (!pair_ok)
        return fail(MOE_ERR_UNSUPPORTED,
                    "weight/activation dtypes (%d, %d) unsupported: use (f32, f32), "
                    "(bf16, bf16) or (fp8_e4m3, bf16)",
                    c->weight_dtype, c->act_dtype);
    if (c->num_experts < 1 || c->num_experts > kMaxExperts)
        return fail(MOE_ERR_UNSUPPORTED, "num_experts %d outside 1..%d", c->num_experts,
                    kMaxExperts);
    const int q = row_quantum(c->weight_dtype);
    if (c->hidden < kRouterChunk || c->hidden > 8192 || c->hidden % kRouterChunk ||
        c->hidden % q)
        return fail(MOE_ERR_UNSUPPORTED,
                    "hidden %d unsupported: need a multiple of %d in [512, 8192]", c->hidden,
                    q > kRouterChunk ? q : kRouterChunk);
    if (c->inter < 1 || c->inter > 8192 || c->inter % q || c->inter % 256)
        return fail(MOE_ERR_UNSUPPORTED, "inter %d unsupported: need a multiple of %d, <= 8192",
                    c->inter, q > 256 ? q : 256);
    if (c->max_batch < 1 || c->max_batch > kMaxBatch)
        return fail(MOE_ERR_UNSUPPORTED, "max_batch %d outside 1..%d (decode batches only)",
                    c->max_batch, kMaxBatch);
    const int kcap = c->num_experts < kMaxTopk ? c->num_experts : kMaxTopk;
    if (c->max_topk < 1 || c->max_topk > kcap)
        return fail(MOE_ERR_UNSUPPORTED, "max_topk %d outside 1..%d", c->max_topk, kcap);
    return ok();
}

namespace {

// Byte range [lo, hi) of a strided matrix.
void mat_range(const moe_mat* m, uintptr_t* lo, uintptr_t* hi) {
    const size_t es = dtype_size(m->dtype);
    *lo = (uintptr_t)m->data;
    *hi = *lo + ((size_t)(m->rows - 1) * (size_t)m->row_stride + (size_t)m->cols) * es;
}

moe_status check_mat(const char* name, const moe_mat* m, int dtype, int rows, int cols) {
    if (!m) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
    if (!m->data) return fail(MOE_ERR_INVALID_ARG, "%s->data is NULL", name);
    if (m->dtype != dtype)
        return fail(MOE_ERR_UNSUPPORTED, "%s dtype %d, expected %d", name, m->dtype, dtype);
    if (m->rows != rows || m->cols != cols)
        return fail(MOE_ERR_INVALID_ARG, "%s is [%d][%d], expected [%d][%d]", name, m->rows,
                    m->cols, rows, cols);
    if (m->row_stride < m->cols)
        return fail(MOE_ERR_INVALID_ARG, "%s row_stride %lld < cols %d", name,
                    (long long)m->row_stride, m->cols);
    if (!aligned16(m->data) || ((size_t)m->row_stride * dtype_size(dtype)) % 16)
        return fail(MOE_ERR_INVALID_ARG, "%s data and row stride must be 16-byte aligned", name);
    return MOE_OK;
}

moe_status validate(const moe_config& c, const moe_mat* x, const moe_mat* router_w,
                    const moe_experts* ex, const moe_topk* tk, const moe_mat* out) {
    if (!x) return fail(MOE_ERR_INVALID_ARG, "x is NULL");
    if (x->rows < 1 || x->rows > c.max_batch)
        return fail(MOE_ERR_UNSUPPORTED, "batch %d outside 1..%d (context max_batch)", x->rows,
                    c.max_batch);
    const int B = x->rows;
    moe_status st;
    if ((st = check_mat("x", x, c.act_dtype, B, c.hidden)) != MOE_OK) return st;
    if ((st = check_mat("out", out, c.act_dtype, B, c.hidden)) != MOE_OK) return st;
    if ((st = check_mat("router_w", router_w, MOE_F32, c.num_experts, c.hidden)) != MOE_OK)
        return st;
    if (!ex) return fail(MOE_ERR_INVALID_ARG, "expert_w is NULL");
    if (ex->num_experts != c.num_experts || ex->hidden != c.hidden || ex->inter != c.inter)
        return fail(MOE_ERR_INVALID_ARG, "expert_w dims (%d, %d, %d) differ from the context's",
                    ex->num_experts, ex->hidden, ex->inter);
    if (ex->dtype != c.weight_dtype)
        return fail(MOE_ERR_UNSUPPORTED, "expert_w dtype %d, context built for %d", ex->dtype,
                    c.weight_dtype);
    if (!ex->w_gate_up || !ex->w_down)
        return fail(MOE_ERR_INVALID_ARG, "expert_w weight pointer is NULL");
    if (!aligned16(ex->w_gate_up) || !aligned16(ex->w_down))
        return fail(MOE_ERR_INVALID_ARG, "expert weights must be 16-byte aligned");
    if (c.weight_dtype == MOE_FP8_E4M3) {
        if (!ex->scale_gate_up || !ex->scale_down)
            return fail(MOE_ERR_INVALID_ARG, "fp8 weights need scale_gate_up and scale_down");
        if (((uintptr_t)ex->scale_gate_up | (uintptr_t)ex->scale_down) & 3u)
            return fail(MOE_ERR_INVALID_ARG, "scales must be 4-byte aligned");
    } else if (ex->scale_gate_up || ex->scale_down) {
        return fail(MOE_ERR_INVALID_ARG, "scales are only taken with fp8 weights");
    }
    if (!tk) return fail(MOE_ERR_INVALID_ARG, "topk is NULL");
    if (tk->k < 1 || tk->k > c.max_topk)
        return fail(MOE_ERR_UNSUPPORTED, "k %d outside 1..%d (context max_topk)", tk->k,
                    c.max_topk);
    if (tk->score_fn != MOE_SCORE_SOFTMAX && tk->score_fn != MOE_SCORE_SIGMOID)
        return fail(MOE_ERR_INVALID_ARG, "score_fn %d is not a moe_score_fn", tk->score_fn);
    if (((uintptr_t)tk->bias | (uintptr_t)tk->idx_out | (uintptr_t)tk->weight_out) & 3u)
        return fail(MOE_ERR_INVALID_ARG, "bias / idx_out / weight_out must be 4-byte aligned");
    // out may be x itself; any other overlap would let the combine read
    // activations it has already overwritten.
    uintptr_t xl, xh, ol, oh;
    mat_range(x, &xl, &xh);
    mat_range(out, &ol, &oh);
    const bool same = x->data == out->data && x->row_stride == out->row_stride;
    if (!same && ol < xh && xl < oh)
        return fail(MOE_ERR_INVALID_ARG, "out overlaps x without being x");
    return MOE_OK;
}

// Makes the context's device current for the scope of a call and restores
// the caller's device afterwards; status is the result of the switch, which
// callers check before any device work.
struct DeviceGuard {
    int prev = -1;
    hipError_t status = hipSuccess;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) status = hipSetDevice(dev);
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev)
            (void)hipSetDevice(prev);  // nothing to report to from a destructor
    }
};

moe_status hip_fail(const char* what, hipError_t e) {
    return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Byte offsets of a forward's workspace for batches of up to max_batch rows
// and max_topk choices: router logits (up to kMaxRouterSplits partial
// slices, fp64), the selection and its weights, the routing plan, h (act)
// and y (fp32); each piece 256-byte aligned.
struct WsLayout {
    size_t logits, topk_idx, topk_w, plan, h, y, sink, total;
};

WsLayout ws_layout(int max_batch, int max_topk, int E, int H, int I, int act) {
    const size_t slots = (size_t)max_batch * max_topk;
    WsLayout L;
    size_t off = 0;
    auto carve = [&](size_t bytes) {
        size_t at = off;
        off = round_up(off + bytes, 256);
        return at;
    };
    L.logits = carve(sizeof(double) * kMaxRouterSplits * max_batch * E);
    L.topk_idx = carve(sizeof(int) * slots);
    L.topk_w = carve(sizeof(float) * slots);
    L.plan = carve(sizeof(DevPlan));
    L.h = carve(dtype_size(act) * slots * I);
    L.y = carve(sizeof(float) * slots * H);
    L.sink = carve(1024);
    L.total = off;
    return L;
}

}  // namespace

// --------------------------------------------------------------- context

extern "C" moe_status moe_context_create(const moe_config* cfg, void* hip_stream,
                                         moe_context** out) {
    if (!out) return fail(MOE_ERR_INVALID_ARG, "moe_context_create: out is NULL");
    *out = nullptr;
    moe_status st = moe_check_config(cfg);
    if (st != MOE_OK) return st;

    moe_context* c = new moe_context();
    memset(c, 0, sizeof *c);
    c->cfg = *cfg;
    c->stream = (hipStream_t)hip_stream;
    c->path = PATH_AUTO;
    c->mfma_min_rows = 1;
    c->split_k = 0;
    c->router = ROUTER_AUTO;
    c->fused_combine = 1;
    c->fused_select = 0;
    c->pf_grid = 128;
    hipError_t e = hipGetDevice(&c->device);
    if (e != hipSuccess) {
        delete c;
        return hip_fail("hipGetDevice", e);
    }

    const size_t slots = (size_t)cfg->max_batch * cfg->max_topk;
    const WsLayout lay = ws_layout(cfg->max_batch, cfg->max_topk, cfg->num_experts, cfg->hidden,
                                   cfg->inter, cfg->act_dtype);
    c->ws_bytes = lay.total;

    e = hipMalloc(&c->ws, c->ws_bytes);
    if (e != hipSuccess) {
        delete c;
        return hip_fail("hipMalloc(workspace)", e);
    }
    char* base = (char*)c->ws;
    c->logits = (double*)(base + lay.logits);
    c->topk_idx = (int*)(base + lay.topk_idx);
    c->topk_w = (float*)(base + lay.topk_w);
    c->plan = (DevPlan*)(base + lay.plan);
    c->h = base + lay.h;
    c->y = (float*)(base + lay.y);
    c->sink = (uint32_t*)(base + lay.sink);
    c->slot_cap = (int)slots;
    // zero the workspace once (every forward writes what it later reads)
    e = hipMemset(c->ws, 0, c->ws_bytes);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_switch, hipEventDisableTiming);
    for (int r = 0; r < kTimingRing; ++r)
        for (int i = 0; e == hipSuccess && i <= MOE_STAGE_COUNT; ++i) e = hipEventCreate(&c->ev[r][i]);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        moe_context_destroy(c);
        return hip_fail("moe_context_create", e);
    }
    g_bound = c;
    *out = c;
    return ok();
}

extern "C" moe_status moe_context_destroy(moe_context* c) {
    if (!c) return ok();
    // release everything even if a step fails; report the first failure
    hipError_t first = hipSuccess;
    auto note = [&](hipError_t e) {
        if (first == hipSuccess && e != hipSuccess) first = e;
    };
    DeviceGuard g(c->device);
    note(g.status);
    if (c->stream || c->ws) note(hipStreamSynchronize(c->stream));
    if (c->side) {
        note(hipStreamSynchronize(c->side));
        note(hipStreamDestroy(c->side));
    }
    if (c->ev_fork) note(hipEventDestroy(c->ev_fork));
    if (c->ev_join) note(hipEventDestroy(c->ev_join));
    if (c->ev_switch) note(hipEventDestroy(c->ev_switch));
    for (int r = 0; r < kTimingRing; ++r)
        for (int i = 0; i <= MOE_STAGE_COUNT; ++i)
            if (c->ev[r][i]) note(hipEventDestroy(c->ev[r][i]));
    if (c->ws) note(hipFree(c->ws));
    if (c->partial) note(hipFree(c->partial));
    if (g_bound == c) g_bound = nullptr;
    delete c;
    return first == hipSuccess ? ok() : hip_fail("moe_context_destroy", first);
}

// Every later launch of the context goes to the new stream, after all work
// already queued on the old one (an event recorded on the old stream, waited
// on by the new): forwards that share the workspace never overlap, and
// synchronising the current stream (destroy, set_path) also waits for work
// queued on every earlier stream.
extern "C" moe_status moe_context_set_stream(moe_context* c, void* hip_stream) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_context_set_stream: ctx is NULL");
    hipStream_t s = (hipStream_t)hip_stream;
    if (s == c->stream) return ok();
    DeviceGuard g(c->device);
    hipError_t e = g.status;
    if (e == hipSuccess) e = hipEventRecord(c->ev_switch, c->stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, c->ev_switch, 0);
    if (e != hipSuccess) return hip_fail("moe_context_set_stream", e);
    c->stream = s;
    return ok();
}

extern "C" moe_status moe_context_set_path(moe_context* c, int32_t path, int32_t mfma_min_rows,
                                           int32_t split_k) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_context_set_path: ctx is NULL");
    if (path < MOE_PATH_AUTO || path > MOE_PATH_MFMA)
        return fail(MOE_ERR_INVALID_ARG, "path %d is not a moe_path", path);
    if (mfma_min_rows < 0 || mfma_min_rows > kMaxBatch)
        return fail(MOE_ERR_INVALID_ARG, "mfma_min_rows %d outside 0..%d", mfma_min_rows,
                    kMaxBatch);
    if (split_k < 0 || split_k > 16)
        return fail(MOE_ERR_INVALID_ARG, "split_k %d outside 0..16", split_k);
    // split-K partial sums: [split_k][slot_cap][max(2I, H)] fp32, grown here
    // (never during a forward) once queued work is done with the old buffer
    const moe_config& cfg = c->cfg;
    const size_t wide = (size_t)(2 * cfg.inter > cfg.hidden ? 2 * cfg.inter : cfg.hidden);
    const size_t need = split_k > 1 ? (size_t)split_k * c->slot_cap * wide * sizeof(float) : 0;
    if (need > c->partial_bytes) {
        DeviceGuard g(c->device);
        hipError_t e = g.status;
        if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
        if (e == hipSuccess && c->partial) e = hipFree(c->partial);
        if (e != hipSuccess) return hip_fail("moe_context_set_path", e);
        c->partial = nullptr;
        c->partial_bytes = 0;
        e = hipMalloc(&c->partial, need);
        if (e != hipSuccess) {
            c->partial = nullptr;
            return hip_fail("hipMalloc(split-K partials)", e);
        }
        c->partial_bytes = need;
    }
    c->path = path;
    if (mfma_min_rows) c->mfma_min_rows = mfma_min_rows;
    c->split_k = split_k;
    return ok();
}

extern "C" moe_status moe_context_set_router(moe_context* c, int32_t kernel) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_context_set_router: ctx is NULL");
    if (kernel < MOE_ROUTER_AUTO || kernel > MOE_ROUTER_MFMA)
        return fail(MOE_ERR_INVALID_ARG, "router kernel %d is not a moe_router_kernel", kernel);
    c->router = kernel;
    return ok();
}

extern "C" moe_status moe_context_set_fused_combine(moe_context* c, int32_t enable) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_context_set_fused_combine: ctx is NULL");
    c->fused_combine = enable != 0;
    return ok();
}

extern "C" moe_status moe_context_set_fused_next_router(moe_context* c, int32_t enable) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_context_set_fused_next_router: ctx is NULL");
    c->fused_next_router = enable != 0;
    return ok();
}

extern "C" moe_status moe_context_set_fused_select(moe_context* c, int32_t enable) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_context_set_fused_select: ctx is NULL");
    c->fused_select = enable != 0;
    return ok();
}

extern "C" moe_status moe_context_set_prefetch_mode(moe_context* c, int32_t start, int32_t grid) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_context_set_prefetch_mode: ctx is NULL");
    if (start < 0 || start > 1) return fail(MOE_ERR_INVALID_ARG, "prefetch start %d not 0 or 1", start);
    if (grid < 0 || grid > 65536)
        return fail(MOE_ERR_INVALID_ARG, "prefetch grid %d outside 0..65536", grid);
    c->pf_start = start;
    c->pf_grid = grid ? grid : 128;
    return ok();
}

extern "C" moe_status moe_context_set_prefetch(moe_context* c, const void* const* ptrs,
                                               const int64_t* bytes, int32_t n) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_context_set_prefetch: ctx is NULL");
    if (n < 0 || n > 8) return fail(MOE_ERR_INVALID_ARG, "prefetch range count %d outside 0..8", n);
    if (n && (!ptrs || !bytes)) return fail(MOE_ERR_INVALID_ARG, "prefetch ptrs/bytes NULL");
    for (int i = 0; i < n; ++i) {
        if (!ptrs[i] || bytes[i] < 0 || !aligned16(ptrs[i]))
            return fail(MOE_ERR_INVALID_ARG, "prefetch range %d: NULL, negative or unaligned", i);
    }
    for (int i = 0; i < n; ++i) {
        c->pf_ptr[i] = ptrs[i];
        c->pf_bytes[i] = bytes[i];
    }
    c->pf_n = n;
    return ok();
}

namespace {

// Read back the oldest recorded event sets until at most `keep` remain.
void collect_timing(moe_context* c, int keep) {
    while (c->ring_pending > keep) {
        const int r = (c->ring_head - c->ring_pending + kTimingRing) % kTimingRing;
        c->ring_pending -= 1;
        if (hipEventSynchronize(c->ev[r][MOE_STAGE_COUNT]) != hipSuccess) continue;
        for (int s = 0; s < MOE_STAGE_COUNT; ++s) {
            float ms = 0.0f;
            if (hipEventElapsedTime(&ms, c->ev[r][s], c->ev[r][s + 1]) == hipSuccess)
                c->stage_ms[s] += ms;
        }
        c->timed += 1;
    }
}

}  // namespace

extern "C" moe_status moe_context_set_timing(moe_context* c, int32_t enable) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_context_set_timing: ctx is NULL");
    DeviceGuard g(c->device);
    if (g.status != hipSuccess) return hip_fail("moe_context_set_timing", g.status);
    collect_timing(c, 0);
    c->timing = enable != 0;
    return ok();
}

extern "C" moe_status moe_context_get_timing(moe_context* c, double* ms, int64_t* count,
                                             int32_t reset) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_context_get_timing: ctx is NULL");
    DeviceGuard g(c->device);
    if (g.status != hipSuccess) return hip_fail("moe_context_get_timing", g.status);
    collect_timing(c, 0);
    for (int s = 0; s < MOE_STAGE_COUNT; ++s)
        if (ms) ms[s] = c->stage_ms[s];
    if (count) *count = c->timed;
    if (reset) {
        for (int s = 0; s < MOE_STAGE_COUNT; ++s) c->stage_ms[s] = 0.0;
        c->timed = 0;
    }
    return ok();
}

extern "C" moe_status moe_context_last_plan(moe_context* c, int32_t* out) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_context_last_plan: ctx is NULL");
    if (!out) return fail(MOE_ERR_INVALID_ARG, "moe_context_last_plan: out is NULL");
    DeviceGuard g(c->device);
    int hdr[5];
    hipError_t e = g.status;
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e == hipSuccess) e = hipMemcpy(hdr, c->plan, sizeof hdr, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail("moe_context_last_plan", e);
    // DevPlan header: num_slots, num_active, n_list[0], n_list[1], max_rows
    out[0] = hdr[1];
    out[1] = hdr[2];
    out[2] = hdr[3];
    out[3] = hdr[4];
    out[4] = c->last_launches;
    out[5] = c->last_router;
    return ok();
}

extern "C" moe_status moe_context_bind(moe_context* c) {
    g_bound = c;
    return ok();
}

extern "C" const char* moe_last_error(void) { return g_error.c_str(); }

// --------------------------------------------------------------- forward

namespace {

// The device buffers one forward works in, and the kernel choices it makes:
// a context's (moe_decode_forward_ctx) or the defaults over the file-scope
// scratch array (moe_decode_forward_noalloc).
struct Workspace {
    double* logits;
    int* topk_idx;
    float* topk_w;
    DevPlan* plan;
    void* h;
    float* y;
    float* partial;  // split-K partial sums (null when split_k <= 1)
    int slot_cap;
};

struct Knobs {
    int path, mfma_min_rows, split_k, router, fused_combine, fused_select;
};

// How a layer of a stack meets its neighbours: logits_ready > 0 when the
// previous layer's combine + router kernel left this many slices of this
// layer's logits in the workspace (its router is not launched);
// next_router_w, when set, is the next layer's router, whose logits this
// layer's combine then computes in the same launch (*next_splits receives
// their slices).
struct StackLink {
    int logits_ready;
    const moe_mat* next_router_w;
    int* next_splits;
};

// The forward's launches on stream s (arguments already validated, the
// device already current).  c, when not null, is the context whose timing
// events and prefetch side stream the forward also uses.
moe_status launch_layer(const moe_config& cfg, const Knobs& kn, const Workspace& ws,
                        hipStream_t s, const moe_mat* x, const moe_mat* router_w,
                        const moe_experts* ex, const moe_topk* tk, moe_mat* out, moe_context* c,
                        int* router_out, int* launches_out, const StackLink& link = {0, nullptr, nullptr}) {
    // clear any error state an unrelated earlier HIP call left on this thread,
    // so that the launch checks below report this forward's own launches
    (void)hipGetLastError();
    hipError_t e = hipSuccess;

    const int B = x->rows, k = tk->k, E = cfg.num_experts;
    const int act = cfg.act_dtype, wdt = cfg.weight_dtype;
    const int slots = B * k;
    const int max_experts = slots < E ? slots : E;
    // MFMA kernels exist for bf16 and fp8 weights.  AUTO follows the batch
    // size first (small-matrix GEMV kernels for one row),
    // then the per-expert row threshold.  Which expert lists can be non-empty
    // is known on the host from B alone: an expert has at most B rows.
    const int mfma_ok = wdt == MOE_BF16 || wdt == MOE_FP8_E4M3;
    const int path = (kn.path == PATH_AUTO && B <= kGemvMaxBatch) ? PATH_GEMV : kn.path;
    const int min_rows = kn.mfma_min_rows;
    // an expert reaches the MFMA kernels under AUTO with min_rows rows, or
    // with more rows than the GEMV kernels stage in one pass
    const int mfma_rows = min_rows < kGemvPassRows + 1 ? min_rows : kGemvPassRows + 1;
    const bool run_mfma =
        mfma_ok && (path == PATH_MFMA || (path == PATH_AUTO && B >= mfma_rows));
    const bool run_gemv =
        !mfma_ok || path == PATH_GEMV || (path == PATH_AUTO && min_rows > 1);
    // AUTO gives the GEMV kernels experts with fewer than min_rows rows, and
    // never more than they stage in one pass
    const int auto_gemv_rows = min_rows - 1 < kGemvPassRows ? min_rows - 1 : kGemvPassRows;
    const int gemv_rows = (path == PATH_AUTO && mfma_ok && auto_gemv_rows < B) ? auto_gemv_rows : B;
    const int split = kn.split_k > 1 ? kn.split_k : 1;
    // batch 1 with every expert on the GEMV kernels: the combine is folded
    // into the down projection (one launch fewer, no y workspace traffic)
    const bool fuse = kn.fused_combine && B == 1 && run_gemv && !run_mfma &&
                      down_combine_supported(wdt, cfg.inter, k);
    // batch 1 on the GEMV kernels with the GEMV router: the gate/up kernel
    // selects the experts itself (one launch fewer)
    const bool select_in_gate_up = kn.fused_select && B == 1 && run_gemv && !run_mfma &&
                                   kn.router != ROUTER_MFMA && gate_up_select_supported(E, k);

    hipEvent_t* ev = nullptr;  // this forward's event set, when timing
    if (c && c->timing) {
        collect_timing(c, kTimingRing - 1);  // waits only if the ring is full
        ev = c->ev[c->ring_head];
        e = hipEventRecord(ev[0], s);
        if (e != hipSuccess) return hip_fail("timing event", e);
    }

    RouterArgs ra;
    memset(&ra, 0, sizeof ra);
    ra.x = x->data;
    ra.x_stride = x->row_stride;
    ra.B = B;
    ra.H = cfg.hidden;
    ra.E = E;
    ra.k = k;
    ra.score_fn = tk->score_fn;
    ra.wr = (const float*)router_w->data;
    ra.wr_stride = router_w->row_stride;
    ra.bias = tk->bias;
    ra.logits = ws.logits;
    ra.router_mode = kn.router;
    ra.rows_per_stage = router_rows_per_stage(cfg.hidden, act, B);
    ra.topk_idx = ws.topk_idx;
    ra.topk_w = ws.topk_w;
    ra.user_idx = tk->idx_out;
    ra.user_w = tk->weight_out;
    ra.plan = ws.plan;
    ra.path_mode = path;
    ra.mfma_min_rows = kn.mfma_min_rows;
    ra.mfma_ok = mfma_ok;
    ra.logits_only = select_in_gate_up && !link.logits_ready;
    ra.logits_ready = link.logits_ready;
    // cache warm-up on the side stream: by default started once this layer's
    // router and top-k are queued (for the next layer's weights: it then does
    // not compete with this layer's own router read), or with the forward's
    // first launch (for weights this layer reads after its routing, such as
    // its most often selected experts); joined back at the end of this
    // forward, so the caller may release the ranges once its own stream has
    // been synchronised
    const bool prefetch = c && c->pf_n > 0;
    auto fork_prefetch = [&]() -> hipError_t {
        hipError_t r = hipEventRecord(c->ev_fork, s);
        if (r == hipSuccess) r = hipStreamWaitEvent(c->side, c->ev_fork, 0);
        if (r == hipSuccess)
            r = launch_prefetch(c->pf_ptr, c->pf_bytes, c->pf_n, c->sink, c->pf_grid, c->side);
        if (r == hipSuccess) r = hipEventRecord(c->ev_join, c->side);
        return r;
    };
    if (prefetch && c->pf_start == 1) {
        e = fork_prefetch();
        if (e != hipSuccess) return hip_fail("prefetch launch", e);
    }
    int router_kernel = 0, launches = prefetch ? 1 : 0;
    int router_launches = 0;
    e = launch_router(ra, act, s, &router_kernel, &router_launches);
    if (e != hipSuccess) return hip_fail("router launch", e);
    launches += router_launches;
    if (ev && (e = hipEventRecord(ev[1], s)) != hipSuccess) return hip_fail("timing event", e);
    if (prefetch && c->pf_start == 0) {
        e = fork_prefetch();
        if (e != hipSuccess) return hip_fail("prefetch launch", e);
    }

    ExpertArgs ea;
    memset(&ea, 0, sizeof ea);
    ea.x = x->data;
    ea.x_stride = x->row_stride;
    ea.k = k;
    ea.H = cfg.hidden;
    ea.I = cfg.inter;
    ea.w_gate_up = ex->w_gate_up;
    ea.w_down = ex->w_down;
    ea.s_gu = ex->scale_gate_up;
    ea.s_d = ex->scale_down;
    ea.plan = ws.plan;
    ea.h = ws.h;
    ea.y = ws.y;
    ea.partial = ws.partial;
    ea.slot_cap = ws.slot_cap;
    ea.split_k = split;
    ea.out = out->data;
    ea.topk_idx = ws.topk_idx;
    ea.topk_w = ws.topk_w;

    // at most B * k / mfma_rows experts reach the MFMA kernels
    const int mfma_experts =
        path == PATH_AUTO ? (max_experts < slots / mfma_rows ? max_experts : slots / mfma_rows)
                          : max_experts;
    // GEMV-served experts, then MFMA-served ones, stage by stage (running the
    // two kinds concurrently on two streams was measured and gained nothing:
    // both are bound by the same HBM bandwidth)
    SelectArgs sa;
    sa.logits = ws.logits;
    sa.bias = tk->bias;
    sa.E = E;
    sa.score_fn = tk->score_fn;
    sa.topk_idx = ws.topk_idx;
    sa.topk_w = ws.topk_w;
    sa.user_idx = tk->idx_out;
    sa.user_w = tk->weight_out;
    sa.plan = ws.plan;
    for (int stage = 0; stage < 2; ++stage) {
        if (run_gemv) {
            e = stage == 0 ? (select_in_gate_up
                                  ? launch_gate_up_select1(ea, sa, act, wdt, 0, s)
                                  : launch_gate_up_gemv(ea, act, wdt, gemv_rows, max_experts, s))
                : fuse     ? launch_down_combine(ea, act, wdt, s)
                           : launch_down_gemv(ea, act, wdt, gemv_rows, max_experts, s);
            if (e != hipSuccess)
                return hip_fail(stage == 0 ? "gate/up GEMV launch" : "down GEMV launch", e);
            launches += 1;
        }
        if (run_mfma) {
            e = stage == 0 ? launch_gate_up_mfma(ea, wdt, B, mfma_experts, s)
                           : launch_down_mfma(ea, wdt, B, mfma_experts, s);
            if (e != hipSuccess)
                return hip_fail(stage == 0 ? "gate/up MFMA launch" : "down MFMA launch", e);
            launches += split > 1 ? 2 : 1;  // the split-K sums are added by a second kernel
        }
        if (ev && (e = hipEventRecord(ev[2 + stage], s)) != hipSuccess)
            return hip_fail("timing event", e);
    }

    CombineArgs ca;
    ca.x = x->data;
    ca.x_stride = x->row_stride;
    ca.out = out->data;
    ca.out_stride = out->row_stride;
    ca.B = B;
    ca.H = cfg.hidden;
    ca.k = k;
    ca.topk_w = ws.topk_w;
    ca.y = ws.y;
    if (link.next_router_w) {
        // this layer's combine + residual in the next layer's router launch
        RouterArgs rn;
        memset(&rn, 0, sizeof rn);
        rn.x = x->data;
        rn.x_stride = x->row_stride;
        rn.B = B;
        rn.H = cfg.hidden;
        rn.E = E;
        rn.wr = (const float*)link.next_router_w->data;
        rn.wr_stride = link.next_router_w->row_stride;
        rn.logits = ws.logits;
        rn.comb_y = ws.y;
        rn.comb_w = ws.topk_w;
        rn.comb_k = k;
        rn.comb_out = out->data;
        rn.comb_out_stride = out->row_stride;
        e = launch_combine_router(rn, act, s, link.next_splits);
        if (e != hipSuccess) return hip_fail("combine + next router launch", e);
        launches += 1;
    } else if (!fuse) {
        e = launch_combine(ca, act, s);
        if (e != hipSuccess) return hip_fail("combine launch", e);
        launches += 1;
    }
    if (prefetch) {
        e = hipStreamWaitEvent(s, c->ev_join, 0);
        if (e != hipSuccess) return hip_fail("prefetch join", e);
    }
    if (ev) {
        e = hipEventRecord(ev[4], s);
        if (e != hipSuccess) return hip_fail("timing event", e);
        c->ring_head = (c->ring_head + 1) % kTimingRing;
        c->ring_pending += 1;
    }
    if (router_out) *router_out = router_kernel;
    if (launches_out) *launches_out = launches;
    return ok();
}

}  // namespace

extern "C" moe_status moe_decode_forward_ctx(moe_context* c, const moe_mat* x,
                                             const moe_mat* router_w, const moe_experts* ex,
                                             const moe_topk* tk, moe_mat* out) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_decode_forward: no context");
    moe_status st = validate(c->cfg, x, router_w, ex, tk, out);
    if (st != MOE_OK) return st;
    DeviceGuard g(c->device);
    if (g.status != hipSuccess) return hip_fail("moe_decode_forward: hipSetDevice", g.status);
    const Workspace ws = {c->logits, c->topk_idx, c->topk_w, c->plan,
                          c->h,      c->y,        c->partial, c->slot_cap};
    const Knobs kn = {c->path, c->mfma_min_rows, c->split_k, c->router, c->fused_combine,
                      c->fused_select};
    return launch_layer(c->cfg, kn, ws, c->stream, x, router_w, ex, tk, out, c, &c->last_router,
                        &c->last_launches);
}

namespace {
constexpr int kMaxStackLayers = 256;
}

extern "C" moe_status moe_decode_forward_stack(moe_context* c, const moe_mat* x,
                                               int32_t n_layers, const moe_mat* router_w,
                                               const moe_experts* ex, const moe_topk* tk,
                                               moe_mat* out) {
    if (!c) return fail(MOE_ERR_NO_CONTEXT, "moe_decode_forward_stack: no context");
    if (n_layers < 1 || n_layers > kMaxStackLayers)
        return fail(MOE_ERR_INVALID_ARG, "moe_decode_forward_stack: n_layers %d outside 1..%d",
                    n_layers, kMaxStackLayers);
    if (!router_w || !ex || !tk || !out)
        return fail(MOE_ERR_INVALID_ARG, "moe_decode_forward_stack: a layer array is NULL");
    // every layer is checked before any work is queued
    for (int l = 0; l < n_layers; ++l) {
        const moe_mat* xin = l == 0 ? x : &out[l - 1];
        moe_status st = validate(c->cfg, xin, &router_w[l], &ex[l], &tk[l], &out[l]);
        if (st != MOE_OK) {
            const std::string msg = g_error;
            return fail(st, "layer %d: %s", l, msg.c_str());
        }
    }
    DeviceGuard g(c->device);
    if (g.status != hipSuccess) return hip_fail("moe_decode_forward_stack: hipSetDevice", g.status);
    const Workspace ws = {c->logits, c->topk_idx, c->topk_w, c->plan,
                          c->h,      c->y,        c->partial, c->slot_cap};
    const Knobs kn = {c->path, c->mfma_min_rows, c->split_k, c->router, c->fused_combine,
                      c->fused_select};
    const moe_config& cfg = c->cfg;
    const int B = x->rows;
    int ready = 0;
    for (int l = 0; l < n_layers; ++l) {
        const moe_mat* xin = l == 0 ? x : &out[l - 1];
        // the combine can compute the next layer's logits when that layer
        // would take the matrix-core router, the batch fits one row tile, the
        // combine is not folded into the down projection (batches of two
        // rows and more) and the output does not overlap the input (the
        // kernel's workgroups read the input while some write the output)
        uintptr_t xl, xh, ol, oh;
        mat_range(xin, &xl, &xh);
        mat_range(&out[l], &ol, &oh);
        const bool fuse_next = c->fused_next_router && l + 1 < n_layers && B >= 2 &&
                               router_uses_mfma(kn.router, B, cfg.num_experts, cfg.hidden) &&
                               combine_router_supported(cfg.num_experts, cfg.hidden, B) &&
                               !(ol < xh && xl < oh);
        int splits = 0;
        const StackLink link = {ready, fuse_next ? &router_w[l + 1] : nullptr, &splits};
        moe_status st = launch_layer(cfg, kn, ws, c->stream, xin, &router_w[l], &ex[l], &tk[l],
                                     &out[l], c, &c->last_router, &c->last_launches, link);
        if (st != MOE_OK) return st;
        ready = fuse_next ? splits : 0;
    }
    return ok();
}

extern "C" moe_status moe_decode_forward(const moe_mat* x, const moe_mat* router_w,
                                         const moe_experts* ex, const moe_topk* tk,
                                         moe_mat* out) {
    if (!g_bound)
        return fail(MOE_ERR_NO_CONTEXT, "moe_decode_forward: no context bound on this thread");
    return moe_decode_forward_ctx(g_bound, x, router_w, ex, tk, out);
}

// ------------------------------------------------ forward without allocation

namespace {

// The workspace of moe_decode_forward_noalloc: a file-scope device array.
// Every GPU the library runs on holds its own copy, at its own address, until
// the process ends.  40 MiB holds the full decode layer (hidden 7168, 896
// experts, top 16, intermediate 2048, bf16 activations) at every batch up to
// 64 rows (35.4 MB at 64 rows).  On the host, `scratch` only names the
// symbol: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is passed to kernels.
constexpr size_t kScratchBytes = size_t(40) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of scratch, per device

// The device address of scratch on device dev (which must be current),
// looked up on the first call there.
hipError_t scratch_address(int dev, void** ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" moe_status moe_decode_forward_noalloc(const moe_mat* x, const moe_mat* router_w,
                                                 const moe_experts* ex, const moe_topk* tk,
                                                 moe_mat* out, void* hip_stream) {
    if (!x || !ex || !tk)
        return fail(MOE_ERR_INVALID_ARG, "moe_decode_forward_noalloc: x, expert_w or topk is NULL");
    // the configuration this call describes, checked as a context's would be
    moe_config cfg;
    cfg.num_experts = ex->num_experts;
    cfg.hidden = ex->hidden;
    cfg.inter = ex->inter;
    cfg.weight_dtype = ex->dtype;
    cfg.act_dtype = x->dtype;
    cfg.max_batch = x->rows;
    cfg.max_topk = tk->k;
    moe_status st = moe_check_config(&cfg);
    if (st != MOE_OK) return st;
    st = validate(cfg, x, router_w, ex, tk, out);
    if (st != MOE_OK) return st;
    const WsLayout lay =
        ws_layout(x->rows, tk->k, cfg.num_experts, cfg.hidden, cfg.inter, cfg.act_dtype);
    if (lay.total > kScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED,
                    "moe_decode_forward_noalloc: %d rows x top-%d of this layer need %zu bytes "
                    "of workspace, more than its fixed %zu-byte scratch array; use a context "
                    "(moe_context_create) for this request",
                    x->rows, tk->k, lay.total, kScratchBytes);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("moe_decode_forward_noalloc: hipGetDevice", e);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_UNSUPPORTED, "moe_decode_forward_noalloc: device %d beyond %d", dev,
                    kMaxDevices);
    void* base = nullptr;
    e = scratch_address(dev, &base);
    if (e != hipSuccess) return hip_fail("moe_decode_forward_noalloc: hipGetSymbolAddress", e);
    char* b = (char*)base;
    const Workspace ws = {(double*)(b + lay.logits), (int*)(b + lay.topk_idx),
                          (float*)(b + lay.topk_w),  (DevPlan*)(b + lay.plan),
                          b + lay.h,                 (float*)(b + lay.y),
                          nullptr,                   x->rows * tk->k};
    // the defaults of a new context: AUTO expert kernels (every expert on MFMA
    // from two rows), AUTO router, combine folded in at batch 1, top-k its own
    // launch, no split-K
    const Knobs kn = {PATH_AUTO, 1, 0, ROUTER_AUTO, 1, 0};
    return launch_layer(cfg, kn, ws, (hipStream_t)hip_stream, x, router_w, ex, tk, out, nullptr,
                        nullptr, nullptr);
}
