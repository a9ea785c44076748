/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) decode-step Mixture-of-Experts
 * layer library, libmoe_decode.so.
 *
 * The operation (ailookout.news, "vLLM speeds up Kimi K3 up to 1.9x on NVIDIA
 * GB300 with agent-assisted kernels", section "How the specialised decode
 * path works"): every token of a decode batch is routed to k of E experts
 * (16 of 896 for Kimi K3), the selected expert FFNs run, and their outputs are
 * combined.  The pages do not write the arithmetic out; this library computes,
 * per row b of x:
 *
 *   s[e]   = sum_h x[b,h] * Wr[e,h] + bias[e]              (router logits)
 *   T      = the k largest s[e], ties to the lower index,   (selection)
 *            in descending order
 *   w[j]   = sigmoid(s[T_j]) / sum sigmoid(s[T])            (MOE_SCORE_SIGMOID)
 *          | exp(s[T_j]) / sum exp(s[T])                    (MOE_SCORE_SOFTMAX)
 *   h      = round_act( silu(sg .* (Wg x)) .* (su .* (Wu x)) )  per expert
 *   y      = sd .* (Wd h)
 *   out[b] = x[b] + sum_j w[j] * y_j                        (rounded once)
 *
 * Accumulation is fp32 for the expert and combine stages and fp64 for the
 * router logits, so that the discrete expert choice is taken essentially
 * exactly.  sg, su, sd are per-output-row fp32 scales of fp8 weights (1 for
 * other types).
 *
 * The path is for decode only: batches of 1 to 64 rows (spectrumweb.co, "vLLM
 * and NVIDIA use coding agents to nearly double Kimi K3 decode speed, then
 * rethink how to review it": decode batches up to 64).  Requests outside what the library supports are refused
 * with MOE_ERR_UNSUPPORTED before any work is queued, so the caller can take
 * its general path instead (upstreambeat.com, "vLLM tests a fast-track review
 * model with Kimi K3's specialized decode path", section "Why the review model
 * matters": unsupported configurations are rejected at startup and
 * unsupported requests fall back to the stock path).
 *
 * Conventions for every entry point:
 *  - Device pointers are HIP device memory on the context's device; host
 *    pointers are named as such.  All matrices are row-major.
 *  - The caller owns every tensor it passes (x, weights, scales, bias, out,
 *    optional index/weight outputs).  A context owns only its workspace, which
 *    it allocates once in moe_context_create (plus the split-K partial sums,
 *    allocated by moe_context_set_path); moe_decode_forward* allocates
 *    nothing.
 *  - Work is queued on the context's HIP stream and the call returns without
 *    waiting; results are valid once that stream has been synchronised.
 *  - Errors are status codes.  Every argument check runs before anything is
 *    queued, so outputs are untouched when a call fails.  moe_last_error()
 *    describes the last failure on the calling thread.  A failed kernel
 *    launch or HIP runtime call is reported as MOE_ERR_DEVICE.
 *  - Calls that share one context must not run concurrently from several host
 *    threads; contexts are independent of each other.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* null pointer, misalignment, bad overlap, bad enum */
    MOE_ERR_UNSUPPORTED = -2, /* valid request this path does not serve: fall back */
    MOE_ERR_DEVICE = -3,      /* HIP runtime or kernel failure */
    MOE_ERR_NO_CONTEXT = -4   /* moe_decode_forward with no bound context */
} moe_status;

typedef enum {
    MOE_F32 = 0,
    MOE_BF16 = 1,
    MOE_FP8_E4M3 = 2 /* OCP e4m3: bias 7, max 448, S.1111.111 = NaN */
} moe_dtype;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

/* Which expert kernel serves an active expert (see moe_context_set_path). */
typedef enum {
    MOE_PATH_AUTO = 0, /* B == 1: GEMV; else rows >= mfma_min_rows -> MFMA, else GEMV */
    MOE_PATH_GEMV = 1, /* every expert on the weight-streaming GEMV kernels */
    MOE_PATH_MFMA = 2  /* every expert on the split-K MFMA kernels (bf16/fp8) */
} moe_path;

/* Which kernel computes the router logits (see moe_context_set_router). */
typedef enum {
    MOE_ROUTER_AUTO = 0, /* one or two rows: GEMV; three rows or more: matrix cores */
    MOE_ROUTER_GEMV = 1, /* vector-unit GEMV, fp64 accumulation */
    MOE_ROUTER_MFMA = 2  /* fp64 matrix cores (v_mfma_f64_16x16x4_f64) */
} moe_router_kernel;

/* Stages reported by moe_context_get_timing. */
typedef enum {
    MOE_STAGE_ROUTER = 0,  /* router GEMV, then top-k + weights + bucketing */
    MOE_STAGE_GATE_UP = 1, /* gate/up projections + SwiGLU (GEMV and MFMA kernels) */
    MOE_STAGE_DOWN = 2,    /* down projection (GEMV and MFMA kernels) */
    MOE_STAGE_COMBINE = 3, /* weighted combine + residual (empty when folded into down) */
    MOE_STAGE_COUNT = 4
} moe_stage;

/* A row-major matrix in device memory.  row_stride is in elements, >= cols. */
typedef struct {
    void* data;
    int32_t dtype; /* moe_dtype */
    int32_t rows;
    int32_t cols;
    int64_t row_stride;
} moe_mat;

/* The expert weights of one layer, contiguous, in device memory:
 *   w_gate_up [E][2I][H]: rows 0..I-1 of each expert are the gate projection,
 *                         rows I..2I-1 the up projection;
 *   w_down    [E][H][I];
 *   scale_gate_up [E][2I], scale_down [E][H]: fp32 per-output-row scales,
 *                         required for MOE_FP8_E4M3, must be NULL otherwise. */
typedef struct {
    int32_t num_experts; /* E */
    int32_t hidden;      /* H */
    int32_t inter;       /* I */
    int32_t dtype;       /* moe_dtype of both weight tensors */
    const void* w_gate_up;
    const void* w_down;
    const float* scale_gate_up;
    const float* scale_down;
} moe_experts;

/* Routing parameters and optional routing outputs (device memory). */
typedef struct {
    int32_t k;          /* experts per token, 1 <= k <= max_topk */
    int32_t score_fn;   /* moe_score_fn */
    const float* bias;  /* [E] fp32 added to the logits, or NULL */
    int32_t* idx_out;   /* [B][k] selected experts in descending logit order, or NULL */
    float* weight_out;  /* [B][k] renormalised weights, or NULL */
} moe_topk;

/* What a context is built for.  Checked once, at creation. */
typedef struct {
    int32_t num_experts;  /* E: 1..2048 */
    int32_t hidden;       /* H: multiple of 512 (fp8 weights: of 1024), 512..8192 */
    int32_t inter;        /* I: multiple of 256 (bf16: 512, fp8: 1024), <= 8192 */
    int32_t weight_dtype; /* MOE_F32 (with MOE_F32 activations), MOE_BF16 or
                             MOE_FP8_E4M3 (both with MOE_BF16 activations) */
    int32_t act_dtype;    /* dtype of x and out */
    int32_t max_batch;    /* 1..64 */
    int32_t max_topk;     /* 1..min(E, 32) */
} moe_config;

typedef struct moe_context moe_context;

/* Host-only check that cfg is a configuration this library serves
 * (upstreambeat.com, "vLLM tests a fast-track review model with Kimi K3's
 * specialized decode path", section "Why the review model matters":
 * unsupported configurations are rejected at startup).  Makes no HIP call
 * (usable at startup, before any device work).  Returns MOE_OK,
 * MOE_ERR_INVALID_ARG (cfg NULL or a bad enum) or MOE_ERR_UNSUPPORTED. */
moe_status moe_check_config(const moe_config* cfg);

/* No passage defines this call: it is plumbing (device memory and streams).
 * Create a context on the current HIP device.  hip_stream is a hipStream_t
 * (NULL = the null stream).  Allocates the workspace once for
 * cfg->max_batch and cfg->max_topk, and binds the new context to the calling
 * thread (see moe_context_bind).  *out receives the context (host pointer,
 * released with moe_context_destroy). */
moe_status moe_context_create(const moe_config* cfg, void* hip_stream, moe_context** out);

/* No passage defines this call: it is plumbing.  Queue later work on another
 * hipStream_t of the same device.  The switch is ordered: every later launch
 * of the context runs after all work already queued on the previous stream
 * (an event recorded there and waited on by the new stream), so forwards of
 * one context never overlap on the device, and moe_context_destroy /
 * moe_context_set_path, which synchronise the current stream, also wait for
 * the work of earlier streams.  Returns MOE_ERR_DEVICE if the event calls
 * fail (the stream is then unchanged). */
moe_status moe_context_set_stream(moe_context* ctx, void* hip_stream);

/* Choose the expert kernels (ailookout.news, "vLLM speeds up Kimi K3 up to
 * 1.9x on NVIDIA GB300 with agent-assisted kernels", section "How the
 * specialised decode path works": the GB300 path picks its kernels from the
 * batch size, GEMV-style kernels for one- and two-row batches and split-K
 * ones for larger batches; on MI355X the matrix-core kernels already match
 * the GEMV ones at two rows).  path: MOE_PATH_AUTO (the default) runs every
 * expert on the GEMV kernels when the batch has one row; above that it
 * sends an expert to the MFMA kernels when at least mfma_min_rows rows are
 * routed to it (1..64; 0 keeps the current value, initially 1, i.e. every
 * expert), else to the GEMV kernels; MOE_PATH_GEMV / MOE_PATH_MFMA force one
 * kind.  fp32 weights always use
 * GEMV.  split_k: K splits of the MFMA kernels (0 or 1: none; up to 16); the
 * split partial sums are added in a fixed order, so results are reproducible.
 * A split_k above 1 may allocate a partial-sum buffer of
 * split_k * max_batch * max_topk * max(2 * inter, hidden) * 4 bytes; this call
 * then first waits for the work queued on the context stream.  Returns
 * MOE_ERR_INVALID_ARG for values out of range, MOE_ERR_DEVICE if that
 * allocation fails (the previous settings are kept). */
moe_status moe_context_set_path(moe_context* ctx, int32_t path, int32_t mfma_min_rows,
                                int32_t split_k);

/* Choose the router kernel (ailookout.news, "vLLM speeds up Kimi K3 up to
 * 1.9x on NVIDIA GB300 with agent-assisted kernels", section "How the
 * specialised decode path works": each token's router scores pick 16 of 896
 * experts).  Both kernels compute every logit as an fp64 sum of exact fp64
 * products, in different orders, so they select the same experts except
 * between logits that differ by a few fp64 ulps; the GEMV kernel streams the
 * router once per forward with its per-row cost on the vector units, the
 * matrix-core kernel moves that per-row cost to the fp64 MFMA units.  kernel:
 * a moe_router_kernel (initially MOE_ROUTER_AUTO).  Takes effect from the
 * next forward.  Returns MOE_ERR_INVALID_ARG for other values. */
moe_status moe_context_set_router(moe_context* ctx, int32_t kernel);

/* Fold the combine + residual into the down projection when a forward has
 * one row and every expert on the GEMV kernels (ailookout.news, "vLLM speeds
 * up Kimi K3 up to 1.9x on NVIDIA GB300 with agent-assisted kernels", section
 * "How the specialised decode path works": the residual add is fused into
 * the epilogue of the kernel before it).  One workgroup then computes a few
 * output columns of all k experts and combines them in choice order with the
 * residual, bit for bit as the separate combine kernel would; it serves
 * k <= 16 with down rows of at most four 16-byte vectors per lane (inter <=
 * 2048 bf16, 4096 fp8, 1024 fp32), otherwise the separate kernels run.
 * enable != 0 turns it on (the initial setting), 0 off.  Takes effect from
 * the next forward. */
moe_status moe_context_set_fused_combine(moe_context* ctx, int32_t enable);

/* For moe_decode_forward_stack: fold each layer's combine + residual into the
 * next layer's router launch (ailookout.news, "vLLM speeds up Kimi K3 up to
 * 1.9x on NVIDIA GB300 with agent-assisted kernels", section "How the
 * specialised decode path works": the residual add is fused into a
 * neighbouring kernel's epilogue, and the specialised path cuts the kernels
 * per layer).  One kernel then computes layer l's output rows (the same fp32
 * operations in the same order as the separate combine kernel, so the same
 * bits), stores them, and takes them straight into layer l+1's router logits
 * on the fp64 matrix cores; layer l+1 starts at its top-k.  It applies when
 * layer l+1 would take the matrix-core router (MOE_ROUTER_AUTO from three
 * rows, or MOE_ROUTER_MFMA), the batch has 2 to 16 rows and layer l's output
 * does not overlap its input; other layers keep the separate launches.
 * enable != 0 turns it on, 0 off (the initial setting).  Takes effect from
 * the next stack. */
moe_status moe_context_set_fused_next_router(moe_context* ctx, int32_t enable);

/* Take the top-k selection inside the gate/up kernel when a forward has one
 * row, every expert on the GEMV kernels and the GEMV router (ailookout.news,
 * "vLLM speeds up Kimi K3 up to 1.9x on NVIDIA GB300 with agent-assisted
 * kernels", section "How the specialised decode path works": the
 * specialised path cuts the kernels per layer).  Every gate/up workgroup
 * then selects the k experts from the router's logits itself (the same
 * exact selection as the top-k kernel) and workgroup 0 writes the routing
 * outputs, so the top-k launch is saved; results are bit for bit those of
 * the separate kernels.  enable != 0 turns it on, 0 off (the initial
 * setting: on MI355X the k-fold selection costs the gate/up stage more than
 * the launch it saves).  Takes effect from the next forward. */
moe_status moe_context_set_fused_select(moe_context* ctx, int32_t enable);

/* Optional cache warm-up of the next layer's weights (ailookout.news, "vLLM
 * speeds up Kimi K3 up to 1.9x on NVIDIA GB300 with agent-assisted kernels",
 * section "How the specialised decode path works": there, an extra kernel
 * pulls the following layer's weights into the caches during other work).  From the next
 * forward on, each forward also reads the given device ranges once, on a side
 * stream of the context: the read starts once the forward's routing is done
 * (so it overlaps the expert weight stream, not the router read), has no data
 * dependence on the forward, and is joined back into the context stream at
 * the end of the forward.  ptrs/bytes are host arrays of n entries (n <= 8; n = 0 turns
 * the warm-up off); each range is 16-byte aligned (a trailing partial 16-byte
 * vector is not read).  The ranges must stay valid until the forwards that
 * read them have completed on the context stream.  The library keeps copies of
 * the pointers, not of the host arrays. */
moe_status moe_context_set_prefetch(moe_context* ctx, const void* const* ptrs,
                                    const int64_t* bytes, int32_t n);

/* When and how wide the cache warm-up of moe_context_set_prefetch runs
 * (same passage).  start 0 (the initial setting): once the forward's routing
 * kernels are queued, for ranges the next layer reads; start 1: with the
 * forward's first launch, concurrently with the router, for ranges this
 * forward reads after its routing (such as the experts that a router bias
 * makes the most often selected).  grid: workgroups of the warm-up kernel (0:
 * the initial 128; a small grid leaves most of the machine to the forward).
 * Returns MOE_ERR_INVALID_ARG for a start other than 0 or 1 or a grid
 * outside 0..65536.  Takes effect from the next forward. */
moe_status moe_context_set_prefetch_mode(moe_context* ctx, int32_t start, int32_t grid);

/* Measurement only; no passage defines these calls.
 * Per-stage GPU time.  With enable != 0, every forward records HIP events
 * between its stages on the context stream.  The events of up to 64 forwards
 * are kept and read back lazily, so timing does not make the host wait
 * between forwards (it waits only when 64 timed forwards are still queued).
 * moe_context_get_timing writes, to the host array ms[MOE_STAGE_COUNT], the
 * summed milliseconds of each stage over the timed forwards so far (waiting
 * for the queued ones), and to *count their number; reset != 0 clears the
 * sums afterwards.  A stage's time runs from the end of the previous stage's
 * last launch to the end of its own, so it includes launch gaps. */
moe_status moe_context_set_timing(moe_context* ctx, int32_t enable);
moe_status moe_context_get_timing(moe_context* ctx, double* ms, int64_t* count, int32_t reset);

/* Measurement only; no passage defines this call.
 * Counters of the last forward (synchronises the context stream).  Host
 * array out[6] = {distinct experts D, experts on the GEMV kernels, experts on
 * the MFMA kernels, most rows on one expert, kernels launched (the side-stream
 * prefetch included), router kernel (MOE_ROUTER_GEMV or MOE_ROUTER_MFMA)}. */
moe_status moe_context_last_plan(moe_context* ctx, int32_t* out);

/* No passage defines this call: it is plumbing.  Make ctx the context that
 * moe_decode_forward uses on the calling thread (NULL unbinds). */
moe_status moe_context_bind(moe_context* ctx);

/* The layer, as the header comment defines it, for the B = x->rows rows of x.
 *   x        [B][H] act_dtype
 *   router_w [E][H] MOE_F32
 *   expert_w the layer's experts (dims and dtype must match the context)
 *   topk     k, score function, optional bias and routing outputs
 *   out      [B][H] act_dtype; may be x itself (same data and stride), must
 *            not otherwise overlap x.
 * Uses the context bound to the calling thread. */
moe_status moe_decode_forward(const moe_mat* x, const moe_mat* router_w,
                              const moe_experts* expert_w, const moe_topk* topk,
                              moe_mat* out);

/* Same, with an explicit context. */
moe_status moe_decode_forward_ctx(moe_context* ctx, const moe_mat* x, const moe_mat* router_w,
                                  const moe_experts* expert_w, const moe_topk* topk,
                                  moe_mat* out);

/* n_layers consecutive layers on one batch (spectrumweb.co, "vLLM and NVIDIA
 * use coding agents to nearly double Kimi K3 decode speed, then rethink how
 * to review it": the decode step runs the model's layers one after another):
 * layer l runs as moe_decode_forward_ctx(ctx, l == 0 ? x : &out[l - 1],
 * &router_w[l], &expert_w[l], &topk[l], &out[l]).  router_w, expert_w, topk
 * and out are host arrays of n_layers (1..256) entries; every layer must fit
 * the context.  All layers are checked before any work is queued (a failure
 * names the layer).  With moe_context_set_fused_next_router on, consecutive
 * layers share a launch (see there); the results are the same bits either
 * way.  moe_context_last_plan then describes the last layer. */
moe_status moe_decode_forward_stack(moe_context* ctx, const moe_mat* x, int32_t n_layers,
                                    const moe_mat* router_w, const moe_experts* expert_w,
                                    const moe_topk* topk, moe_mat* out);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * layer as moe_decode_forward_ctx with a new context's defaults (AUTO expert
 * kernels and router, combine folded in at batch 1, no split-K, no prefetch,
 * no timing), queued on hip_stream (a hipStream_t of the current device;
 * NULL = the null stream), with no context and no allocation: its workspace
 * is a fixed 40 MiB file-scope device array that the library holds on each
 * GPU it runs on until the process ends.  Arguments as for
 * moe_decode_forward; the configuration they describe (E, H, I, weight type
 * from expert_w, activation type from x, B = x->rows, k = topk->k) must pass
 * moe_check_config.  A request whose workspace exceeds the array (the full
 * 7168 / 896 / top-16 / 2048 bf16 layer fits at every batch up to 64 rows) is
 * refused with MOE_ERR_UNSUPPORTED before any device work; so is every other
 * argument error, as for the other entry points.  Every call on one GPU
 * shares that GPU's array: calls on one GPU whose work overlaps on the device
 * (other streams, other host threads) race and give undefined results;
 * calls ordered on one stream are safe.  The array keeps the last call's
 * contents; no call depends on them. */
moe_status moe_decode_forward_noalloc(const moe_mat* x, const moe_mat* router_w,
                                      const moe_experts* expert_w, const moe_topk* topk,
                                      moe_mat* out, void* hip_stream);

/* No passage defines this call: it is plumbing.  Release the workspace and
 * streams (waits for queued work, also work queued before a stream switch).
 * Unbinds ctx from the calling thread.  NULL is a no-op. */
moe_status moe_context_destroy(moe_context* ctx);

/* No passage defines this call: it is plumbing.  Text of the last failure on
 * the calling thread ("" if none); never NULL. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
