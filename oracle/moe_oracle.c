/*
 * moe_oracle.c -- plain, slow, CPU reference of the decode-step
 * Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU path shares no
 * code, header, table or helper with it.
 *
 * What is computed (the method):
 *   ailookout.news, "vLLM speeds up Kimi K3 up to 1.9x on NVIDIA GB300 with
 *   agent-assisted kernels", section "How the specialised decode path works":
 *   every token activates 16 of 896 experts; the selected expert FFNs run and
 *   their results are combined.  The pages do not write the arithmetic out, so
 *   the plainest reading is used and every step below says which one:
 *     1. router logits  s[b,e] = sum_h x[b,h] * Wr[e,h]  (+ bias[e])
 *     2. selection: the k largest logits, ties to the lower expert index,
 *        listed in descending order
 *     3. weights: sigmoid of the selected logits divided by their sum, or
 *        softmax restricted to the selected logits
 *     4. expert FFN (SwiGLU, no biases):
 *          g = s_g * (Wg x), u = s_u * (Wu x), a = silu(g) * u,
 *          h = a rounded to the activation type, y = s_d * (Wd h)
 *     5. out[b] = x[b] + sum_j w[b,j] * y[b,j]   (unrounded)
 *
 * Every sum is accumulated in double precision, in ascending index order.
 * Inputs are decoded exactly from their stored bits (bf16, OCP fp8 e4m3,
 * fp32).  Work is split over independent outputs only (OpenMP), so results
 * are bit-identical at any thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3 = 2 };
enum { OR_SOFTMAX = 0, OR_SIGMOID = 1 };

/* ---------------------------------------------------------------- decode */

/* bf16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit e4m3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, largest finite 448, subnormals m*2^-9. */
double oracle_e4m3_value(uint8_t code) {
    int s = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

static double elem(const void* p, int dtype, int64_t i) {
    switch (dtype) {
    case OR_F32: return (double)((const float*)p)[i];
    case OR_BF16: return oracle_bf16_value(((const uint16_t*)p)[i]);
    default: return oracle_e4m3_value(((const uint8_t*)p)[i]);
    }
}

static size_t elem_size(int dtype) {
    return dtype == OR_F32 ? 4 : dtype == OR_BF16 ? 2 : 1;
}

/* Round a double straight to bf16 (8 significant bits), nearest-even, with
 * one rounding step (never through binary32, which would round twice).
 * Returns the bit pattern.  Finite inputs only. */
uint16_t oracle_round_bf16(double v) {
    double r;
    if (v == 0.0) {
        r = v;
    } else {
        int ex;
        double f = frexp(fabs(v), &ex);          /* |v| = f * 2^ex, f in [0.5,1) */
        if (ex - 1 >= -126) {
            r = ldexp(rint(ldexp(f, 8)), ex - 8); /* 8 significant bits */
        } else {
            r = ldexp(rint(ldexp(fabs(v), 133)), -133); /* subnormal spacing */
        }
        if (v < 0) r = -r;
    }
    float rf = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return (uint16_t)(u >> 16);
}

/* The activation-type rounding applied to h (step 4). */
static double round_act(double v, int act_dtype) {
    if (act_dtype == OR_BF16) return oracle_bf16_value(oracle_round_bf16(v));
    return (double)(float)v; /* binary32, nearest-even */
}

/* ---------------------------------------------------------------- router */

/* Step 1.  x: [B][x_stride] of x_dtype, wr: [E][H] fp32, bias: [E] or NULL.
 * logits: [B][E].  The bias is added after the dot product. */
void oracle_router_logits(const void* x, int x_dtype, int64_t x_stride, int B,
                          int H, const float* wr, int E, const float* bias,
                          double* logits) {
    int64_t n = (int64_t)B * E;
#pragma omp parallel for schedule(static)
    for (int64_t be = 0; be < n; ++be) {
        int b = (int)(be / E), e = (int)(be % E);
        double s = 0.0;
        for (int h = 0; h < H; ++h)
            s += elem(x, x_dtype, (int64_t)b * x_stride + h) * (double)wr[(int64_t)e * H + h];
        if (bias) s += (double)bias[e];
        logits[be] = s;
    }
}

/* Strict total order: a before b when its logit is larger, or equal with a
 * lower expert index. */
static int ranks_before(double sa, int a, double sb, int b) {
    return sa > sb || (sa == sb && a < b);
}

/* Step 3 for a given selection of every row: the renormalised weights of the
 * experts idx[b][0..k-1] (any k distinct experts, in any order).  Sigmoid:
 * p_j = 1 / (1 + exp(-s_j)), w_j = p_j / sum_j' p_j'.  Softmax restricted to
 * the selection: p_j = exp(s_j - m) with m the largest logit of the row (over
 * all E, so that no exp overflows), w_j = p_j / sum_j' p_j'.  Sums run in
 * selection order.  logits [B][E], idx [B][k] -> w [B][k]. */
void oracle_selection_weights(const double* logits, int B, int E, int k, int score_fn,
                              const int32_t* idx, double* w) {
    for (int b = 0; b < B; ++b) {
        const double* s = logits + (int64_t)b * E;
        const int32_t* ib = idx + (int64_t)b * k;
        double* wb = w + (int64_t)b * k;
        double total = 0.0;
        if (score_fn == OR_SIGMOID) {
            for (int j = 0; j < k; ++j) {
                wb[j] = 1.0 / (1.0 + exp(-s[ib[j]]));
                total += wb[j];
            }
        } else {
            double m = s[0];
            for (int e = 1; e < E; ++e)
                if (s[e] > m) m = s[e];
            for (int j = 0; j < k; ++j) {
                wb[j] = exp(s[ib[j]] - m);
                total += wb[j];
            }
        }
        for (int j = 0; j < k; ++j) wb[j] /= total;
    }
}

/* Steps 2 and 3 for every row.  logits [B][E] -> idx [B][k], w [B][k].
 * Selection is k passes, each taking the best expert not yet taken; the
 * weights are those of oracle_selection_weights for that selection. */
void oracle_topk(const double* logits, int B, int E, int k, int score_fn,
                 int32_t* idx, double* w) {
    char* taken = (char*)malloc((size_t)E);
    for (int b = 0; b < B; ++b) {
        const double* s = logits + (int64_t)b * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || ranks_before(s[e], e, s[best], best)))
                    best = e;
            taken[best] = 1;
            idx[(int64_t)b * k + j] = best;
        }
    }
    free(taken);
    oracle_selection_weights(logits, B, E, k, score_fn, idx, w);
}

/* ------------------------------------------------------------ expert FFN */

/* Step 4 for one token and one expert.
 * x_row: [H] of act_dtype.  wgu: this expert's [2I][H] (rows 0..I-1 gate,
 * rows I..2I-1 up), wd: [H][I], both w_dtype.  s_gu: [2I], s_d: [H] (per
 * output row scales, fp8 only; NULL means 1).  h_out: [I] or NULL.
 * y: [H]. */
void oracle_expert_ffn(const void* x_row, int act_dtype, int H, int I,
                       const void* wgu, const void* wd, int w_dtype,
                       const float* s_gu, const float* s_d, double* h_out,
                       double* y) {
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp parallel for schedule(static)
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; ++c) {
            double xv = elem(x_row, act_dtype, c);
            g += xv * elem(wgu, w_dtype, (int64_t)i * H + c);
            u += xv * elem(wgu, w_dtype, (int64_t)(I + i) * H + c);
        }
        if (s_gu) {
            g *= (double)s_gu[i];
            u *= (double)s_gu[I + i];
        }
        double a = g / (1.0 + exp(-g)) * u; /* silu(g) * u */
        h[i] = round_act(a, act_dtype);
    }
#pragma omp parallel for schedule(static)
    for (int n = 0; n < H; ++n) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i) acc += h[i] * elem(wd, w_dtype, (int64_t)n * I + i);
        if (s_d) acc *= (double)s_d[n];
        y[n] = acc;
    }
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)I);
    free(h);
}

/* --------------------------------------------------------------- combine */

/* Step 5.  x: [B][x_stride], w: [B][k], y: [B][k][H] -> out [B][H]. */
void oracle_combine(const void* x, int x_dtype, int64_t x_stride, int B, int H,
                    int k, const double* w, const double* y, double* out) {
    for (int b = 0; b < B; ++b)
        for (int n = 0; n < H; ++n) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += w[(int64_t)b * k + j] * y[((int64_t)b * k + j) * H + n];
            out[(int64_t)b * H + n] = elem(x, x_dtype, (int64_t)b * x_stride + n) + acc;
        }
}

/* ----------------------------------------------------------- whole layer */

/* Steps 1-5.  w_gate_up: [E][2I][H], w_down: [E][H][I]; scale_gate_up:
 * [E][2I], scale_down: [E][H] (NULL unless fp8).  Outputs: idx [B][k],
 * w [B][k], out [B][H].  Returns 0, or -1 when a size is out of range. */
int oracle_moe_forward(const void* x, int act_dtype, int B, int H,
                       const float* router_w, const float* bias, int E, int k,
                       int score_fn, const void* w_gate_up, const void* w_down,
                       int w_dtype, const float* scale_gate_up,
                       const float* scale_down, int I, int32_t* idx, double* w,
                       double* out) {
    if (B < 1 || H < 1 || E < 1 || I < 1 || k < 1 || k > E) return -1;
    double* logits = (double*)malloc(sizeof(double) * (size_t)B * E);
    double* y = (double*)malloc(sizeof(double) * (size_t)B * k * H);
    oracle_router_logits(x, act_dtype, H, B, H, router_w, E, bias, logits);
    oracle_topk(logits, B, E, k, score_fn, idx, w);
    size_t es = elem_size(w_dtype), ea = elem_size(act_dtype);
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < k; ++j) {
            int e = idx[(int64_t)b * k + j];
            const char* gu = (const char*)w_gate_up + (size_t)e * 2 * I * H * es;
            const char* dn = (const char*)w_down + (size_t)e * H * I * es;
            oracle_expert_ffn((const char*)x + (size_t)b * H * ea, act_dtype, H, I, gu, dn,
                              w_dtype, scale_gate_up ? scale_gate_up + (size_t)e * 2 * I : NULL,
                              scale_down ? scale_down + (size_t)e * H : NULL, NULL,
                              y + ((int64_t)b * k + j) * H);
        }
    oracle_combine(x, act_dtype, H, B, H, k, w, y, out);
    free(logits);
    free(y);
    return 0;
}

/* --------------------------------------------------------------- threads */

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
