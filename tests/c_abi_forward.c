/*
 * c_abi_forward.c -- the layer called from plain C through the C ABI of
 * libmoe_decode.so (include/moe_decode.h), with HIP device memory and no
 * Python or PyTorch, checked against the C oracle (test infrastructure:
 * oracle/moe_oracle.c, linked from libmoe_oracle.so).
 *
 * A small bf16 layer (E 32, H 512, I 512, top-8, sigmoid scores, bias), at
 * batch 1 (GEMV kernels, the combine folded into the down projection) and at
 * batch 4 (matrix-core kernels).  Acceptance as for every parity test:
 * expert indices equal the oracle's, or differ only in swaps of experts
 * whose oracle logits lie within 1e-6; routing weights within 1e-5; outputs
 * within 2e-2 max-abs and 5e-3 relative L2 of the oracle's unrounded ones.
 * Exit status 0 and a final line "c abi ok" on success.
 *
 * Built by __graft_entry__.build() into tests/_build/ (gcc, HIP runtime).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_decode.h"

/* the oracle's entry points (oracle/moe_oracle.c) */
int oracle_moe_forward(const void* x, int act_dtype, int B, int H, const float* router_w,
                       const float* bias, int E, int k, int score_fn, const void* w_gate_up,
                       const void* w_down, int w_dtype, const float* scale_gate_up,
                       const float* scale_down, int I, int32_t* idx, double* w, double* out);
void oracle_router_logits(const void* x, int x_dtype, int64_t x_stride, int B, int H,
                          const float* router_w, int E, const float* bias, double* logits);
double oracle_bf16_value(uint16_t bits);

enum { E = 32, H = 512, I = 512, K = 8, MAXB = 4 };
enum { ORACLE_BF16 = 1, ORACLE_SIGMOID = 1 };

#define HIP_OK(call)                                                            \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) {                                                 \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));   \
            exit(2);                                                            \
        }                                                                       \
    } while (0)

#define MOE_OK_(call)                                                           \
    do {                                                                        \
        moe_status s_ = (call);                                                 \
        if (s_ != MOE_OK) {                                                     \
            fprintf(stderr, "%s failed (%d): %s\n", #call, (int)s_,             \
                    moe_last_error());                                          \
            exit(3);                                                            \
        }                                                                       \
    } while (0)

/* splitmix64: a counter-based stream of 64-bit values */
static uint64_t mix(uint64_t z) {
    z += 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

/* uniform in [-a, a), from element i of stream s */
static double uniform(uint64_t s, uint64_t i, double a) {
    const double u = (double)(mix(s * 0x100000001b3ull + i) >> 11) / 9007199254740992.0;
    return (2.0 * u - 1.0) * a;
}

/* bf16 bits of an input value (through fp32, to nearest even; any bf16
 * value is a valid input, so the double rounding does not matter) */
static uint16_t bf16_bits(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void fill_bf16(uint16_t* p, size_t n, uint64_t s, double a) {
    for (size_t i = 0; i < n; ++i) p[i] = bf16_bits(uniform(s, i, a));
}

static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

/* one forward at batch B through moe_decode_forward_ctx; returns the number
 * of rows excused as near-tie swaps, or exits on a failed check */
static int check_batch(moe_context* ctx, int B, const uint16_t* x_h, const float* router_h,
                       const float* bias_h, const uint16_t* gu_h, const uint16_t* dn_h,
                       void* router_d, void* bias_d, void* gu_d, void* dn_d) {
    void* x_d = to_device(x_h, sizeof(uint16_t) * B * H);
    void* out_d = NULL;
    int32_t* idx_d = NULL;
    float* w_d = NULL;
    HIP_OK(hipMalloc(&out_d, sizeof(uint16_t) * B * H));
    HIP_OK(hipMalloc((void**)&idx_d, sizeof(int32_t) * B * K));
    HIP_OK(hipMalloc((void**)&w_d, sizeof(float) * B * K));

    moe_mat x = {x_d, MOE_BF16, B, H, H};
    moe_mat out = {out_d, MOE_BF16, B, H, H};
    moe_mat router = {router_d, MOE_F32, E, H, H};
    moe_experts ex = {E, H, I, MOE_BF16, gu_d, dn_d, NULL, NULL};
    moe_topk tk = {K, MOE_SCORE_SIGMOID, (const float*)bias_d, idx_d, w_d};
    MOE_OK_(moe_decode_forward_ctx(ctx, &x, &router, &ex, &tk, &out));
    HIP_OK(hipDeviceSynchronize());

    uint16_t* out_h = malloc(sizeof(uint16_t) * B * H);
    int32_t* idx_h = malloc(sizeof(int32_t) * B * K);
    float* w_h = malloc(sizeof(float) * B * K);
    HIP_OK(hipMemcpy(out_h, out_d, sizeof(uint16_t) * B * H, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(idx_h, idx_d, sizeof(int32_t) * B * K, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(w_h, w_d, sizeof(float) * B * K, hipMemcpyDeviceToHost));

    int32_t* idx_o = malloc(sizeof(int32_t) * B * K);
    double* w_o = malloc(sizeof(double) * B * K);
    double* out_o = malloc(sizeof(double) * B * H);
    double* logits = malloc(sizeof(double) * B * E);
    if (oracle_moe_forward(x_h, ORACLE_BF16, B, H, router_h, bias_h, E, K, ORACLE_SIGMOID,
                           gu_h, dn_h, ORACLE_BF16, NULL, NULL, I, idx_o, w_o, out_o) != 0) {
        fprintf(stderr, "oracle refused the sizes\n");
        exit(4);
    }
    oracle_router_logits(x_h, ORACLE_BF16, H, B, H, router_h, E, bias_h, logits);

    int excused = 0;
    double max_abs = 0.0, num = 0.0, den = 0.0;
    for (int b = 0; b < B; ++b) {
        int same = 1;
        for (int j = 0; j < K; ++j) same &= idx_h[b * K + j] == idx_o[b * K + j];
        if (!same) {
            /* every position where the lists differ must hold a pair of
             * experts whose oracle logits lie within 1e-6 */
            for (int j = 0; j < K; ++j) {
                const int g = idx_h[b * K + j], o = idx_o[b * K + j];
                if (g == o) continue;
                if (g < 0 || g >= E || fabs(logits[b * E + g] - logits[b * E + o]) >= 1e-6) {
                    fprintf(stderr, "batch %d row %d: expert %d where the oracle has %d\n", B,
                            b, g, o);
                    exit(5);
                }
            }
            ++excused;
            continue;  /* its weights and output follow another selection */
        }
        for (int j = 0; j < K; ++j)
            if (fabs((double)w_h[b * K + j] - w_o[b * K + j]) > 1e-5) {
                fprintf(stderr, "batch %d row %d: weight %d %.9g against %.9g\n", B, b, j,
                        (double)w_h[b * K + j], w_o[b * K + j]);
                exit(6);
            }
        for (int n = 0; n < H; ++n) {
            const double d = oracle_bf16_value(out_h[b * H + n]) - out_o[b * H + n];
            if (fabs(d) > max_abs) max_abs = fabs(d);
            num += d * d;
            den += out_o[b * H + n] * out_o[b * H + n];
        }
    }
    const double rel = den > 0.0 ? sqrt(num / den) : 0.0;
    printf("batch %d: rows excused %d, max_abs %.3e, rel_l2 %.3e\n", B, excused, max_abs, rel);
    if (max_abs > 2e-2 || rel > 5e-3) {
        fprintf(stderr, "batch %d: output outside 2e-2 / 5e-3\n", B);
        exit(7);
    }
    free(out_h), free(idx_h), free(w_h), free(idx_o), free(w_o), free(out_o), free(logits);
    HIP_OK(hipFree(x_d));
    HIP_OK(hipFree(out_d));
    HIP_OK(hipFree(idx_d));
    HIP_OK(hipFree(w_d));
    return excused;
}

int main(void) {
    setvbuf(stdout, NULL, _IONBF, 0);
    const size_t n_gu = (size_t)E * 2 * I * H, n_dn = (size_t)E * H * I;
    uint16_t* gu_h = malloc(sizeof(uint16_t) * n_gu);
    uint16_t* dn_h = malloc(sizeof(uint16_t) * n_dn);
    float* router_h = malloc(sizeof(float) * E * H);
    float bias_h[E];
    uint16_t x_h[MAXB * H];
    fill_bf16(gu_h, n_gu, 1, 0.04);
    fill_bf16(dn_h, n_dn, 2, 0.04);
    for (size_t i = 0; i < (size_t)E * H; ++i) router_h[i] = (float)uniform(3, i, 0.04);
    for (int e = 0; e < E; ++e) bias_h[e] = (float)uniform(4, e, 0.5);
    fill_bf16(x_h, (size_t)MAXB * H, 5, 1.7);

    moe_config cfg = {E, H, I, MOE_BF16, MOE_BF16, MAXB, K};
    MOE_OK_(moe_check_config(&cfg));
    moe_context* ctx = NULL;
    MOE_OK_(moe_context_create(&cfg, NULL, &ctx));
    void* router_d = to_device(router_h, sizeof(float) * E * H);
    void* bias_d = to_device(bias_h, sizeof(bias_h));
    void* gu_d = to_device(gu_h, sizeof(uint16_t) * n_gu);
    void* dn_d = to_device(dn_h, sizeof(uint16_t) * n_dn);

    check_batch(ctx, 1, x_h, router_h, bias_h, gu_h, dn_h, router_d, bias_d, gu_d, dn_d);
    check_batch(ctx, MAXB, x_h, router_h, bias_h, gu_h, dn_h, router_d, bias_d, gu_d, dn_d);

    /* a request the library does not serve is refused before any work */
    moe_mat x_bad = {NULL, MOE_BF16, 65, H, H};
    moe_mat o_bad = {NULL, MOE_BF16, 65, H, H};
    moe_mat r = {router_d, MOE_F32, E, H, H};
    moe_experts ex = {E, H, I, MOE_BF16, gu_d, dn_d, NULL, NULL};
    moe_topk tk = {K, MOE_SCORE_SIGMOID, NULL, NULL, NULL};
    if (moe_decode_forward_ctx(ctx, &x_bad, &r, &ex, &tk, &o_bad) == MOE_OK) {
        fprintf(stderr, "a 65-row request was accepted\n");
        return 8;
    }

    MOE_OK_(moe_context_destroy(ctx));
    HIP_OK(hipFree(router_d));
    HIP_OK(hipFree(bias_d));
    HIP_OK(hipFree(gu_d));
    HIP_OK(hipFree(dn_d));
    free(gu_h), free(dn_h), free(router_h);
    printf("c abi ok\n");
    return 0;
}
