// combine.hip -- weighted combine + residual epilogue.
//
// Combine (ailookout.news, "vLLM speeds up Kimi K3 up to 1.9x on NVIDIA GB300
// with agent-assisted kernels", section "How the specialised decode path
// works": the selected experts' results are combined):
//   out[b, n] = round_act( x[b, n] + sum_{j ascending} w[b, j] * y[b*k + j, n] )
// in fp32, one rounding at the end.  Each thread owns 4 consecutive columns of
// one row; the loads of y for up to 16 choices are issued together before any
// is used, so a thread waits for about one memory round trip per 16 choices.
// Workgroups of one wave spread a row over H / 256 CUs.
// All loads and the store are 16-byte (fp32) or 8-byte (bf16) per lane and
// coalesced.  out may alias x exactly: every element is read before it is
// written, by the same thread.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kThreads = 64;
constexpr int kBatchLoads = 16;

template <int ACT>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs p) {
    const int b = blockIdx.y;
    const int n0 = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (n0 >= p.H) return;
    const int64_t xi = (int64_t)b * p.x_stride + n0;
    float xv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) xv[t] = load_act<ACT>(p.x, xi + t);

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const float* yb = p.y + (int64_t)b * p.k * p.H + n0;
    const float* wb = p.topk_w + (int64_t)b * p.k;
    for (int j0 = 0; j0 < p.k; j0 += kBatchLoads) {
        f32x4 yv[kBatchLoads];
        float wv[kBatchLoads];
#pragma unroll
        for (int q = 0; q < kBatchLoads; ++q)
            if (j0 + q < p.k) {
                yv[q] = *(const f32x4*)(yb + (int64_t)(j0 + q) * p.H);
                wv[q] = wb[j0 + q];
            }
#pragma unroll
        for (int q = 0; q < kBatchLoads; ++q)
            if (j0 + q < p.k) {
                acc[0] = fmaf(wv[q], yv[q].x, acc[0]);
                acc[1] = fmaf(wv[q], yv[q].y, acc[1]);
                acc[2] = fmaf(wv[q], yv[q].z, acc[2]);
                acc[3] = fmaf(wv[q], yv[q].w, acc[3]);
            }
    }
    const int64_t oi = (int64_t)b * p.out_stride + n0;
#pragma unroll
    for (int t = 0; t < 4; ++t) store_act<ACT>(p.out, oi + t, xv[t] + acc[t]);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int act, hipStream_t s) {
    const dim3 grid((a.H / 4 + kThreads - 1) / kThreads, a.B);
    if (act == DT_F32) combine_kernel<DT_F32><<<grid, kThreads, 0, s>>>(a);
    else combine_kernel<DT_BF16><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
