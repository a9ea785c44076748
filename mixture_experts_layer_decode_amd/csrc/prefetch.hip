// prefetch.hip -- side-stream cache warm-up of the next layer's weights.
//
// ailookout.news, "vLLM speeds up Kimi K3 up to 1.9x on NVIDIA GB300 with
// agent-assisted kernels", section "How the specialised decode path works":
// during the GPUs' waits for each other, an extra kernel pulls the following
// layer's weights into the caches, since decoding for one user is bound by
// weight reads from memory.
//
// The kernel reads every 16-byte vector of the registered ranges once (plain
// loads, so the lines are allocated in L2 and the MALL) and folds them into a
// value that is stored only if it equals a sentinel the host picked, so the
// loads cannot be removed.  It has no data dependence on the forward: it is a
// cache hint only.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRanges = 8;

struct PrefetchArgs {
    const u32x4* ptr[kMaxRanges];
    int64_t n16[kMaxRanges];  // 16-byte vectors in each range
    int n;
    uint32_t sentinel;
    uint32_t* sink;
};

__global__ __launch_bounds__(kThreads) void prefetch_kernel(PrefetchArgs p) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int r = 0; r < p.n; ++r) {
        const u32x4* base = p.ptr[r];
        const int64_t n = p.n16[r];
        int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
        // four independent loads in flight per thread
        for (; i + 3 * stride < n; i += 4 * stride) {
            const u32x4 a = base[i], b = base[i + stride];
            const u32x4 c = base[i + 2 * stride], d = base[i + 3 * stride];
            acc ^= a.x ^ b.y ^ c.z ^ d.w;
        }
        for (; i < n; i += stride) acc ^= base[i].x;
    }
    if (acc == p.sentinel) p.sink[threadIdx.x] = acc;
}

}  // namespace

// ptrs / bytes: host arrays of n <= 8 device ranges (16-byte aligned; a
// trailing partial vector is not read).  sink: device scratch of >= 256
// uint32.  grid: workgroups to use (a small grid leaves the main stream most
// of the machine).
hipError_t launch_prefetch(const void* const* ptrs, const int64_t* bytes, int n, uint32_t* sink,
                           int grid, hipStream_t s) {
    PrefetchArgs a;
    a.n = n < kMaxRanges ? n : kMaxRanges;
    for (int i = 0; i < kMaxRanges; ++i) {
        a.ptr[i] = i < a.n ? (const u32x4*)ptrs[i] : nullptr;
        a.n16[i] = i < a.n ? bytes[i] / 16 : 0;
    }
    a.sentinel = 0x9e3779b9u;
    a.sink = sink;
    prefetch_kernel<<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
