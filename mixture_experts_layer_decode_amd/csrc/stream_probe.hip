// stream_probe.hip -- measurement only, not part of the layer: a plain
// streaming read of a device buffer, so that the weight-streaming kernels can
// be compared with what this card's HBM delivers to a kernel that does
// nothing else.  Built as its own library (libmoe_probe.so), loaded by the
// benchmark; see include/moe_probe.h.
//
// Workgroup g reads its own contiguous share of the buffer; each step its 256
// lanes issue 16 non-temporal 16-byte loads (64 KB, contiguous across the
// workgroup), and fold them into one word per lane.  Contiguous shares per
// workgroup read faster on this card than a grid-stride walk, which spreads
// every load instruction over the whole buffer.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/moe_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFlight = 16;  // 16-byte loads per lane per step
constexpr int64_t kStep16 = (int64_t)kThreads * kInFlight;  // 16-byte units per step

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* p, int64_t per16,
                                                               uint32_t* sink) {
    const u32x4* base = p + (int64_t)blockIdx.x * per16;
    uint32_t acc = 0;
    for (int64_t j = threadIdx.x; j < per16; j += kStep16) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(base + j + u * kThreads);
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // keeps the loads live; the store happens only for one folded value
    if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

}  // namespace

extern "C" int32_t moe_probe_stream_read(const void* buf, int64_t bytes, int32_t grid,
                                         void* hip_stream, uint32_t* sink) {
    if (!buf || !sink || grid < 1 || bytes <= 0) return -1;
    if ((uintptr_t)buf % 16) return -1;
    const int64_t unit = (int64_t)grid * kStep16 * 16;  // every workgroup, whole steps
    if (bytes % unit) return -1;
    const int64_t per16 = bytes / 16 / grid;
    stream_read_kernel<<<grid, kThreads, 0, (hipStream_t)hip_stream>>>((const u32x4*)buf, per16,
                                                                       sink);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
