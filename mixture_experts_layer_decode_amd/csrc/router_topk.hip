// router_topk.hip -- router GEMV, top-k selection, routing weights and
// token-to-expert bucketing, in one launch.
//
// ailookout.news, "vLLM speeds up Kimi K3 up to 1.9x on NVIDIA GB300 with
// agent-assisted kernels", section "How the specialised decode path works":
// each token activates 16 of 896 experts.  The router matrix is read once per
// forward (25.7 MB fp32 at 896 x 7168), so phase 1 is a bandwidth-bound
// GEMV; the selection and bucketing that follow are tiny and latency-bound,
// so the last workgroup to finish phase 1 does them instead of paying for more
// launches.
//
// Phase 1 (every workgroup): each wave owns one expert row of the router and
//   computes its logits against all B rows of x, in fp64 (bf16 x fp32 products
//   are exact in fp64, so the only error is the fp64 summation, ~1e-16).
// Phase 2 (last workgroup only, elected by an arrival counter): per row, k
//   rounds of a wave-wide argmax over (logit, expert) with ties to the lower
//   index; routing weights in fp64; then a bitonic sort of (expert, slot) keys
//   gives the expert buckets and the GEMV / MFMA work lists.
//
// Cross-workgroup hand-off: each workgroup's logit stores are released with a
// device-scope fence before its arrival increment, and the last workgroup
// issues a device-scope fence after observing the final count and before it
// reads any logit.  Logits are read with ordinary loads (never the
// non-temporal or read-only variants used for weights), so no read can be
// moved above the fence.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 512;      // router columns per wave-step (8 per lane)
constexpr int kChunksInFlight = 7;
constexpr int kMaxPerLane = kMaxExperts / kWave;  // logits held per lane in top-k

// Load 8 activations x[i .. i+8) as fp32.
template <int ACT> __device__ __forceinline__ void load_act8(const void* x, int64_t i, float (&v)[8]);
template <> __device__ __forceinline__ void load_act8<DT_BF16>(const void* x, int64_t i,
                                                              float (&v)[8]) {
    u32x4 r = load16((const uint16_t*)x + i);
    v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x);
    v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
    v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z);
    v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
}
template <> __device__ __forceinline__ void load_act8<DT_F32>(const void* x, int64_t i,
                                                             float (&v)[8]) {
    f32x4 a = *(const f32x4*)((const float*)x + i);
    f32x4 b = *(const f32x4*)((const float*)x + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// (va, ea) ranks before (vb, eb): larger logit, or equal with lower index.
__device__ __forceinline__ bool ranks_before(double va, int ea, double vb, int eb) {
    return va > vb || (va == vb && ea < eb);
}

// Inclusive prefix sum of arr[0..n), n <= kMaxSlots, in place (all threads).
__device__ void block_inclusive_scan(int* arr, int n, int* s_wave) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    constexpr int kPer = kMaxSlots / kThreads;
    const int base = tid * kPer;
    int local[kPer];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (base + i < n) sum += arr[base + i];
        local[i] = sum;
    }
    int v = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    __syncthreads();  // every read of arr above happens before any write below
    if (lane == kWave - 1) s_wave[wave] = v;
    __syncthreads();
    int off = v - sum;
    for (int w = 0; w < wave; ++w) off += s_wave[w];
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (base + i < n) arr[base + i] = local[i] + off;
    __syncthreads();
}

// Ascending bitonic sort of keys[0..P), P a power of two <= kMaxSlots.
__device__ void block_bitonic_sort(int* keys, int P) {
    for (int size = 2; size <= P; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < P / 2; i += kThreads) {
                int pos = 2 * i - (i & (stride - 1));
                int partner = pos + stride;
                bool ascending = (pos & size) == 0;
                int a = keys[pos], b = keys[partner];
                if ((a > b) == ascending) {
                    keys[pos] = b;
                    keys[partner] = a;
                }
            }
            __syncthreads();
        }
}

template <int ACT, int BMAX>
__global__ __launch_bounds__(kThreads) void router_topk_kernel(RouterArgs p) {
    __shared__ int s_keys[kMaxSlots];
    __shared__ int s_scan[kMaxSlots];
    __shared__ int s_act_e[kMaxSlots];
    __shared__ int s_act_start[kMaxSlots];
    __shared__ int s_act_count[kMaxSlots];
    __shared__ int s_wave[kWaves];
    __shared__ int s_last;
    __shared__ int s_max_rows;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    // ---------------------------------------------------------- phase 1
    const int e = blockIdx.x * kWaves + wave;
    if (e < p.E) {
        double acc[BMAX];
#pragma unroll
        for (int b = 0; b < BMAX; ++b) acc[b] = 0.0;
        const float* row = p.wr + (int64_t)e * p.wr_stride;
        const int nc = p.H / kChunk;
        for (int c0 = 0; c0 < nc; c0 += kChunksInFlight) {
            u32x4 w0[kChunksInFlight], w1[kChunksInFlight];
#pragma unroll
            for (int c = 0; c < kChunksInFlight; ++c)
                if (c0 + c < nc) {
                    const float* q = row + (c0 + c) * kChunk + lane * 8;
                    w0[c] = load_weights16(q);
                    w1[c] = load_weights16(q + 4);
                }
#pragma unroll
            for (int c = 0; c < kChunksInFlight; ++c)
                if (c0 + c < nc) {
                    const int h = (c0 + c) * kChunk + lane * 8;
                    const float w[8] = {__uint_as_float(w0[c].x), __uint_as_float(w0[c].y),
                                        __uint_as_float(w0[c].z), __uint_as_float(w0[c].w),
                                        __uint_as_float(w1[c].x), __uint_as_float(w1[c].y),
                                        __uint_as_float(w1[c].z), __uint_as_float(w1[c].w)};
#pragma unroll
                    for (int b = 0; b < BMAX; ++b)
                        if (b < p.B) {
                            float xv[8];
                            load_act8<ACT>(p.x, (int64_t)b * p.x_stride + h, xv);
                            double s = acc[b];
#pragma unroll
                            for (int t = 0; t < 8; ++t) s = fma((double)xv[t], (double)w[t], s);
                            acc[b] = s;
                        }
                }
        }
        const double bias = p.bias ? (double)p.bias[e] : 0.0;
#pragma unroll
        for (int b = 0; b < BMAX; ++b)
            if (b < p.B) {
                double s = wave_sum(acc[b]);
                if (lane == 0) p.logits[(int64_t)b * p.E + e] = s + bias;
            }
    }

    // ------------------------------------------------- elect the last block
    __threadfence();  // release this block's logits (device scope)
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(p.counter, 1) == (int)gridDim.x - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();  // acquire: every block's logits are visible below
    if (threadIdx.x == 0) atomicExch(p.counter, 0);  // ready for the next launch

    // ------------------------------------------------------ phase 2: top-k
    const int k = p.k;
    const int n = p.B * k;
    for (int b = wave; b < p.B; b += kWaves) {
        double v[kMaxPerLane];
        uint32_t avail = 0;
        const double* lg = p.logits + (int64_t)b * p.E;
        const int per_lane = (p.E + kWave - 1) / kWave;  // wave-uniform
#pragma unroll
        for (int t = 0; t < kMaxPerLane; ++t) {
            const int ee = lane + t * kWave;
            v[t] = 0.0;
            if (t < per_lane && ee < p.E) {
                v[t] = lg[ee];
                avail |= 1u << t;
            }
        }
        double sel_v = 0.0;  // lane j keeps the j-th selected logit
        int sel_e = 0;
        for (int j = 0; j < k; ++j) {
            double bv = 0.0;
            int be = 0x7fffffff;  // no candidate
#pragma unroll
            for (int t = 0; t < kMaxPerLane; ++t) {
                const int ee = lane + t * kWave;
                if (t < per_lane && ((avail >> t) & 1u) &&
                    (be == 0x7fffffff || ranks_before(v[t], ee, bv, be))) {
                    bv = v[t];
                    be = ee;
                }
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const double ov = __shfl_xor(bv, o, kWave);
                const int oe = __shfl_xor(be, o, kWave);
                if (oe != 0x7fffffff && (be == 0x7fffffff || ranks_before(ov, oe, bv, be))) {
                    bv = ov;
                    be = oe;
                }
            }
            if ((be & (kWave - 1)) == lane) avail &= ~(1u << (be / kWave));
            if (lane == j) {
                sel_v = bv;
                sel_e = be;
            }
        }
        // routing weights (fp64), lanes 0..k-1 hold the selection in order
        const double top = __shfl(sel_v, 0, kWave);
        double pj = 0.0;
        if (lane < k)
            pj = p.score_fn == 1 ? 1.0 / (1.0 + exp(-sel_v)) : exp(sel_v - top);
        const double total = wave_sum(pj);
        if (lane < k) {
            const int slot = b * k + lane;
            const float wj = (float)(pj / total);
            p.topk_idx[slot] = sel_e;
            p.topk_w[slot] = wj;
            if (p.user_idx) p.user_idx[slot] = sel_e;
            if (p.user_w) p.user_w[slot] = wj;
            s_keys[slot] = (sel_e << kSlotBits) | slot;
        }
    }

    // ---------------------------------------------------- phase 2: buckets
    int P = 1;
    while (P < n) P <<= 1;
    for (int i = n + threadIdx.x; i < P; i += kThreads) s_keys[i] = 0x7fffffff;
    if (threadIdx.x == 0) s_max_rows = 0;
    __syncthreads();
    block_bitonic_sort(s_keys, P);

    DevPlan* plan = p.plan;
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const int key = s_keys[i];
        plan->perm[i] = key & (kMaxSlots - 1);
        s_scan[i] = (i == 0 || (s_keys[i - 1] >> kSlotBits) != (key >> kSlotBits)) ? 1 : 0;
    }
    __syncthreads();
    block_inclusive_scan(s_scan, n, s_wave);
    const int D = s_scan[n - 1];
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const int ee = s_keys[i] >> kSlotBits;
        const int a = s_scan[i] - 1;
        if (i == 0 || (s_keys[i - 1] >> kSlotBits) != ee) {
            s_act_e[a] = ee;
            s_act_start[a] = i;
        }
        if (i == n - 1 || (s_keys[i + 1] >> kSlotBits) != ee) s_act_count[a] = i + 1;
    }
    __syncthreads();
    // classify: rows >= mfma_min_rows go to the MFMA kernels (AUTO)
    for (int a = threadIdx.x; a < D; a += kThreads) {
        const int m = s_act_count[a] - s_act_start[a];
        s_act_count[a] = m;
        atomicMax(&s_max_rows, m);
        int cls = CLS_GEMV;
        if (p.mfma_ok) {
            if (p.path_mode == PATH_MFMA) cls = CLS_MFMA;
            else if (p.path_mode == PATH_AUTO && m >= p.mfma_min_rows) cls = CLS_MFMA;
        }
        s_scan[a] = cls;
    }
    __syncthreads();
    block_inclusive_scan(s_scan, D, s_wave);
    for (int a = threadIdx.x; a < D; a += kThreads) {
        const int before = a == 0 ? 0 : s_scan[a - 1];
        const int cls = s_scan[a] - before;
        const int pos = cls == CLS_MFMA ? before : a - before;
        plan->list_expert[cls][pos] = s_act_e[a];
        plan->list_start[cls][pos] = s_act_start[a];
        plan->list_count[cls][pos] = s_act_count[a];
    }
    if (threadIdx.x == 0) {
        const int n_mfma = s_scan[D - 1];
        plan->num_slots = n;
        plan->num_active = D;
        plan->n_list[CLS_GEMV] = D - n_mfma;
        plan->n_list[CLS_MFMA] = n_mfma;
        plan->max_rows = s_max_rows;
    }
}

template <int ACT>
hipError_t launch_router_act(const RouterArgs& a, int grid, hipStream_t s) {
    const dim3 g(grid), b(kThreads);
    if (a.B <= 1) router_topk_kernel<ACT, 1><<<g, b, 0, s>>>(a);
    else if (a.B <= 2) router_topk_kernel<ACT, 2><<<g, b, 0, s>>>(a);
    else if (a.B <= 4) router_topk_kernel<ACT, 4><<<g, b, 0, s>>>(a);
    else if (a.B <= 8) router_topk_kernel<ACT, 8><<<g, b, 0, s>>>(a);
    else if (a.B <= 16) router_topk_kernel<ACT, 16><<<g, b, 0, s>>>(a);
    else if (a.B <= 32) router_topk_kernel<ACT, 32><<<g, b, 0, s>>>(a);
    else router_topk_kernel<ACT, 64><<<g, b, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

// One wave per expert row: grid = ceil(E / 4) blocks of 256 threads.
hipError_t launch_router(const RouterArgs& a, int act, int grid, hipStream_t s) {
    return act == DT_F32 ? launch_router_act<DT_F32>(a, grid, s)
                         : launch_router_act<DT_BF16>(a, grid, s);
}

}  // namespace moe
