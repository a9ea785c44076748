// router_topk.hip -- router GEMV, then top-k selection, routing weights and
// token-to-expert bucketing.
//
// ailookout.news, "vLLM speeds up Kimi K3 up to 1.9x on NVIDIA GB300 with
// agent-assisted kernels", section "How the specialised decode path works":
// each token activates 16 of 896 experts.  The router matrix is read once per
// forward (25.7 MB fp32 at 896 x 7168), so the first kernel is a
// bandwidth-bound GEMV; selection and bucketing are tiny and latency-bound.
//
// router_gemv_kernel (one row): four waves per expert row, each holding a
//   quarter of the row in registers with all its loads issued at once, so the
//   router is read in about one memory round trip; x is staged in LDS a few
//   rows at a time and applied to the registers.  Logits accumulate in fp64:
//   a bf16 (or fp32) x fp32 product is exact in fp64, so the only error is the
//   fp64 summation, ~1e-16 relative.
// router_mfma_kernel (two rows and more): the same fp64 products and sums on
//   the fp64 matrix cores, 16 experts x 16 rows per tile, over four column
//   ranges whose partial logits the top-k kernel adds in order.
// topk_bucket_kernel: 512-thread workgroups.  Per row, one wave selects the
//   k best (logit, expert) pairs, ties to the lower index, by an exact
//   threshold method (select_topk); the routing weights are computed in fp64;
//   then the slots are grouped by expert into the GEMV / MFMA work lists
//   (build_plan: one rank pass up to 256 slots, a counting sort above).  Up to
//   8 rows, one workgroup does it all; above that, the rows are spread over
//   several workgroups and bucket_kernel follows as its own launch.  Data
//   passes between workgroups only through kernel boundaries, never through a
//   device-scope fence (on gfx950 each such fence writes back and invalidates
//   an XCD's L2).

#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"
#include "select_device.h"

namespace moe {

namespace {

constexpr int kChunk = 512;  // router columns per wave-wide step (8 per lane)

// ---------------------------------------------------------------- router GEMV

constexpr int kGemvThreads = 1024;
constexpr int kGemvWaves = kGemvThreads / kWave;
constexpr int kExpPerBlock = 4;                         // expert rows per workgroup
constexpr int kQuarters = kGemvWaves / kExpPerBlock;    // waves (K ranges) per row
constexpr int kMaxStageRows = 32;                       // rows of x per LDS stage
constexpr int kStageBytes = 65536 - 4096;               // LDS for x (the rest: sums)

// 8 activations at a[0..8) (LDS) as fp32.
template <int ACT> __device__ __forceinline__ void act8(const void* a, float (&v)[8]);
template <> __device__ __forceinline__ void act8<DT_BF16>(const void* a, float (&v)[8]) {
    const u32x4 r = *(const u32x4*)a;
    v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x);
    v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
    v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z);
    v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
}
template <> __device__ __forceinline__ void act8<DT_F32>(const void* a, float (&v)[8]) {
    const f32x4 lo = *(const f32x4*)a;
    const f32x4 hi = *((const f32x4*)a + 1);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
}

// A workgroup of 16 waves serves 4 expert rows; the 4 waves of a row each take
// a quarter of its 512-column chunks and hold that part of the row in
// registers (all loads issued at once).  x is staged in LDS a few rows at a
// time, shared by the 4 rows.  Each wave accumulates its quarter in fp64 (two
// rows at a time, four independent chains per row); the quarters are added
// through LDS in a fixed order.  NCQ: most chunks per quarter (H <= 4 * NCQ *
// 512).
template <int ACT, int NCQ>
__global__ __launch_bounds__(kGemvThreads) void router_gemv_kernel(RouterArgs p) {
    typedef typename Storage<ACT>::type at;
    extern __shared__ __align__(16) unsigned char smem[];
    at* xs = (at*)smem;  // [rows_per_stage][H]
    __shared__ double part[kMaxStageRows][kExpPerBlock][kQuarters];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int el = wave % kExpPerBlock, kq = wave / kExpPerBlock;
    const int e = blockIdx.x * kExpPerBlock + el;
    const bool live = e < p.E;
    const int H = p.H;
    const int nc = H / kChunk;
    const int c0 = kq * nc / kQuarters, c1 = (kq + 1) * nc / kQuarters;

    // this wave's part of the router row, 8 fp32 per lane per chunk
    u32x4 w[NCQ][2];
    if (live) {
        const float* row = p.wr + (int64_t)e * p.wr_stride + lane * 8;
#pragma unroll
        for (int c = 0; c < NCQ; ++c)
            if (c0 + c < c1) {
                w[c][0] = load_weights16(row + (c0 + c) * kChunk);
                w[c][1] = load_weights16(row + (c0 + c) * kChunk + 4);
            }
    }

    constexpr int kVec = 16 / (int)sizeof(at);
    for (int b0 = 0; b0 < p.B; b0 += p.rows_per_stage) {
        const int rs = min(p.rows_per_stage, p.B - b0);
        __syncthreads();  // the previous stage's reads of xs and part are done
        for (int r = 0; r < rs; ++r) {
            const at* src = (const at*)p.x + (int64_t)(b0 + r) * p.x_stride;
            for (int c = threadIdx.x * kVec; c < H; c += kGemvThreads * kVec)
                *(u32x4*)(xs + (int64_t)r * H + c) = load16(src + c);
        }
        __syncthreads();
        for (int r0 = 0; r0 < rs; r0 += 2) {
            double acc[2][4] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
#pragma unroll
            for (int c = 0; c < NCQ; ++c)
                if (c0 + c < c1) {
                    const float wv[8] = {
                        __uint_as_float(w[c][0].x), __uint_as_float(w[c][0].y),
                        __uint_as_float(w[c][0].z), __uint_as_float(w[c][0].w),
                        __uint_as_float(w[c][1].x), __uint_as_float(w[c][1].y),
                        __uint_as_float(w[c][1].z), __uint_as_float(w[c][1].w)};
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        if (r0 + q < rs) {
                            float xv[8];
                            act8<ACT>(xs + (int64_t)(r0 + q) * H + (c0 + c) * kChunk + lane * 8, xv);
#pragma unroll
                            for (int t = 0; t < 8; ++t)
                                acc[q][t & 3] = fma((double)xv[t], (double)wv[t], acc[q][t & 3]);
                        }
                }
#pragma unroll
            for (int q = 0; q < 2; ++q)
                if (r0 + q < rs) {
                    const double sum = wave_sum((acc[q][0] + acc[q][1]) + (acc[q][2] + acc[q][3]));
                    if (lane == 0) part[r0 + q][el][kq] = sum;
                }
        }
        __syncthreads();
        // logits of this stage: quarters added in the order 0, 1, 2, 3
        for (int i = threadIdx.x; i < rs * kExpPerBlock; i += kGemvThreads) {
            const int r = i / kExpPerBlock, ee = i % kExpPerBlock;
            const int eg = blockIdx.x * kExpPerBlock + ee;
            if (eg < p.E) {
                p.logits[(int64_t)(b0 + r) * p.E + eg] =
                    ((part[r][ee][0] + part[r][ee][1]) + part[r][ee][2]) + part[r][ee][3];
            }
        }
    }
}

// One row: the same work and the same arithmetic order as router_gemv_kernel
// (so the same logits, bit for bit), without the LDS stage of x.  Each lane
// loads the 8 activations that meet each of its weight vectors straight into
// registers, before its weight loads: loads return in order, so a chunk's
// products start as soon as that chunk's weights arrive instead of after a
// workgroup barrier that waits for every wave's weights.
template <int ACT, int NCQ>
__global__ __launch_bounds__(kGemvThreads) void router_gemv1_kernel(RouterArgs p) {
    typedef typename Storage<ACT>::type at;
    __shared__ double part[kExpPerBlock][kQuarters];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int el = wave % kExpPerBlock, kq = wave / kExpPerBlock;
    const int e = blockIdx.x * kExpPerBlock + el;
    const bool live = e < p.E;
    const int H = p.H;
    const int nc = H / kChunk;
    const int c0 = kq * nc / kQuarters, c1 = (kq + 1) * nc / kQuarters;

    constexpr int kXVec = 8 * (int)sizeof(at) / 16;  // 16-byte loads per 8 activations
    u32x4 xr[NCQ][kXVec];
    const at* xrow = (const at*)p.x + lane * 8;
#pragma unroll
    for (int c = 0; c < NCQ; ++c)
        if (c0 + c < c1) {
#pragma unroll
            for (int v = 0; v < kXVec; ++v)
                xr[c][v] = load16(xrow + (c0 + c) * kChunk + v * (16 / (int)sizeof(at)));
        }
    u32x4 w[NCQ][2];
    if (live) {
        const float* row = p.wr + (int64_t)e * p.wr_stride + lane * 8;
#pragma unroll
        for (int c = 0; c < NCQ; ++c)
            if (c0 + c < c1) {
                w[c][0] = load_weights16(row + (c0 + c) * kChunk);
                w[c][1] = load_weights16(row + (c0 + c) * kChunk + 4);
            }
    }
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int c = 0; c < NCQ; ++c)
        if (c0 + c < c1) {
            const float wv[8] = {
                __uint_as_float(w[c][0].x), __uint_as_float(w[c][0].y),
                __uint_as_float(w[c][0].z), __uint_as_float(w[c][0].w),
                __uint_as_float(w[c][1].x), __uint_as_float(w[c][1].y),
                __uint_as_float(w[c][1].z), __uint_as_float(w[c][1].w)};
            float xv[8];
            act8<ACT>(xr[c], xv);
#pragma unroll
            for (int t = 0; t < 8; ++t) acc[t & 3] = fma((double)xv[t], (double)wv[t], acc[t & 3]);
        }
    const double sum = wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
    if (lane == 0) part[el][kq] = sum;
    __syncthreads();
    if (threadIdx.x < kExpPerBlock) {
        const int eg = blockIdx.x * kExpPerBlock + threadIdx.x;
        if (eg < p.E)
            p.logits[eg] = ((part[threadIdx.x][0] + part[threadIdx.x][1]) + part[threadIdx.x][2]) +
                           part[threadIdx.x][3];
    }
}

// ------------------------------------------------------ router on matrix cores
//
// The same logits on the fp64 matrix cores, for batches where the GEMV's
// per-row fp32-to-fp64 conversions dominate.  v_mfma_f64_16x16x4_f64 takes
// from lane l the A element [l % 16][l / 16] and the B element [l / 16][l % 16]
// and returns D[l / 16 + 4 i][l % 16], i = 0..3.  A holds 16 rows of x, B
// 16 router rows (experts), 4 columns per step.  Products of bf16 (or fp32)
// activations and fp32 weights are exact in fp64 and the matrix core adds in
// fp64, so the logits are as accurate as the GEMV kernel's.
//
// Lane (c = l % 16, q = l / 16) loads 16 bytes of its expert row, columns
// 16 t + 4 q .. 16 t + 4 q + 3, and the same columns of its x row, and feeds
// them to four successive steps: step r of column group t contracts columns
// 16 t + 4 q + r, q = 0..3.  Each column is contracted once, with the same
// column on both operands: the plain dot product, summed in another order.
//
// A workgroup of 16 waves serves 16 experts over one of gridDim.y column
// ranges; its waves split that range and their 16 x 16 tiles are added
// through LDS in wave order.  Each workgroup writes its range's partial sums,
// which the top-k kernel adds in split order.  All row tiles of the batch are
// served by the same workgroup from the router columns held in registers.
constexpr int kRmWaves = 16;
constexpr int kRmThreads = kRmWaves * kWave;
// ROUTER_AUTO: matrix cores from this many rows.  With the four partial
// slices the top-k adds, the GEMV router is still about 1 us faster per
// layer at two rows; the matrix cores win from three rows up.
constexpr int kRouterMfmaMinBatch = 3;

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f64x4 mfma_f64(double a, double b, f64x4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// 4 activations at x + off as fp32.
template <int ACT> struct XQuad;
template <> struct XQuad<DT_BF16> {
    u32x2 v;
    __device__ __forceinline__ void load(const void* x, int64_t off) {
        v = *(const u32x2*)((const uint16_t*)x + off);
    }
    __device__ __forceinline__ float get(int r) const {
        const uint32_t w = r < 2 ? v.x : v.y;
        return (r & 1) ? bf16_hi(w) : bf16_lo(w);
    }
};
template <> struct XQuad<DT_F32> {
    f32x4 v;
    __device__ __forceinline__ void load(const void* x, int64_t off) {
        v = *(const f32x4*)((const float*)x + off);
    }
    __device__ __forceinline__ float get(int r) const { return v[r]; }
};

// 4 activations of the next layer's input, combined from the previous
// layer's expert outputs (the router with the combine folded in), held in the
// activation type.
template <int ACT> struct XQuadC;
template <> struct XQuadC<DT_BF16> {
    uint32_t lo, hi;  // two packed bf16 pairs
    __device__ __forceinline__ void set(int r, float v) {
        const uint32_t b = f32_to_bf16_bits(v);
        if (r == 0) lo = b;
        else if (r == 1) lo |= b << 16;
        else if (r == 2) hi = b;
        else hi |= b << 16;
    }
    __device__ __forceinline__ float get(int r) const {
        const uint32_t w = r < 2 ? lo : hi;
        return (r & 1) ? bf16_hi(w) : bf16_lo(w);
    }
};
template <> struct XQuadC<DT_F32> {
    float v[4];
    __device__ __forceinline__ void set(int r, float x) { v[r] = x; }
    __device__ __forceinline__ float get(int r) const { return v[r]; }
};

// Columns col .. col + 3 of row `row` of the previous layer's output:
// x[row, n] + sum_j w[row, j] * y[row * k + j, n], j ascending, in fp32, then
// rounded once to the activation type: the operations and order of
// combine_kernel, so the values are bit for bit the ones it would store.
// With `store` they are also written to the previous layer's out.
template <int ACT>
__device__ __forceinline__ void combine_quad(const RouterArgs& p, int row, int col, bool store,
                                             XQuadC<ACT>& o) {
    constexpr int kBatch = 8;  // loads of y in flight per thread
    const int k = p.comb_k, H = p.H;
    const float* yb = p.comb_y + (int64_t)row * k * H + col;
    const float* wb = p.comb_w + (int64_t)row * k;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j0 = 0; j0 < k; j0 += kBatch) {
        f32x4 yv[kBatch];
        float wv[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (j0 + j < k) {
                yv[j] = *(const f32x4*)(yb + (int64_t)(j0 + j) * H);
                wv[j] = wb[j0 + j];
            }
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (j0 + j < k) {
                acc[0] = fmaf(wv[j], yv[j].x, acc[0]);
                acc[1] = fmaf(wv[j], yv[j].y, acc[1]);
                acc[2] = fmaf(wv[j], yv[j].z, acc[2]);
                acc[3] = fmaf(wv[j], yv[j].w, acc[3]);
            }
    }
    const int64_t xi = (int64_t)row * p.x_stride + col;
    const int64_t oi = (int64_t)row * p.comb_out_stride + col;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float v = load_act<ACT>(p.x, xi + t) + acc[t];
        if (store) store_act<ACT>(p.comb_out, oi + t, v);
        o.set(t, v);
    }
}

// NT: most column groups of 16 per wave.  COMB: the router of the next layer
// with the previous layer's combine + residual folded in (p.x is the previous
// layer's input; the combined rows are computed in each workgroup from y and
// the routing weights, and stored by the workgroups of the first expert tile).
// The grid is then one-dimensional with the split as the fast index, so that
// the workgroups of one XCD (dealt round robin) all take the same column
// range and re-read one quarter of y from their own L2.
template <int ACT, int NT, bool COMB>
__global__ __launch_bounds__(kRmThreads) void router_mfma_kernel(RouterArgs p) {
    __shared__ double red[kRmWaves][256];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int c = lane & 15, q = lane >> 4;
    const int S = COMB ? p.k_splits : (int)gridDim.y;
    const int s = COMB ? (int)blockIdx.x % S : (int)blockIdx.y;
    const int tile = COMB ? (int)blockIdx.x / S : (int)blockIdx.x;
    const int e0 = tile * 16;
    const int G = p.H / 16;
    const int gs0 = s * G / S, gs1 = (s + 1) * G / S;
    const int g0 = gs0 + wave * (gs1 - gs0) / kRmWaves;
    const int ng = gs0 + (wave + 1) * (gs1 - gs0) / kRmWaves - g0;

    // Every load is unconditional, from a clamped address: a conditional
    // load would make the compiler wait for all loads in flight before
    // writing the register in the other branch.  Rows past the batch and
    // experts past E only feed outputs that are never stored; groups past
    // ng are not contracted.
    const int gmax = G - 1;
    // the first row tile's x before the router columns: loads return in
    // order, so the first steps wait only for x and the first weight loads
    // and the matrix cores run while the rest of the weights arrive (with the
    // combine folded in, the first tile's rows are combined first, which
    // keeps its loads of y and the router columns out of the registers at
    // the same time)
    typedef typename std::conditional<COMB, XQuadC<ACT>, XQuad<ACT>>::type XQ;
    XQ xq[NT];
    if constexpr (COMB) {
        const int row = min(c, p.B - 1);
        const bool store = tile == 0 && c < p.B;
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (t < ng) combine_quad<ACT>(p, row, (g0 + t) * 16 + 4 * q, store, xq[t]);
    } else {
        const int64_t xoff = (int64_t)min(c, p.B - 1) * p.x_stride + 4 * q;
#pragma unroll
        for (int t = 0; t < NT; ++t) xq[t].load(p.x, xoff + min(g0 + t, gmax) * 16);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the load order: x first
    u32x4 w[NT];
    const float* wrow = p.wr + (int64_t)min(e0 + c, p.E - 1) * p.wr_stride + 4 * q;
#pragma unroll
    for (int t = 0; t < NT; ++t) w[t] = load_weights16(wrow + min(g0 + t, gmax) * 16);
    __builtin_amdgcn_sched_barrier(0);

    for (int r0 = 0; r0 < (COMB ? 16 : p.B); r0 += 16) {
        if constexpr (COMB) {
            // one row tile only (batches of up to 16 rows): the combine of a
            // second tile beside the router columns would not fit the registers
        } else if (r0 > 0) {
            const int64_t xoff = (int64_t)min(r0 + c, p.B - 1) * p.x_stride + 4 * q;
#pragma unroll
            for (int t = 0; t < NT; ++t) xq[t].load(p.x, xoff + min(g0 + t, gmax) * 16);
        }
        f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < ng) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc = mfma_f64((double)xq[t].get(r), (double)__uint_as_float(w[t][r]), acc);
            }
            // convert each group just before its steps (hoisting every
            // conversion ahead of the chain would take 128 more VGPRs)
            __builtin_amdgcn_sched_barrier(0);
        }
        if (r0 > 0) __syncthreads();  // the previous tile's sums are read
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][(q + 4 * i) * 16 + c] = acc[i];
        __syncthreads();
        if (threadIdx.x < 256) {
            const int m = threadIdx.x >> 4, n = threadIdx.x & 15;
            double sum = red[0][threadIdx.x];
#pragma unroll
            for (int v = 1; v < kRmWaves; ++v) sum += red[v][threadIdx.x];
            if (r0 + m < p.B && e0 + n < p.E)
                p.logits[((int64_t)s * p.B + r0 + m) * p.E + e0 + n] = sum;
        }
    }
}

// ------------------------------------------------------- top-k and buckets

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kRankSortMax = 256;  // slots up to which the plan is built in one rank pass

// Inclusive prefix sum of arr[0..n), n <= kMaxSlots, in place (all threads).
__device__ void block_inclusive_scan(int* arr, int n, int* s_wave) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    constexpr int kPer = kMaxSlots / kSelThreads;
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

// Lane l's logits of row b: experts l, l + 64, ... (0 past E), the router's
// partial sums added in split order, then the bias.  Adding +0.0 turns -0
// into +0, so that equal logits have equal keys.
template <int PL>
__device__ __forceinline__ void load_logit_row(const RouterArgs& p, int b, double (&v)[PL]) {
    const int lane = threadIdx.x & (kWave - 1);
    const double* lg = p.logits + (int64_t)b * p.E;
    const int S = p.k_splits;
    if (PL <= 16 && S > 1) {
        // every partial is loaded before any is added (one memory round trip;
        // loads past S or E read a valid element that is not used)
        const int64_t split = (int64_t)p.B * p.E;
        double part[kMaxRouterSplits][PL];
#pragma unroll
        for (int j = 0; j < kMaxRouterSplits; ++j)
#pragma unroll
            for (int t = 0; t < PL; ++t) {
                const int ee = min(lane + t * kWave, p.E - 1);
                part[j][t] = lg[(j < S ? j : 0) * split + ee];
            }
#pragma unroll
        for (int t = 0; t < PL; ++t) {
            double sum = part[0][t];
#pragma unroll
            for (int j = 1; j < kMaxRouterSplits; ++j)
                if (j < S) sum += part[j][t];
            v[t] = lane + t * kWave < p.E ? sum : 0.0;
        }
    } else {
        const int64_t split = (int64_t)p.B * p.E;
#pragma unroll
        for (int t = 0; t < PL; ++t) {
            const int ee = lane + t * kWave;
            v[t] = ee < p.E ? lg[ee] : 0.0;
        }
#pragma unroll 1
        for (int j = 1; j < S; ++j)
#pragma unroll
            for (int t = 0; t < PL; ++t) {
                const int ee = lane + t * kWave;
                if (ee < p.E) v[t] += lg[j * split + ee];
            }
    }
#pragma unroll
    for (int t = 0; t < PL; ++t) {
        const int ee = lane + t * kWave;
        if (p.bias && ee < p.E) v[t] += (double)p.bias[ee];
        v[t] += 0.0;
    }
}

// The expert buckets of the n = B * k slots, from keys[i] = (expert << 11) |
// slot (all threads; keys filled by the caller before a barrier this function
// starts with): the slots sorted by (expert, slot), the distinct experts with
// their first slot and row count, split into the GEMV and MFMA lists.
struct BucketLds {
    alignas(16) int keys[kMaxSlots];
    int scan[kMaxSlots];
    int act_e[kMaxSlots];
    int act_start[kMaxSlots];
    int act_count[kMaxSlots];
    int e_start[kMaxExperts];  // counting sort: first position of each expert
    int wave_sums[kSelWaves];
    int wave_sums2[kSelWaves];
    int max_rows;
};

// The slots grouped by expert for n > kRankSortMax, by a stable counting sort
// (all threads; the caller's keys in place, no barrier needed before): counts
// per expert by LDS atomics, one scan over the experts of (count | present <<
// 16) that gives every expert its first position and its index in the active
// list, the slots dropped at their expert's cursor, then put in slot order
// within each expert's range (each slot counts the smaller slots of its
// range).  Writes perm and the active lists (act_count = end of the range);
// returns D.
__device__ int bucket_by_counting(const RouterArgs& p, int n, BucketLds& L) {
    constexpr int kPer = kMaxSlots / kSelThreads;
    static_assert(kMaxExperts <= kMaxSlots, "the expert scan uses the slot scan");
    const int E = p.E;
    for (int e = threadIdx.x; e < E; e += kSelThreads) L.scan[e] = 0;
    __syncthreads();
    int mine[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int i = q * kSelThreads + threadIdx.x;
        mine[q] = i < n ? L.keys[i] : 0;
        if (i < n) atomicAdd(&L.scan[mine[q] >> kSlotBits], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kSelThreads) {
        const int c = L.scan[e];
        L.scan[e] = c | (c > 0 ? 1 << 16 : 0);
    }
    __syncthreads();
    block_inclusive_scan(L.scan, E, L.wave_sums);
    int first[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = q * kSelThreads + threadIdx.x;
        first[q] = 0;
        if (e < E) {
            const int incl = L.scan[e];
            const int c = (incl - (e ? L.scan[e - 1] : 0)) & 0xffff;
            first[q] = (incl & 0xffff) - c;
            if (c) {
                const int a = (incl >> 16) - 1;
                L.act_e[a] = e;
                L.act_start[a] = first[q];
                L.act_count[a] = first[q] + c;
            }
        }
    }
    const int D = L.scan[E - 1] >> 16;
    __syncthreads();  // every read of the scan happens before the cursors below
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int e = q * kSelThreads + threadIdx.x;
        if (e < E) L.scan[e] = L.e_start[e] = first[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int i = q * kSelThreads + threadIdx.x;
        if (i < n) L.keys[atomicAdd(&L.scan[mine[q] >> kSlotBits], 1)] = i;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int i = q * kSelThreads + threadIdx.x;
        if (i < n) {
            const int e = mine[q] >> kSlotBits;
            const int st = L.e_start[e], end = L.scan[e];
            int rank = 0;
            for (int j = st; j < end; ++j) rank += L.keys[j] < i ? 1 : 0;
            p.plan->perm[st + rank] = i;
        }
    }
    return D;
}

// Expert class of an active expert with m routed rows: MFMA when the path
// forces it, or under AUTO from mfma_min_rows rows up and for every expert
// with more rows than the GEMV kernels stage per pass (weight types with an
// MFMA kernel only); GEMV otherwise.
__device__ __forceinline__ int expert_class(const RouterArgs& p, int m) {
    if (!p.mfma_ok) return CLS_GEMV;
    if (p.path_mode == PATH_MFMA) return CLS_MFMA;
    return p.path_mode == PATH_AUTO && (m >= p.mfma_min_rows || m > kGemvPassRows) ? CLS_MFMA
                                                                                    : CLS_GEMV;
}

// The plan for n <= kRankSortMax slots (all threads; keys[i] = expert <<
// kSlotBits | i in LDS, filled by the caller).  Each slot is served by T
// adjacent lanes (T = 2 .. 64, the most that fit in the workgroup), which
// split one pass over all keys, four at a time with same-address LDS reads,
// and add their counts with lane shuffles: the slot's rank (its position in
// perm: slots ordered by expert, then slot), the first position of its expert
// (the keys of smaller experts) and its expert's row count.  The slot at its
// expert's first position is that expert's representative; the
// representatives of each class are numbered by ballots over the thread
// index, so the two work lists are written with one barrier and no scan.
// List entries follow the representatives' slot order, not the expert order;
// the expert kernels do not depend on it.
__device__ void build_plan_small(const RouterArgs& p, int n, BucketLds& L) {
    static_assert(2 * kRankSortMax <= kSelThreads, "at least two lanes per slot");
    int T = 2;
    while (T < kWave && 2 * T * n <= kSelThreads) T *= 2;
    const int i = threadIdx.x, lane = i & (kWave - 1), wave = i / kWave;
    const int slot = i / T, sub = i & (T - 1);
    if (i == 0) L.max_rows = 0;
    if (i < ((n + 3) & ~3) - n) L.keys[n + i] = 0x7fffffff;  // past every expert
    __syncthreads();
    const bool live = slot < n;
    const int mine = live ? L.keys[slot] : 0;
    const int e = mine >> kSlotBits;
    // smaller keys; keys of smaller experts; keys of experts up to e
    const int lo = e << kSlotBits, hi = (e + 1) << kSlotBits;
    int pos = 0, lt = 0, le = 0;
    if (live) {
        const int4* k4 = (const int4*)L.keys;
        const int n4 = (n + 3) >> 2;
#pragma unroll 2
        for (int j = sub; j < n4; j += T) {
            const int4 v = k4[j];
            pos += (v.x < mine) + (v.y < mine) + (v.z < mine) + (v.w < mine);
            lt += (v.x < lo) + (v.y < lo) + (v.z < lo) + (v.w < lo);
            le += (v.x < hi) + (v.y < hi) + (v.z < hi) + (v.w < hi);
        }
    }
    for (int o = 1; o < T; o <<= 1) {
        pos += __shfl_xor(pos, o, kWave);
        lt += __shfl_xor(lt, o, kWave);
        le += __shfl_xor(le, o, kWave);
    }
    const int m = le - lt;
    const bool rep = live && sub == 0 && pos == lt;
    const int cls = expert_class(p, m);
    const uint64_t bm = __ballot(rep && cls == CLS_MFMA);
    const uint64_t bg = __ballot(rep && cls == CLS_GEMV);
    if (lane == 0) {
        L.wave_sums[wave] = __popcll(bm);
        L.wave_sums2[wave] = __popcll(bg);
    }
    if (rep) atomicMax(&L.max_rows, m);
    __syncthreads();
    int om = 0, og = 0, tm = 0, tg = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const int a = L.wave_sums[w], b = L.wave_sums2[w];
        if (w < wave) {
            om += a;
            og += b;
        }
        tm += a;
        tg += b;
    }
    DevPlan* plan = p.plan;
    if (live && sub == 0) plan->perm[pos] = slot;
    if (rep) {
        const uint64_t below = (1ull << lane) - 1ull;
        const int a = cls == CLS_MFMA ? om + __popcll(bm & below) : og + __popcll(bg & below);
        plan->list_expert[cls][a] = e;
        plan->list_start[cls][a] = lt;
        plan->list_count[cls][a] = m;
    }
    if (i == 0) {
        plan->num_slots = n;
        plan->num_active = tm + tg;
        plan->n_list[CLS_GEMV] = tg;
        plan->n_list[CLS_MFMA] = tm;
        plan->max_rows = L.max_rows;
    }
}

__device__ void build_plan(const RouterArgs& p, int n, BucketLds& L) {
    // small batches: one rank pass and ballots; larger ones: a counting sort
    // over the experts, then a scan of the expert classes
    if (n <= kRankSortMax) {
        build_plan_small(p, n, L);
        return;
    }
    if (threadIdx.x == 0) L.max_rows = 0;
    DevPlan* plan = p.plan;
    const int D = bucket_by_counting(p, n, L);
    __syncthreads();
    // classify: rows >= mfma_min_rows go to the MFMA kernels (AUTO)
    for (int a = threadIdx.x; a < D; a += kSelThreads) {
        const int m = L.act_count[a] - L.act_start[a];
        L.act_count[a] = m;
        atomicMax(&L.max_rows, m);
        L.scan[a] = expert_class(p, m);
    }
    __syncthreads();
    block_inclusive_scan(L.scan, D, L.wave_sums);
    for (int a = threadIdx.x; a < D; a += kSelThreads) {
        const int before = a == 0 ? 0 : L.scan[a - 1];
        const int cls = L.scan[a] - before;
        const int pos = cls == CLS_MFMA ? before : a - before;
        plan->list_expert[cls][pos] = L.act_e[a];
        plan->list_start[cls][pos] = L.act_start[a];
        plan->list_count[cls][pos] = L.act_count[a];
    }
    if (threadIdx.x == 0) {
        const int n_mfma = L.scan[D - 1];
        plan->num_slots = n;
        plan->num_active = D;
        plan->n_list[CLS_GEMV] = D - n_mfma;
        plan->n_list[CLS_MFMA] = n_mfma;
        plan->max_rows = L.max_rows;
    }
}

// Top-k of row b by this wave: selection, routing weights, the routing
// outputs; returns the selected expert in lanes < k.
template <int PL>
__device__ __forceinline__ int select_row(const RouterArgs& p, int b, double* cv, int* ce,
                                          double* sv, int* se) {
    const int lane = threadIdx.x & (kWave - 1);
    const int k = p.k;
    double v[PL];
    load_logit_row<PL>(p, b, v);
    double sel_v = 0.0;  // lane j keeps the j-th selected logit
    int sel_e = 0;
    select_topk<PL>(v, p.E, k, cv, ce, sv, se, sel_v, sel_e);
    const float wj = routing_weight(sel_v, k, p.score_fn);
    if (lane < k) {
        const int slot = b * k + lane;
        p.topk_idx[slot] = sel_e;
        p.topk_w[slot] = wj;
        if (p.user_idx) p.user_idx[slot] = sel_e;
        if (p.user_w) p.user_w[slot] = wj;
    }
    return sel_e;
}

// PL: logits held per lane in the top-k rounds (E <= 64 * PL).
// PLAN: one workgroup does every row (one wave per row) and then the
// buckets; otherwise each workgroup does kSelWaves rows and
// bucket_kernel follows.
template <int PL, bool PLAN>
__global__ __launch_bounds__(kSelThreads) void topk_bucket_kernel(RouterArgs p) {
    __shared__ BucketLds L;
    __shared__ double s_cv[kSelWaves][kWave];  // top-k candidates of each wave's row
    __shared__ int s_ce[kSelWaves][kWave];
    __shared__ double s_sv[kSelWaves][kMaxTopk];  // the selection, in order
    __shared__ int s_se[kSelWaves][kMaxTopk];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int k = p.k;
    const int n = p.B * k;

    if (!PLAN) {
        const int b = blockIdx.x * kSelWaves + wave;
        if (b < p.B) select_row<PL>(p, b, s_cv[wave], s_ce[wave], s_sv[wave], s_se[wave]);
        return;
    }

    if (p.B == 1) {
        // one row: its k experts are distinct, so every expert has one slot
        // and the plan follows the selection order without any sort
        if (wave != 0) return;
        const int sel_e = select_row<PL>(p, 0, s_cv[0], s_ce[0], s_sv[0], s_se[0]);
        const int cls = p.mfma_ok && (p.path_mode == PATH_MFMA ||
                                      (p.path_mode == PATH_AUTO && p.mfma_min_rows <= 1))
                            ? CLS_MFMA
                            : CLS_GEMV;
        DevPlan* plan = p.plan;
        if (lane < k) {
            plan->perm[lane] = lane;
            plan->list_expert[cls][lane] = sel_e;
            plan->list_start[cls][lane] = lane;
            plan->list_count[cls][lane] = 1;
        }
        if (lane == 0) {
            plan->num_slots = k;
            plan->num_active = k;
            plan->n_list[cls] = k;
            plan->n_list[1 - cls] = 0;
            plan->max_rows = 1;
        }
        return;
    }

    for (int b = wave; b < p.B; b += kSelWaves) {
        const int sel_e = select_row<PL>(p, b, s_cv[wave], s_ce[wave], s_sv[wave], s_se[wave]);
        if (lane < k) L.keys[b * k + lane] = (sel_e << kSlotBits) | (b * k + lane);
    }
    build_plan(p, n, L);
}

// The buckets after a multi-workgroup top-k: keys from the routing it wrote.
__global__ __launch_bounds__(kSelThreads) void bucket_kernel(RouterArgs p) {
    __shared__ BucketLds L;
    const int n = p.B * p.k;
    for (int i = threadIdx.x; i < n; i += kSelThreads)
        L.keys[i] = (p.topk_idx[i] << kSlotBits) | i;
    build_plan(p, n, L);
}

template <bool PLAN>
void launch_topk(const RouterArgs& a, int grid, hipStream_t s) {
    const int pl = (a.E + kWave - 1) / kWave;
    if (pl <= 1) topk_bucket_kernel<1, PLAN><<<grid, kSelThreads, 0, s>>>(a);
    else if (pl <= 2) topk_bucket_kernel<2, PLAN><<<grid, kSelThreads, 0, s>>>(a);
    else if (pl <= 4) topk_bucket_kernel<4, PLAN><<<grid, kSelThreads, 0, s>>>(a);
    else if (pl <= 8) topk_bucket_kernel<8, PLAN><<<grid, kSelThreads, 0, s>>>(a);
    else if (pl <= 16) topk_bucket_kernel<16, PLAN><<<grid, kSelThreads, 0, s>>>(a);
    else topk_bucket_kernel<32, PLAN><<<grid, kSelThreads, 0, s>>>(a);
}

template <int ACT>
hipError_t launch_router_gemv(const RouterArgs& a, hipStream_t s) {
    const dim3 grid((a.E + kExpPerBlock - 1) / kExpPerBlock), block(kGemvThreads);
    const size_t lds = (size_t)a.rows_per_stage * a.H * sizeof(typename Storage<ACT>::type);
    const int ncq = (a.H / kChunk + kQuarters - 1) / kQuarters;
    if (a.B == 1) {
        if (ncq <= 1) router_gemv1_kernel<ACT, 1><<<grid, block, 0, s>>>(a);
        else if (ncq <= 2) router_gemv1_kernel<ACT, 2><<<grid, block, 0, s>>>(a);
        else router_gemv1_kernel<ACT, 4><<<grid, block, 0, s>>>(a);
        return hipGetLastError();
    }
    if (ncq <= 1) router_gemv_kernel<ACT, 1><<<grid, block, lds, s>>>(a);
    else if (ncq <= 2) router_gemv_kernel<ACT, 2><<<grid, block, lds, s>>>(a);
    else router_gemv_kernel<ACT, 4><<<grid, block, lds, s>>>(a);
    return hipGetLastError();
}

// Splits of the column range over workgroups for the matrix-core router (at
// most one 16-expert tile per CU and split, more if a wave would otherwise
// need more than 8 column groups of 16), and the groups per wave that follow;
// groups = 0 if even kMaxRouterSplits splits leave more than 8 per wave.
struct RmShape {
    int splits, groups;
};
RmShape router_mfma_shape(int E, int H) {
    const int tiles = (E + 15) / 16;
    int S = 256 / tiles;
    S = S < 1 ? 1 : (S > kMaxRouterSplits ? kMaxRouterSplits : S);
    const int G = H / 16;
    for (;; ++S) {
        const int per_wg = (G + S - 1) / S;
        const int per_wave = (per_wg + kRmWaves - 1) / kRmWaves;
        if (per_wave <= 8) return {S, per_wave};
        if (S == kMaxRouterSplits) return {S, 0};
    }
}

template <int ACT, bool COMB>
hipError_t launch_router_mfma(const RouterArgs& a, RmShape sh, hipStream_t s) {
    const int tiles = (a.E + 15) / 16;
    const dim3 grid = COMB ? dim3(tiles * sh.splits) : dim3(tiles, sh.splits);
    const dim3 block(kRmThreads);
    if (sh.groups <= 1) router_mfma_kernel<ACT, 1, COMB><<<grid, block, 0, s>>>(a);
    else if (sh.groups <= 2) router_mfma_kernel<ACT, 2, COMB><<<grid, block, 0, s>>>(a);
    else if (sh.groups <= 4) router_mfma_kernel<ACT, 4, COMB><<<grid, block, 0, s>>>(a);
    else router_mfma_kernel<ACT, 8, COMB><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

// Rows of x staged in LDS per pass of the router GEMV (with the partial
// sums, at most 64 KB of LDS).
int router_rows_per_stage(int H, int act, int B) {
    const int row_bytes = H * (act == DT_F32 ? 4 : 2);
    int r = kStageBytes / row_bytes;
    if (r < 1) r = 1;
    if (r > kMaxStageRows) r = kMaxStageRows;
    return r < B ? r : B;
}

// The router, then the top-k and buckets.
//
// Router: the GEMV kernel (ceil(E / 4) workgroups of 16 waves; H a multiple
// of 512, at most 8192; rows_per_stage set by router_rows_per_stage), or the
// matrix-core kernel (ceil(E / 16) x splits workgroups of 16 waves; H a
// multiple of 16).  ROUTER_AUTO takes the matrix cores from
// kRouterMfmaMinBatch rows up.
// Top-k: one workgroup for batches of up to 8 rows (one wave per row); above
// that, one wave per row over ceil(B / 8) workgroups, then one workgroup for
// the buckets.
// Whether launch_router takes the matrix-core router for this request.
bool router_uses_mfma(int router_mode, int B, int E, int H) {
    const RmShape sh = router_mfma_shape(E, H);
    const bool gemv_ok = H % kChunk == 0 && H <= 4 * 4 * kChunk;
    bool mfma = router_mode == ROUTER_MFMA || (router_mode == ROUTER_AUTO && B >= kRouterMfmaMinBatch);
    if (sh.groups == 0) mfma = false;
    if (!gemv_ok && sh.groups > 0) mfma = true;
    return mfma;
}

// The combine + router kernel serves one 16-row tile of the batch.
constexpr int kCombineRouterMaxBatch = 16;

bool combine_router_supported(int E, int H, int B) {
    return B <= kCombineRouterMaxBatch && router_mfma_shape(E, H).groups > 0;
}

hipError_t launch_combine_router(const RouterArgs& a0, int act, hipStream_t s, int* splits) {
    RouterArgs a = a0;
    const RmShape sh = router_mfma_shape(a.E, a.H);
    if (!combine_router_supported(a.E, a.H, a.B)) return hipErrorInvalidValue;
    a.k_splits = sh.splits;
    *splits = sh.splits;
    return act == DT_F32 ? launch_router_mfma<DT_F32, true>(a, sh, s)
                         : launch_router_mfma<DT_BF16, true>(a, sh, s);
}

hipError_t launch_router(const RouterArgs& a0, int act, hipStream_t s, int* kernel, int* launches) {
    RouterArgs a = a0;
    if (a.logits_ready > 0) {
        // the previous layer's combine + router kernel left the logits
        a.k_splits = a.logits_ready;
        *kernel = ROUTER_MFMA;
        *launches = a.B <= kSelWaves ? 1 : 2;
        if (a.B <= kSelWaves) {
            launch_topk<true>(a, 1, s);
        } else {
            launch_topk<false>(a, (a.B + kSelWaves - 1) / kSelWaves, s);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            bucket_kernel<<<1, kSelThreads, 0, s>>>(a);
        }
        return hipGetLastError();
    }
    const RmShape sh = router_mfma_shape(a.E, a.H);
    const bool gemv_ok = a.H % kChunk == 0 && a.H <= 4 * 4 * kChunk;
    bool mfma = a.router_mode == ROUTER_MFMA ||
                (a.router_mode == ROUTER_AUTO && a.B >= kRouterMfmaMinBatch);
    if (sh.groups == 0) mfma = false;
    if (!gemv_ok && sh.groups > 0) mfma = true;
    if (a.logits_only && gemv_ok) mfma = false;  // one slice of logits for the selecting kernel
    hipError_t e;
    if (mfma) {
        a.k_splits = sh.splits;
        e = act == DT_F32 ? launch_router_mfma<DT_F32, false>(a, sh, s)
                          : launch_router_mfma<DT_BF16, false>(a, sh, s);
    } else {
        a.k_splits = 1;
        e = act == DT_F32 ? launch_router_gemv<DT_F32>(a, s) : launch_router_gemv<DT_BF16>(a, s);
    }
    if (e != hipSuccess) return e;
    *kernel = mfma ? ROUTER_MFMA : ROUTER_GEMV;
    if (a.logits_only) {
        *launches = 1;
        return mfma ? hipErrorInvalidValue : hipSuccess;
    }
    *launches = a.B <= kSelWaves ? 2 : 3;
    if (a.B <= kSelWaves) {
        launch_topk<true>(a, 1, s);
    } else {
        launch_topk<false>(a, (a.B + kSelWaves - 1) / kSelWaves, s);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        bucket_kernel<<<1, kSelThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace moe
