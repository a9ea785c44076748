// expert_mfma.hip -- split-K grouped GEMM on the gfx950 matrix cores for
// experts that several rows of the batch are routed to.
//
// ailookout.news, "vLLM speeds up Kimi K3 up to 1.9x on NVIDIA GB300 with
// agent-assisted kernels", section "How the specialised decode path works":
// kernels are chosen by batch size, small-matrix kernels at batch one or two
// and split-K kernels above that.  Here the choice is made per expert, on the
// device, from the number of rows routed to it (the routing plan's MFMA list).
//
// The work is still bound by HBM (about m flop per weight byte for m rows,
// against a ridge near 310), so the matrix cores are there to keep the VALU
// and LDS out of the way as m grows, not to be saturated.  An M tile of 16
// rows is padded with zero rows; the padding costs matrix-core cycles only.
//
// Instruction: v_mfma_f32_16x16x32_bf16, D[16x16] += A[16x32] * B[32x16].
//   A (activations): lane l holds row l%16, K elements 8*(l/16) .. +8;
//   B (weights):     lane l holds column l%16, K elements 8*(l/16) .. +8;
//   D:               lane l holds rows 4*(l/16) + i (i = 0..3), column l%16.
// A sum over K does not depend on the order of its terms, so within a K block
// of 128 elements the lanes may feed the MFMAs any K order that the weight
// and activation fragments share.  The order is chosen so that every weight
// load instruction reads 64 contiguous bytes of each of 16 rows (the four
// lanes of a row read consecutive 16-byte pieces): bf16 instruction q feeds
// MFMA q, an fp8 instruction feeds two MFMAs.
//
// fp8 (OCP e4m3) weights are converted to bf16 in registers, which is exact;
// the per-output-row scale multiplies the fp32 accumulator.
//
// Work units: (active expert, block of 16*NT output rows, K split s), one
// unit per workgroup.  Within a unit the four waves split K among themselves
// and their partial sums are added through LDS in a fixed order.  With
// split_k == 1 the epilogue is applied directly (SwiGLU into h, or the scaled
// down projection into y); otherwise each split writes fp32 partial sums
// [s][slot][cols] that a later pass adds in the fixed order s = 0, 1, ..., so
// results do not depend on scheduling.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kKB = 128;  // K elements per block step (4 MFMAs of K = 32)

// Weight fragment of one 16-row tile for one K block of 128 elements.  Lane
// l (n = l%16, g = l/16) reads weight row n; in load instruction i the four
// lanes of a row read 64 contiguous bytes at byte offset 64i + 16g.  off(q, g)
// is the element offset, within the K block, of the 8 elements lane group g
// feeds to MFMA q; the activation fragment is read at the same offsets.
template <int WDT> struct WFrag;

template <> struct WFrag<DT_BF16> {
    static constexpr int kLoads = 4;  // 16 bytes = one MFMA operand each
    __device__ __forceinline__ static int off(int q, int g) { return 32 * q + 8 * g; }
    __device__ __forceinline__ static void load(const void* row, int64_t k, int g,
                                                u32x4 (&v)[kLoads]) {
        const uint16_t* p = (const uint16_t*)row + k + 8 * g;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) v[i] = load_weights16(p + 32 * i);
    }
    __device__ __forceinline__ static bf16x8 op(const u32x4 (&v)[kLoads], int q) {
        return __builtin_bit_cast(bf16x8, v[q]);
    }
};

template <> struct WFrag<DT_FP8> {
    static constexpr int kLoads = 2;  // 16 bytes = two MFMA operands each
    __device__ __forceinline__ static int off(int q, int g) {
        return 64 * (q >> 1) + 16 * g + 8 * (q & 1);
    }
    __device__ __forceinline__ static void load(const void* row, int64_t k, int g,
                                                u32x4 (&v)[kLoads]) {
        const uint8_t* p = (const uint8_t*)row + k + 16 * g;
        v[0] = load_weights16(p);
        v[1] = load_weights16(p + 64);
    }
    // eight e4m3 codes -> eight bf16, exactly: through fp32 (v_cvt_pk_f32_fp8),
    // keeping the upper halves.  The direct fp8 -> bf16 conversion with a unit
    // scale (v_cvt_scalef32_pk_bf16_fp8) dropped the last mantissa bit of half
    // of the codes when checked on gfx950.
    __device__ __forceinline__ static bf16x8 op(const u32x4 (&v)[kLoads], int q) {
        const u32x4 w = v[q >> 1];
        const uint32_t d0 = (q & 1) ? w.z : w.x;
        const uint32_t d1 = (q & 1) ? w.w : w.y;
        uint32_t a0, a1, b0, b1;
        fp8x4_to_bf16x4(d0, a0, a1);
        fp8x4_to_bf16x4(d1, b0, b1);
        return __builtin_bit_cast(bf16x8, u32x4{a0, a1, b0, b1});
    }
};

// Activation fragment of one 16-row M tile for one K block: lane l supplies
// row l%16 at the offsets off(q, l/16) (zero for padding rows, row == nullptr).
template <int WDT>
__device__ __forceinline__ void load_act_frag(const uint16_t* row, int64_t k, int g,
                                              u32x4 (&a)[4]) {
    if (row) {
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = load16(row + k + WFrag<WDT>::off(q, g));
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = u32x4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}

// ------------------------------------------------------------- gate / up

// Sum the four waves' accumulator tiles (kept in LDS as red[wave][tile][lane *
// 4 + r]) in the order wave 0, 1, 2, 3: thread t of the workgroup gets
// element t of each tile, i.e. D row 4 * ((t / 4) / 16) + t % 4, column
// (t / 4) % 16 of that tile.
template <int TILES>
__device__ __forceinline__ float reduce_waves(const float (*red)[TILES][kWave * 4], int tile) {
    const int t = threadIdx.x;
    return ((red[0][tile][t] + red[1][tile][t]) + red[2][tile][t]) + red[3][tile][t];
}

// One unit per workgroup: NT 16-row tiles of gate rows and the matching up
// rows of one expert, over the K range of split s.  The four waves take the
// unit's K blocks in turn (wave w: blocks w, w + 4, ...), so together they
// read 1 KB of each weight row per step, then their accumulators are summed
// through LDS in a fixed order and the SwiGLU epilogue is applied.
template <int WDT, int NT>
__global__ __launch_bounds__(kThreads) void gate_up_mfma_kernel(ExpertArgs p) {
    typedef WFrag<WDT> F;
    __shared__ float red[kWaves][2 * NT][kWave * 4];  // gate tiles, then up tiles
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int ln = lane & 15, lg = lane >> 4;
    const int H = p.H, I = p.I;
    const DevPlan* plan = p.plan;
    const int S = p.split_k;
    constexpr int kRows = 16 * NT;
    const int blocks = I / kRows;
    const int units = plan->n_list[CLS_MFMA] * blocks * S;
    const int nkb = H / kKB;
    constexpr int kWB = WDT == DT_FP8 ? 1 : 2;  // weight bytes per element

    for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int s = unit % S;
        const int rest = unit / S;
        const int blk = rest % blocks;
        const int a = rest / blocks;
        const int e = plan->list_expert[CLS_MFMA][a];
        const int start = plan->list_start[CLS_MFMA][a];
        const int m = plan->list_count[CLS_MFMA][a];
        const int i0 = blk * kRows;
        const int kb0 = s * nkb / S, kb1 = (s + 1) * nkb / S;
        const char* wexp = (const char*)p.w_gate_up + (int64_t)e * 2 * I * H * kWB;

        for (int mp = 0; mp < m; mp += 16) {
            // this lane's activation row (A operand): row mp + ln of the expert
            const uint16_t* arow = nullptr;
            if (mp + ln < m) {
                const int slot = plan->perm[start + mp + ln];
                arow = (const uint16_t*)p.x + (int64_t)(slot / p.k) * p.x_stride;
            }
            f32x4 ag[NT], au[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) ag[t] = au[t] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 2
            for (int kb = kb0 + wave; kb < kb1; kb += kWaves) {
                const int64_t k = (int64_t)kb * kKB;
                u32x4 wg[NT][F::kLoads], wu[NT][F::kLoads];
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int i = i0 + 16 * t + ln;
                    F::load(wexp + (int64_t)i * H * kWB, k, lg, wg[t]);
                    F::load(wexp + (int64_t)(I + i) * H * kWB, k, lg, wu[t]);
                }
                u32x4 af[4];
                load_act_frag<WDT>(arow, k, lg, af);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        ag[t] = mfma16(af[q], F::op(wg[t], q), ag[t]);
                        au[t] = mfma16(af[q], F::op(wu[t], q), au[t]);
                    }
            }

            __syncthreads();  // the previous pass's reads of red are done
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                *(f32x4*)&red[wave][t][lane * 4] = ag[t];
                *(f32x4*)&red[wave][NT + t][lane * 4] = au[t];
            }
            __syncthreads();
            const int li = threadIdx.x >> 2, r = threadIdx.x & 3;
            const int row = mp + 4 * (li >> 4) + r;
            if (row < m) {
                const int slot = plan->perm[start + row];
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int col = i0 + 16 * t + (li & 15);
                    float sg = 1.0f, su = 1.0f;
                    if (p.s_gu) {
                        sg = p.s_gu[(int64_t)e * 2 * I + col];
                        su = p.s_gu[(int64_t)e * 2 * I + I + col];
                    }
                    const float g = reduce_waves<2 * NT>(red, t) * sg;
                    const float u = reduce_waves<2 * NT>(red, NT + t) * su;
                    if (S == 1) {
                        store_act<DT_BF16>(p.h, (int64_t)slot * I + col, silu_mul(g, u));
                    } else {
                        float* part = p.partial + ((int64_t)s * p.slot_cap + slot) * 2 * I;
                        part[col] = g;
                        part[I + col] = u;
                    }
                }
            }
        }
    }
}

// h[slot, i] = round(silu(sum_s g_s) * sum_s u_s) for the slots of MFMA
// experts, summing the split partials in the order s = 0, 1, ...
__global__ __launch_bounds__(kThreads) void gate_up_reduce_kernel(ExpertArgs p) {
    const DevPlan* plan = p.plan;
    const int I = p.I, S = p.split_k;
    const int n_exp = plan->n_list[CLS_MFMA];
    // one block per (expert, row) pair, walked by the grid
    int pair = 0;
    for (int a = 0; a < n_exp; ++a) {
        const int m = plan->list_count[CLS_MFMA][a];
        const int start = plan->list_start[CLS_MFMA][a];
        for (int r = 0; r < m; ++r, ++pair) {
            if (pair % (int)gridDim.x != (int)blockIdx.x) continue;
            const int slot = plan->perm[start + r];
            for (int i = threadIdx.x; i < I; i += kThreads) {
                float g = 0.0f, u = 0.0f;
                for (int s = 0; s < S; ++s) {
                    const float* part = p.partial + ((int64_t)s * p.slot_cap + slot) * 2 * I;
                    g += part[i];
                    u += part[I + i];
                }
                store_act<DT_BF16>(p.h, (int64_t)slot * I + i, silu_mul(g, u));
            }
        }
    }
}

// ------------------------------------------------------------------ down

// One unit per workgroup: NT 16-row tiles of one expert's down rows over the
// K range of split s, the four waves taking its K blocks in turn.
template <int WDT, int NT>
__global__ __launch_bounds__(kThreads) void down_mfma_kernel(ExpertArgs p) {
    typedef WFrag<WDT> F;
    __shared__ float red[kWaves][NT][kWave * 4];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int ln = lane & 15, lg = lane >> 4;
    const int H = p.H, I = p.I;
    const DevPlan* plan = p.plan;
    const int S = p.split_k;
    constexpr int kRows = 16 * NT;
    const int blocks = H / kRows;
    const int units = plan->n_list[CLS_MFMA] * blocks * S;
    const int nkb = I / kKB;
    constexpr int kWB = WDT == DT_FP8 ? 1 : 2;

    for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int s = unit % S;
        const int rest = unit / S;
        const int blk = rest % blocks;
        const int a = rest / blocks;
        const int e = plan->list_expert[CLS_MFMA][a];
        const int start = plan->list_start[CLS_MFMA][a];
        const int m = plan->list_count[CLS_MFMA][a];
        const int n0 = blk * kRows;
        const int kb0 = s * nkb / S, kb1 = (s + 1) * nkb / S;
        const char* wexp = (const char*)p.w_down + (int64_t)e * H * I * kWB;

        for (int mp = 0; mp < m; mp += 16) {
            const uint16_t* arow = nullptr;
            if (mp + ln < m) {
                const int slot = plan->perm[start + mp + ln];
                arow = (const uint16_t*)p.h + (int64_t)slot * I;
            }
            f32x4 acc[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 2
            for (int kb = kb0 + wave; kb < kb1; kb += kWaves) {
                const int64_t k = (int64_t)kb * kKB;
                u32x4 w[NT][F::kLoads];
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    F::load(wexp + (int64_t)(n0 + 16 * t + ln) * I * kWB, k, lg, w[t]);
                u32x4 af[4];
                load_act_frag<WDT>(arow, k, lg, af);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int t = 0; t < NT; ++t) acc[t] = mfma16(af[q], F::op(w[t], q), acc[t]);
            }

            __syncthreads();
#pragma unroll
            for (int t = 0; t < NT; ++t) *(f32x4*)&red[wave][t][lane * 4] = acc[t];
            __syncthreads();
            const int li = threadIdx.x >> 2, r = threadIdx.x & 3;
            const int row = mp + 4 * (li >> 4) + r;
            if (row < m) {
                const int slot = plan->perm[start + row];
                float* dst = S == 1 ? p.y : p.partial + (int64_t)s * p.slot_cap * H;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int n = n0 + 16 * t + (li & 15);
                    const float sd = p.s_d ? p.s_d[(int64_t)e * H + n] : 1.0f;
                    dst[(int64_t)slot * H + n] = reduce_waves<NT>(red, t) * sd;
                }
            }
        }
    }
}

// y[slot, n] = sum_s partial[s][slot][n] for the slots of MFMA experts, in
// the order s = 0, 1, ...
__global__ __launch_bounds__(kThreads) void down_reduce_kernel(ExpertArgs p) {
    const DevPlan* plan = p.plan;
    const int H = p.H, S = p.split_k;
    const int n_exp = plan->n_list[CLS_MFMA];
    int pair = 0;
    for (int a = 0; a < n_exp; ++a) {
        const int m = plan->list_count[CLS_MFMA][a];
        const int start = plan->list_start[CLS_MFMA][a];
        for (int r = 0; r < m; ++r, ++pair) {
            if (pair % (int)gridDim.x != (int)blockIdx.x) continue;
            const int slot = plan->perm[start + r];
            for (int n = threadIdx.x; n < H; n += kThreads) {
                float v = 0.0f;
                for (int s = 0; s < S; ++s) v += p.partial[((int64_t)s * p.slot_cap + slot) * H + n];
                p.y[(int64_t)slot * H + n] = v;
            }
        }
    }
}

constexpr int kNT = 2;  // 32 output rows per unit

int grid_for(int units) { return units < 1 ? 1 : (units < 8192 ? units : 8192); }

int reduce_grid() { return 512; }

}  // namespace

// max_experts: an upper bound on the MFMA list (sizes the grids).  Weight
// types: DT_BF16 or DT_FP8, with bf16 activations.  I and H must be
// multiples of 128 and of 16 * kNT.
hipError_t launch_gate_up_mfma(const ExpertArgs& a, int wdt, int max_rows, int max_experts,
                               hipStream_t s) {
    (void)max_rows;
    const int grid = grid_for(max_experts * (a.I / (16 * kNT)) * a.split_k);
    if (wdt == DT_FP8) gate_up_mfma_kernel<DT_FP8, kNT><<<grid, kThreads, 0, s>>>(a);
    else gate_up_mfma_kernel<DT_BF16, kNT><<<grid, kThreads, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.split_k == 1) return e;
    gate_up_reduce_kernel<<<reduce_grid(), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_down_mfma(const ExpertArgs& a, int wdt, int max_rows, int max_experts,
                            hipStream_t s) {
    (void)max_rows;
    const int grid = grid_for(max_experts * (a.H / (16 * kNT)) * a.split_k);
    if (wdt == DT_FP8) down_mfma_kernel<DT_FP8, kNT><<<grid, kThreads, 0, s>>>(a);
    else down_mfma_kernel<DT_BF16, kNT><<<grid, kThreads, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.split_k == 1) return e;
    down_reduce_kernel<<<reduce_grid(), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
