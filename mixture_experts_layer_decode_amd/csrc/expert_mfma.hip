// expert_mfma.hip -- split-K grouped GEMM on the gfx950 matrix cores for
// experts that several rows of the batch are routed to.
//
// ailookout.news, "vLLM speeds up Kimi K3 up to 1.9x on NVIDIA GB300 with
// agent-assisted kernels", section "How the specialised decode path works":
// the GB300 path picks its kernels from the batch size, with split-K
// kernels for batches beyond two rows.  Here the choice is made per expert, on the
// device, from the number of rows routed to it (the routing plan's MFMA list).
//
// The work is still bound by HBM (about m flop per weight byte for m rows,
// against a ridge near 310), so the matrix cores are there to keep the VALU
// and LDS out of the way as m grows, not to be saturated.  An M tile of 16
// rows is padded (with copies of the expert's last row, whose products are
// never used); the padding costs matrix-core cycles only.
//
// Instruction: v_mfma_f32_16x16x32_bf16, D[16x16] += A[16x32] * B[32x16].
//   A (activations): lane l holds row l%16, K elements 8*(l/16) .. +8;
//   B (weights):     lane l holds column l%16, K elements 8*(l/16) .. +8;
//   D:               lane l holds rows 4*(l/16) + i (i = 0..3), column l%16.
// MFMA q of a K block of 128 elements takes elements 32q + 8g .. +8 from
// lane group g = l/16, for the weights (read back from LDS, see the weight
// tiles below) and for the activations alike.
//
// fp8 (OCP e4m3) weights are converted to bf16 after the LDS read, which is
// exact; the per-output-row scale multiplies the fp32 accumulator.
//
// Work units: (active expert, block of 32 output rows -- 16 gate + 16 up
// rows, or 32 down rows (64 for fp8) --, K split s), walked by the
// workgroups (one unit each when the grid holds them all; a wave loads the
// next unit's first weights while it finishes the current one).  Within a unit
// the four waves split K among themselves and their partial sums are added
// through LDS in a fixed order.  With split_k == 1 the epilogue is applied
// directly (SwiGLU into h, or the scaled down projection into y); otherwise
// each split writes fp32 partial sums [s][slot][cols] that a later pass adds
// in the fixed order s = 0, 1, ..., so results do not depend on scheduling.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

constexpr int kKB = 128;  // K elements per block step (4 MFMAs of K = 32)
constexpr int kXcdChunk = 16;  // units dealt to an XCD at a time (xcd_walk)

// ----------------------------------------------------------- weight tiles
//
// A wave works on a tile of 32 weight rows x one K block of 128 elements: 16
// gate rows and the matching 16 up rows, or 32 (fp8: 64) down rows.  The tile is read
// from HBM with fully contiguous 1 KB load instructions (bf16: 4 rows x 256
// bytes, fp8: 8 rows x 128 bytes), written to the wave's own LDS region (rows
// padded by 16 bytes against bank conflicts) and read back in the MFMA
// operand layout.  Only the wave that wrote a region reads it, so no
// workgroup barrier is involved; the next K block's loads are issued (after
// the current block's activations) before the current block's LDS reads and
// MFMAs, so they overlap.
template <int WDT, int ROWS> struct Tile {
    static constexpr int kWB = WDT == DT_FP8 ? 1 : 2;      // bytes per element
    static constexpr int kRowBytes = kKB * kWB;             // one K block of a row
    static constexpr int kStride = kRowBytes + 16;          // padded LDS row
    static constexpr int kLanesPerRow = kRowBytes / 16;
    static constexpr int kRowsPerLoad = kWave / kLanesPerRow;
    static constexpr int kRows = ROWS;
    static constexpr int kTiles = ROWS / 16;                // 16 x 16 MFMA output tiles
    static constexpr int kLoads = kRows / kRowsPerLoad;      // bf16 32 rows: 8, fp8: 4 or 8
    static constexpr int kBytes = kRows * kStride;          // LDS per wave
};

// Output rows of one unit: 32 (16 gate + 16 up rows, or 32 down rows), and 64
// down rows for fp8 weights, whose rows are half as long, so that a down unit
// streams the same 128 KB as a bf16 one (at 16 rows over four fp8 layers the
// 64 KB units streamed at 6.1 TB/s against gate/up's 6.6).
constexpr int unit_rows(int wdt, bool gate_up) { return !gate_up && wdt == DT_FP8 ? 64 : 32; }

// LDS words of one MFMA B operand: 8 elements of row n at element offset o.
__device__ __forceinline__ bf16x8 lds_operand_bf16(const unsigned char* row, int o) {
    return __builtin_bit_cast(bf16x8, *(const u32x4*)(row + 2 * o));
}
__device__ __forceinline__ bf16x8 lds_operand_fp8(const unsigned char* row, int o) {
    // eight e4m3 codes -> eight bf16, exactly: through fp32 (v_cvt_pk_f32_fp8),
    // keeping the upper halves.  The direct fp8 -> bf16 conversion with a unit
    // scale (v_cvt_scalef32_pk_bf16_fp8) dropped the last mantissa bit of half
    // of the codes when checked on gfx950.
    const uint2 w = *(const uint2*)(row + o);
    uint32_t a0, a1, b0, b1;
    fp8x4_to_bf16x4(w.x, a0, a1);
    fp8x4_to_bf16x4(w.y, b0, b1);
    return __builtin_bit_cast(bf16x8, u32x4{a0, a1, b0, b1});
}

// Activation fragment of one 16-row M tile for one K block: lane l supplies
// row l%16, elements 32q + 8(l/16) .. +8 for MFMA q.  Lanes of the tile's
// padding rows load a real row too (the expert's last one): the rows of an
// MFMA product are independent and the epilogue writes only real rows, so
// their products are never used, and no lane writes zeros into registers
// whose loads may still be in flight (which would wait for every load).
__device__ __forceinline__ void load_act_frag(const uint16_t* row, int64_t k, int g,
                                              u32x4 (&a)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = load16(row + k + 32 * q + 8 * g);
}

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}

// LDS writes and reads of this wave are ordered with respect to each other.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Sum the four waves' accumulator tiles (kept in LDS as red[wave][tile][lane *
// 4 + r]) in the order wave 0, 1, 2, 3: thread t of the workgroup gets
// element t of each tile, i.e. D row 4 * ((t / 4) / 16) + t % 4, column
// (t / 4) % 16 of that tile.
template <int NT>
__device__ __forceinline__ float reduce_waves(const float (*red)[NT][kWave * 4], int tile) {
    const int t = threadIdx.x;
    return ((red[0][tile][t] + red[1][tile][t]) + red[2][tile][t]) + red[3][tile][t];
}

// A workgroup walks its units (one when the grid holds them all).  GATE_UP:
// 16 gate rows (tile 0) and the matching 16 up rows (tile 1) of one expert,
// K = H, activations x, SwiGLU epilogue into h.  Otherwise: 32 down rows (64
// for fp8; tiles 0 .. NT-1), K = I, activations h, epilogue into y.  The four waves take the unit's K blocks in turn (wave w: blocks w,
// w + 4, ...) over the K range of split s; their accumulators are added
// through LDS in a fixed order.
template <int WDT, bool GATE_UP, int ROWS>
__global__ __launch_bounds__(kThreads) void expert_mfma_kernel(ExpertArgs p) {
    typedef Tile<WDT, ROWS> T;
    constexpr int HALF = ROWS / 2;  // gate/up: gate rows (then as many up rows) per unit
    constexpr int NT = T::kTiles;
    __shared__ __align__(16) unsigned char stage[kWaves][T::kBytes];
    __shared__ float red[kWaves][NT][kWave * 4];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int ln = lane & 15, lg = lane >> 4;
    const int H = p.H, I = p.I;
    const int K = GATE_UP ? H : I;
    const DevPlan* plan = p.plan;
    const int S = p.split_k;
    const int blocks = GATE_UP ? I / HALF : H / T::kRows;
    const int units = plan->n_list[CLS_MFMA] * blocks * S;
    const int nkb = K / kKB;
    unsigned char* my = stage[wave];
    // this lane's row and byte column in every load instruction
    const int lrow = lane / T::kLanesPerRow, lcol = (lane % T::kLanesPerRow) * 16;

    // chunks of 16 units per XCD, against the plain order, interleaved in
    // one process: bf16 8 rows 507.8 -> 492.0 us per layer, 64 rows 7855 ->
    // 7776; fp8 16 rows 770.2 -> 767.0, 64 rows 1846 -> 1844 (one
    // contiguous range per XCD: bf16 493.3 / 7781, but fp8 798.7 / 1984)
    const XcdWalk walk = xcd_walk(kXcdChunk);
    const int64_t row_bytes = (int64_t)K * T::kWB;
    // this lane's part of every load instruction, relative to a unit's first
    // row: everything else is uniform across the wave
    const uint32_t loff = (uint32_t)(lrow * row_bytes) + lcol;
    // tile rows of load instruction i, relative to the unit's first row
    // (gate/up: the first HALF tile rows are gate rows, the next HALF the up
    // rows I below)
    auto irow = [&](int i) -> int64_t {
        const int r0 = i * T::kRowsPerLoad;
        return GATE_UP ? (r0 < HALF ? r0 : (int64_t)I + (r0 - HALF)) : r0;
    };
    // A unit of the walk: its split, block, expert and rows (unit >= units:
    // past the end).
    struct Item {
        int unit, s, blk, e, start, m, kb0, kb1;
        const unsigned char* w;  // the unit's first weight row
    };
    auto decode = [&](int unit) -> Item {
        Item it;
        it.unit = unit;
        if (unit >= units) return it;
        it.s = unit % S;
        const int rest = unit / S;
        it.blk = rest % blocks;
        const int a = rest / blocks;
        it.e = plan->list_expert[CLS_MFMA][a];
        it.start = plan->list_start[CLS_MFMA][a];
        it.m = plan->list_count[CLS_MFMA][a];
        it.kb0 = it.s * nkb / S;
        it.kb1 = (it.s + 1) * nkb / S;
        it.w = (const unsigned char*)(GATE_UP ? p.w_gate_up : p.w_down) +
               (GATE_UP ? (int64_t)it.e * 2 * I + it.blk * HALF
                        : (int64_t)it.e * H + it.blk * T::kRows) * row_bytes;
        return it;
    };
    // the weights of this wave's K block kb of a unit
    u32x4 wv[T::kLoads];
    auto load_block = [&](const Item& it, int kb) {
#pragma unroll
        for (int i = 0; i < T::kLoads; ++i)
            wv[i] = load_weights16(it.w + irow(i) * row_bytes + (int64_t)kb * T::kRowBytes + loff);
    };

    // The workgroup walks its units; while a wave works on its last K block
    // of a work item (a unit's 16-row tile), the first block of the next item
    // -- the unit's next row tile, or the next unit of the walk -- is already
    // being loaded, so the weight stream does not stop at item boundaries.
    int pos = walk.first;
    Item it = decode(walk.unit(pos));
    bool have = false;  // wv holds this wave's first block of the current item
    while (it.unit < units) {
        pos += walk.step;
        const Item nx = decode(walk.unit(pos));
        for (int mp = 0; mp < it.m; mp += 16) {
            // this lane's activation row (A operand): row mp + ln of the
            // expert, or its last row for the tile's padding lanes
            const int ar = mp + ln < it.m ? mp + ln : it.m - 1;
            const int aslot = plan->perm[it.start + ar];
            const uint16_t* arow = GATE_UP ? (const uint16_t*)p.x + (int64_t)(aslot / p.k) * p.x_stride
                                           : (const uint16_t*)p.h + (int64_t)aslot * I;
            f32x4 acc[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

            int kb = it.kb0 + wave;
            if (!have && kb < it.kb1) load_block(it, kb);
            have = false;
            // this wave's K block kb: its weights (in wv) go to the wave's LDS
            // region, its activations are loaded, then -- through `next` --
            // the weights of the wave's next block are loaded into wv, then
            // the products.  A wave's loads complete in the order they were
            // issued, so the products wait only for the activations, issued
            // before the next weights, which stay in flight meanwhile.
            auto step = [&](int kb, auto next) {
                wave_lds_fence();  // the previous block's operand reads are done
#pragma unroll
                for (int i = 0; i < T::kLoads; ++i)
                    *(u32x4*)(my + (i * T::kRowsPerLoad + lrow) * T::kStride + lcol) = wv[i];
                u32x4 af[4];
                load_act_frag(arow, (int64_t)kb * kKB, lg, af);
                next();
                wave_lds_fence();  // this block's tile is in LDS
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const unsigned char* row = my + (16 * t + ln) * T::kStride;
                        const bf16x8 b = WDT == DT_FP8 ? lds_operand_fp8(row, 32 * q + 8 * lg)
                                                       : lds_operand_bf16(row, 32 * q + 8 * lg);
                        acc[t] = mfma16(af[q], b, acc[t]);
                    }
            };
            // every block but the wave's last of this item: the next block of
            // the item, loaded unconditionally, so that the compiler counts
            // the loads in flight exactly
            for (; kb + kWaves < it.kb1; kb += kWaves) step(kb, [&] { load_block(it, kb + kWaves); });
            // the last: the first block of the next item -- this unit's next
            // row tile, or the next unit of the walk -- if there is one
            if (kb < it.kb1)
                step(kb, [&] {
                    if (mp + 16 < it.m) {
                        load_block(it, it.kb0 + wave);
                        have = true;
                    } else if (nx.unit < units && nx.kb0 + wave < nx.kb1) {
                        load_block(nx, nx.kb0 + wave);
                        have = true;
                    }
                });

            __syncthreads();  // the previous pass's reads of red are done
#pragma unroll
            for (int t = 0; t < NT; ++t) *(f32x4*)&red[wave][t][lane * 4] = acc[t];
            __syncthreads();
            const int li = threadIdx.x >> 2, r = threadIdx.x & 3;
            const int row = mp + 4 * (li >> 4) + r;
            if (row < it.m) {
                const int slot = plan->perm[it.start + row];
                if (GATE_UP) {
                    // tiles 0 .. NT/2-1 hold gate rows, NT/2 .. NT-1 the matching up rows
#pragma unroll
                    for (int t = 0; t < NT / 2; ++t) {
                        const int col = it.blk * HALF + 16 * t + (li & 15);
                        float sg = 1.0f, su = 1.0f;
                        if (p.s_gu) {
                            sg = p.s_gu[(int64_t)it.e * 2 * I + col];
                            su = p.s_gu[(int64_t)it.e * 2 * I + I + col];
                        }
                        const float g = reduce_waves<NT>(red, t) * sg;
                        const float u = reduce_waves<NT>(red, t + NT / 2) * su;
                        if (S == 1) {
                            store_act<DT_BF16>(p.h, (int64_t)slot * I + col, silu_mul(g, u));
                        } else {
                            float* part = p.partial + ((int64_t)it.s * p.slot_cap + slot) * 2 * I;
                            part[col] = g;
                            part[I + col] = u;
                        }
                    }
                } else {
                    float* dst = S == 1 ? p.y : p.partial + (int64_t)it.s * p.slot_cap * H;
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const int n = it.blk * T::kRows + 16 * t + (li & 15);
                        const float sd = p.s_d ? p.s_d[(int64_t)it.e * H + n] : 1.0f;
                        dst[(int64_t)slot * H + n] = reduce_waves<NT>(red, t) * sd;
                    }
                }
            }
        }
        it = nx;
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

// Workgroups for an upper bound of `units` (the host does not know how many
// distinct experts the routing selected).  Workgroups past the real unit
// count exit at once but still cost their dispatch, and workgroups that walk
// several units leave a ragged last round, so the cap grows with the rows:
// interleaved in one process, cap 8192 / 16384 / 32768 at 8 bf16 rows 491.6 /
// 495.9 / 505.7 us per layer, at 64 rows 7779.7 / 7733.2 / 7706.6; 16 rows of
// one fp8 layer 779.2 / 765.7 / 777.1.
int grid_for(int units, int rows) {
    const int cap = rows <= 8 ? 8192 : rows <= 32 ? 16384 : 32768;
    return units < 1 ? 1 : (units < cap ? units : cap);
}

int reduce_grid() { return 512; }

}  // namespace

// max_experts: an upper bound on the MFMA list (sizes the grids).  Weight
// types: DT_BF16 or DT_FP8, with bf16 activations.  H and I must be multiples
// of 128 (and I of 16, H of 32, or of 64 with fp8 weights).
hipError_t launch_gate_up_mfma(const ExpertArgs& a, int wdt, int max_rows, int max_experts,
                               hipStream_t s) {
    const int grid = grid_for(max_experts * (a.I / (unit_rows(wdt, true) / 2)) * a.split_k, max_rows);
    if (wdt == DT_FP8)
        expert_mfma_kernel<DT_FP8, true, unit_rows(DT_FP8, true)><<<grid, kThreads, 0, s>>>(a);
    else
        expert_mfma_kernel<DT_BF16, true, unit_rows(DT_BF16, true)><<<grid, kThreads, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.split_k == 1) return e;
    gate_up_reduce_kernel<<<reduce_grid(), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_down_mfma(const ExpertArgs& a, int wdt, int max_rows, int max_experts,
                            hipStream_t s) {
    const int grid = grid_for(max_experts * (a.H / unit_rows(wdt, false)) * a.split_k, max_rows);
    if (wdt == DT_FP8)
        expert_mfma_kernel<DT_FP8, false, unit_rows(DT_FP8, false)><<<grid, kThreads, 0, s>>>(a);
    else
        expert_mfma_kernel<DT_BF16, false, unit_rows(DT_BF16, false)><<<grid, kThreads, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.split_k == 1) return e;
    down_reduce_kernel<<<reduce_grid(), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
