// expert_gemv.hip -- weight-streaming GEMV kernels for experts with few rows.
//
// ailookout.news, "vLLM speeds up Kimi K3 up to 1.9x on NVIDIA GB300 with
// agent-assisted kernels", section "How the specialised decode path works":
// the GB300 path picks its kernels from the batch size, GEMV-style ones for
// one- and two-row batches, because decoding for a single user is bound by
// the rate at which weights come out of memory.  These kernels are the GEMV
// side: each active expert's
// weight rows are read exactly once, as contiguous 16-byte-per-lane loads
// (every wave-wide load instruction covers 1 KB of one row), and applied to
// all (at most a few) rows routed to that expert, whose activations sit in
// LDS.
//
// Work is split into units of (active expert, block of output rows) and the
// grid walks the unit list the router kernel left in device memory, so the
// host never needs to know how many experts were selected.
//
// gate_up: for each unit, rows i of the gate and up projections of expert e
//   h[slot, i] = round_act( silu(s_g * <Wg[e,i,:], x_b>) * (s_u * <Wu[e,i,:], x_b>) )
// down: y[slot, n] = s_d * <Wd[e,n,:], h[slot,:]>   (fp32 workspace)
// All dot products accumulate in fp32 and are summed across the wave by a
// fixed butterfly, so results are reproducible run to run.

#include "moe_device.h"
#include "moe_internal.h"
#include "select_device.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// Copy the activation rows of `rows` slots (listed in perm) into LDS.
// src row of slot s is base + (s / div) * stride; `len` elements each.
template <typename T>
__device__ __forceinline__ void stage_rows(T* dst, const void* base, int64_t stride,
                                           const int* perm, int rows, int div, int len) {
    constexpr int kPerVec = 16 / sizeof(T);
    for (int r = 0; r < rows; ++r) {
        const int src_row = perm[r] / div;
        const T* src = (const T*)base + (int64_t)src_row * stride;
        for (int c = threadIdx.x * kPerVec; c < len; c += kThreads * kPerVec)
            *(u32x4*)(dst + (int64_t)r * len + c) = load16(src + c);
    }
}

// ------------------------------------------------------------- gate / up

// The gate/up rows of one unit (block blk of expert e, rows of x listed by
// slot in slots[0..m)): rows i of the gate and up projections for the unit's
// row pairs, SwiGLU into h.  xs: LDS for MG rows of x.  STAGED: the batch's
// one row is already in xs (m = 1): no staging and no barrier.
template <int WDT, int ACT, int MG, int U, int PW, bool STAGED = false>
__device__ __forceinline__ void gate_up_unit(const ExpertArgs& p, typename Storage<ACT>::type* xs,
                                             int e, int blk, const int* slots, int m) {
    typedef typename Storage<WDT>::type wt;
    typedef typename Storage<ACT>::type at;
    constexpr int VEC = vec_elems<WDT>();
    typedef WOps<WDT> Ops;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int H = p.H, I = p.I;
    constexpr int kPairsPerUnit = kWaves * PW;
    const int nv = H / (kWave * VEC);  // wave-wide loads per weight row
    const wt* wexp = (const wt*)p.w_gate_up + (int64_t)e * 2 * I * H;

    for (int r0 = 0; r0 < m; r0 += MG) {
        const int mg = min(MG, m - r0);
        if constexpr (!STAGED) {
            __syncthreads();  // LDS reuse across passes and units
            stage_rows<at>(xs, p.x, p.x_stride, slots + r0, mg, p.k, H);
            __syncthreads();
        }

        for (int q = 0; q < PW; ++q) {
            const int i = blk * kPairsPerUnit + wave * PW + q;
            if (i >= I) break;
            const wt* rg = wexp + (int64_t)i * H;
            const wt* ru = wexp + (int64_t)(I + i) * H;
            float ag[MG], au[MG];
#pragma unroll
            for (int r = 0; r < MG; ++r) ag[r] = au[r] = 0.0f;

            for (int t0 = 0; t0 < nv; t0 += U) {
                u32x4 vg[U], vu[U];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (t0 + u < nv) {
                        const int off = ((t0 + u) * kWave + lane) * VEC;
                        vg[u] = load_weights16(rg + off);
                        vu[u] = load_weights16(ru + off);
                    }
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (t0 + u < nv) {
                        const int off = ((t0 + u) * kWave + lane) * VEC;
                        uint32_t og[Ops::kOps], ou[Ops::kOps];
                        Ops::unpack(vg[u], og);
                        Ops::unpack(vu[u], ou);
#pragma unroll
                        for (int r = 0; r < MG; ++r)
                            if (r < mg) {
                                ag[r] = Ops::dot(og, xs + (int64_t)r * H + off, ag[r]);
                                au[r] = Ops::dot(ou, xs + (int64_t)r * H + off, au[r]);
                            }
                    }
            }

            float sg = 1.0f, su = 1.0f;
            if (p.s_gu) {
                sg = p.s_gu[(int64_t)e * 2 * I + i];
                su = p.s_gu[(int64_t)e * 2 * I + I + i];
            }
#pragma unroll
            for (int r = 0; r < MG; ++r)
                if (r < mg) {
                    const float g = wave_sum(ag[r]) * sg;
                    const float u = wave_sum(au[r]) * su;
                    if (lane == 0) store_act<ACT>(p.h, (int64_t)slots[r0 + r] * I + i, silu_mul(g, u));
                }
        }
    }
}

// The batch's one row of x (row 0, H elements) into xs, by the threads from
// `first` on.
template <typename T>
__device__ __forceinline__ void stage_row0(T* xs, const void* x, int H, int first) {
    constexpr int kPerVec = 16 / sizeof(T);
    for (int c = ((int)threadIdx.x - first) * kPerVec; c < H; c += (kThreads - first) * kPerVec)
        *(u32x4*)(xs + c) = load16((const T*)x + c);
}

// MG: most activation rows per pass; U: 16-byte loads per weight row in
// flight per step; PW: gate/up row pairs per wave per unit.  Each unit
// stages its rows of x and waits at a barrier, also at batch 1: staging the
// one row once per workgroup and streaming the units without barriers was
// slower (236.3 against 233.3 us per batch-1 layer, interleaved in one
// process), as the waves of a workgroup drift apart in the weight rows.
template <int WDT, int ACT, int MG, int U, int PW>
__global__ __launch_bounds__(kThreads) void gate_up_gemv_kernel(ExpertArgs p) {
    typedef typename Storage<ACT>::type at;
    extern __shared__ __align__(16) unsigned char smem[];
    at* xs = (at*)smem;  // [MG][H]
    constexpr int kPairsPerUnit = kWaves * PW;
    const int units_per_expert = (p.I + kPairsPerUnit - 1) / kPairsPerUnit;
    const DevPlan* plan = p.plan;
    const int units = plan->n_list[CLS_GEMV] * units_per_expert;

    // units dealt to the XCDs 16 at a time: at batch 1, interleaved in one
    // process, 220.1 -> 219.3 us per layer (64 at a time: 219.6)
    const XcdWalk walk = xcd_walk(16);
    for (int pos = walk.first;; pos += walk.step) {
        const int unit = walk.unit(pos);
        if (unit >= units) break;
        const int a = unit / units_per_expert;
        const int blk = unit - a * units_per_expert;
        gate_up_unit<WDT, ACT, MG, U, PW>(p, xs, plan->list_expert[CLS_GEMV][a], blk,
                                          plan->perm + plan->list_start[CLS_GEMV][a],
                                          plan->list_count[CLS_GEMV][a]);
    }
}

// Batch 1, selection included.  Wave 0 of every workgroup takes the top k of
// the router's logits (the same exact selection as the top-k kernel,
// select_topk) into LDS; workgroup 0 also computes the routing weights and
// writes the routing outputs and the plan (every expert one row, listed under
// CLS_GEMV in selection order), which later kernels read across the kernel
// boundary.  Then the workgroup walks the gate/up units of the k experts as
// gate_up_gemv_kernel does (slot j = choice j, x row 0, staged once by the
// other waves while wave 0 selects).  This saves the top-k launch, but every
// workgroup selects: at batch 1 on the full bf16 layer, interleaved in one
// process, the router stage fell by 5.6 us and gate/up grew by 9.6 to 18.4 us
// (grids of 1024 to 8192 workgroups: 239.4 to 246.3 against 233.3 us per
// layer), so it is an option, off by default.  PL: logits per lane (E <= 64 *
// PL).
template <int WDT, int ACT, int U, int PW, int PL>
__global__ __launch_bounds__(kThreads) void gate_up_select1_kernel(ExpertArgs p, SelectArgs q) {
    typedef typename Storage<ACT>::type at;
    extern __shared__ __align__(16) unsigned char smem[];
    at* xs = (at*)smem;  // [1][H]
    __shared__ double s_cv[kWave];
    __shared__ int s_ce[kWave];
    __shared__ double s_sv[kMaxTopk];
    __shared__ int s_se[kMaxTopk];
    __shared__ int s_sel[kMaxTopk];   // the selection, in order
    __shared__ int s_slot[kMaxTopk];  // slot of choice j: j
    const int lane = threadIdx.x & (kWave - 1);
    const int k = p.k;
    // waves 1.. stage the row of x while wave 0 selects
    if (threadIdx.x >= kWave) stage_row0<at>(xs, p.x, p.H, kWave);
    if (threadIdx.x < kWave) {
        double v[PL];
#pragma unroll
        for (int t = 0; t < PL; ++t) {
            const int ee = lane + t * kWave;
            v[t] = ee < q.E ? q.logits[ee] : 0.0;
            if (q.bias && ee < q.E) v[t] += (double)q.bias[ee];
            v[t] += 0.0;  // -0 -> +0: equal logits have equal keys
        }
        double sel_v = 0.0;
        int sel_e = 0;
        select_topk<PL>(v, q.E, k, s_cv, s_ce, s_sv, s_se, sel_v, sel_e);
        if (lane < k) {
            s_sel[lane] = sel_e;
            s_slot[lane] = lane;
        }
        if (blockIdx.x == 0) {
            const float wj = routing_weight(sel_v, k, q.score_fn);
            DevPlan* plan = q.plan;
            if (lane < k) {
                q.topk_idx[lane] = sel_e;
                q.topk_w[lane] = wj;
                if (q.user_idx) q.user_idx[lane] = sel_e;
                if (q.user_w) q.user_w[lane] = wj;
                plan->perm[lane] = lane;
                plan->list_expert[CLS_GEMV][lane] = sel_e;
                plan->list_start[CLS_GEMV][lane] = lane;
                plan->list_count[CLS_GEMV][lane] = 1;
            }
            if (lane == 0) {
                plan->num_slots = k;
                plan->num_active = k;
                plan->n_list[CLS_GEMV] = k;
                plan->n_list[CLS_MFMA] = 0;
                plan->max_rows = 1;
            }
        }
    }
    __syncthreads();  // the selection and the row of x are in LDS

    constexpr int kPairsPerUnit = kWaves * PW;
    const int units_per_expert = (p.I + kPairsPerUnit - 1) / kPairsPerUnit;
    const int units = k * units_per_expert;
    const XcdWalk walk = xcd_walk(16);
    for (int pos = walk.first;; pos += walk.step) {
        const int unit = walk.unit(pos);
        if (unit >= units) break;
        const int a = unit / units_per_expert;
        const int blk = unit - a * units_per_expert;
        gate_up_unit<WDT, ACT, 1, U, PW, true>(p, xs, s_sel[a], blk, s_slot + a, 1);
    }
}

// ------------------------------------------------------------------ down

// R: output rows processed together per wave; RW: output rows per wave per
// unit (a multiple of R); U: 16-byte loads per row in flight per step.
template <int WDT, int ACT, int MG, int U, int R, int RW>
__global__ __launch_bounds__(kThreads) void down_gemv_kernel(ExpertArgs p) {
    typedef typename Storage<WDT>::type wt;
    typedef typename Storage<ACT>::type at;
    constexpr int VEC = vec_elems<WDT>();
    typedef WOps<WDT> Ops;
    extern __shared__ __align__(16) unsigned char smem[];
    at* hs = (at*)smem;  // [MG][I]

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int H = p.H, I = p.I;
    constexpr int kRowsPerUnit = kWaves * RW;
    const int units_per_expert = (H + kRowsPerUnit - 1) / kRowsPerUnit;
    const DevPlan* plan = p.plan;
    const int units = plan->n_list[CLS_GEMV] * units_per_expert;
    const int nv = I / (kWave * VEC);

    for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int a = unit / units_per_expert;
        const int blk = unit - a * units_per_expert;
        const int e = plan->list_expert[CLS_GEMV][a];
        const int start = plan->list_start[CLS_GEMV][a];
        const int m = plan->list_count[CLS_GEMV][a];
        const wt* wexp = (const wt*)p.w_down + (int64_t)e * H * I;

        for (int r0 = 0; r0 < m; r0 += MG) {
            const int mg = min(MG, m - r0);
            __syncthreads();
            stage_rows<at>(hs, p.h, I, plan->perm + start + r0, mg, 1, I);
            __syncthreads();

            for (int n0 = blk * kRowsPerUnit + wave * RW; n0 < blk * kRowsPerUnit + (wave + 1) * RW;
                 n0 += R) {
                if (n0 >= H) break;
                float acc[R][MG];
#pragma unroll
                for (int q = 0; q < R; ++q)
#pragma unroll
                    for (int r = 0; r < MG; ++r) acc[q][r] = 0.0f;

                for (int t0 = 0; t0 < nv; t0 += U) {
                    u32x4 v[R][U];
#pragma unroll
                    for (int q = 0; q < R; ++q)
#pragma unroll
                        for (int u = 0; u < U; ++u)
                            if (t0 + u < nv && n0 + q < H)
                                v[q][u] = load_weights16(wexp + (int64_t)(n0 + q) * I +
                                                         ((t0 + u) * kWave + lane) * VEC);
#pragma unroll
                    for (int q = 0; q < R; ++q)
#pragma unroll
                        for (int u = 0; u < U; ++u)
                            if (t0 + u < nv && n0 + q < H) {
                                const int off = ((t0 + u) * kWave + lane) * VEC;
                                uint32_t o[Ops::kOps];
                                Ops::unpack(v[q][u], o);
#pragma unroll
                                for (int r = 0; r < MG; ++r)
                                    if (r < mg)
                                        acc[q][r] = Ops::dot(o, hs + (int64_t)r * I + off, acc[q][r]);
                            }
                }

#pragma unroll
                for (int q = 0; q < R; ++q) {
                    if (n0 + q >= H) break;
                    const float sd = p.s_d ? p.s_d[(int64_t)e * H + n0 + q] : 1.0f;
#pragma unroll
                    for (int r = 0; r < MG; ++r)
                        if (r < mg) {
                            const float yv = wave_sum(acc[q][r]) * sd;
                            if (lane == 0) {
                                const int slot = plan->perm[start + r0 + r];
                                p.y[(int64_t)slot * H + n0 + q] = yv;
                            }
                        }
                }
            }
        }
    }
}

// ------------------------------------------------------ one-row experts
//
// Down projection of experts with a single routed row (every expert at batch
// 1): the row of h is read once per unit straight into registers (I / 512
// 16-byte vectors per lane in bf16), each lane taking exactly the elements
// that meet its weight vectors, so no LDS staging or workgroup barrier
// precedes the weight stream.  NV: most 16-byte weight vectors per lane in
// one weight row (the row length is at most NV * 64 * VEC).

// 16-byte activation vectors that meet one 16-byte weight vector.
template <int WDT> constexpr int act_vecs() { return WDT == DT_FP8 ? 2 : 1; }

template <int WDT, int ACT, int NV>
__device__ __forceinline__ void load_act_row(const void* row, int nv, int lane,
                                             u32x4 (&a)[NV][act_vecs<WDT>()]) {
    typedef typename Storage<ACT>::type at;
    constexpr int VEC = vec_elems<WDT>();
    constexpr int kPer16 = 16 / (int)sizeof(at);
#pragma unroll
    for (int t = 0; t < NV; ++t)
#pragma unroll
        for (int v = 0; v < act_vecs<WDT>(); ++v)
            a[t][v] = t < nv ? load16((const at*)row + (t * kWave + lane) * VEC + v * kPer16)
                             : u32x4{0u, 0u, 0u, 0u};
}

template <int WDT, int ACT, int NV, int U, int R, int RW>
__global__ __launch_bounds__(kThreads) void down_gemv1_kernel(ExpertArgs p) {
    typedef typename Storage<WDT>::type wt;
    constexpr int VEC = vec_elems<WDT>();
    typedef WOps<WDT> Ops;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int H = p.H, I = p.I;
    constexpr int kRowsPerUnit = kWaves * RW;
    const int units_per_expert = (H + kRowsPerUnit - 1) / kRowsPerUnit;
    const DevPlan* plan = p.plan;
    const int units = plan->n_list[CLS_GEMV] * units_per_expert;
    const int nv = I / (kWave * VEC);

    for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int a = unit / units_per_expert;
        const int blk = unit - a * units_per_expert;
        const int e = plan->list_expert[CLS_GEMV][a];
        const int slot = plan->perm[plan->list_start[CLS_GEMV][a]];
        const wt* wexp = (const wt*)p.w_down + (int64_t)e * H * I;
        u32x4 hr[NV][act_vecs<WDT>()];
        load_act_row<WDT, ACT, NV>((const char*)p.h + (int64_t)slot * I *
                                                          (int64_t)sizeof(typename Storage<ACT>::type),
                                   nv, lane, hr);

        for (int n0 = blk * kRowsPerUnit + wave * RW; n0 < blk * kRowsPerUnit + (wave + 1) * RW;
             n0 += R) {
            if (n0 >= H) break;
            float acc[R];
#pragma unroll
            for (int q = 0; q < R; ++q) acc[q] = 0.0f;
#pragma unroll
            for (int t0 = 0; t0 < NV; t0 += U) {
                u32x4 v[R][U];
#pragma unroll
                for (int q = 0; q < R; ++q)
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        if (t0 + u < NV && t0 + u < nv && n0 + q < H)
                            v[q][u] = load_weights16(wexp + (int64_t)(n0 + q) * I +
                                                     ((t0 + u) * kWave + lane) * VEC);
#pragma unroll
                for (int q = 0; q < R; ++q)
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        if (t0 + u < NV && t0 + u < nv && n0 + q < H) {
                            uint32_t o[Ops::kOps];
                            Ops::unpack(v[q][u], o);
                            acc[q] = Ops::dotr(o, hr[t0 + u], acc[q]);
                        }
            }
#pragma unroll
            for (int q = 0; q < R; ++q) {
                if (n0 + q >= H) break;
                const float sd = p.s_d ? p.s_d[(int64_t)e * H + n0 + q] : 1.0f;
                const float yv = wave_sum(acc[q]) * sd;
                if (lane == 0) p.y[(int64_t)slot * H + n0 + q] = yv;
            }
        }
    }
}

// ------------------------------------------------------------- launchers

template <int WDT, int ACT, int MG>
hipError_t gate_up_mg(const ExpertArgs& a, int max_units, hipStream_t s) {
    constexpr int U = 7;
    // row pairs per wave, timed alone on 16 experts (7168 x 2048): with one
    // activation row, one pair for bf16 (133.9 us against 136.3 us with two,
    // whose larger units leave fewer workgroups to spread) and fp32 (266.2
    // against 269.8 us), two for fp8, whose rows are half as long (74.0
    // against 75.9 us); with more rows, two (bf16 at two rows: 145.7 against
    // 148.4 us)
    constexpr int PW = MG == 1 && WDT != DT_FP8 ? 1 : 2;
    const int units = ((a.I + kWaves * PW - 1) / (kWaves * PW)) * max_units;
    const int grid = units < 8192 ? units : 8192;
    const size_t lds = (size_t)MG * a.H * sizeof(typename Storage<ACT>::type);
    gate_up_gemv_kernel<WDT, ACT, MG, U, PW><<<grid, kThreads, lds, s>>>(a);
    return hipGetLastError();
}

// Batch 1 with the selection in the kernel: as gate_up_mg at one row (one
// row pair per wave for bf16 and fp32, two for fp8), over the k experts.
template <int WDT, int ACT, int PL>
hipError_t gate_up_select1_pl(const ExpertArgs& a, const SelectArgs& q, int grid, hipStream_t s) {
    constexpr int U = 7;
    constexpr int PW = WDT != DT_FP8 ? 1 : 2;
    const int units = ((a.I + kWaves * PW - 1) / (kWaves * PW)) * a.k;
    if (grid <= 0) grid = units < 8192 ? units : 8192;
    const size_t lds = (size_t)a.H * sizeof(typename Storage<ACT>::type);
    gate_up_select1_kernel<WDT, ACT, U, PW, PL><<<grid, kThreads, lds, s>>>(a, q);
    return hipGetLastError();
}

template <int WDT, int ACT>
hipError_t gate_up_select1_typed(const ExpertArgs& a, const SelectArgs& q, int grid,
                                 hipStream_t s) {
    const int pl = (q.E + kWave - 1) / kWave;
    if (pl <= 1) return gate_up_select1_pl<WDT, ACT, 1>(a, q, grid, s);
    if (pl <= 2) return gate_up_select1_pl<WDT, ACT, 2>(a, q, grid, s);
    if (pl <= 4) return gate_up_select1_pl<WDT, ACT, 4>(a, q, grid, s);
    if (pl <= 8) return gate_up_select1_pl<WDT, ACT, 8>(a, q, grid, s);
    if (pl <= 16) return gate_up_select1_pl<WDT, ACT, 16>(a, q, grid, s);
    return gate_up_select1_pl<WDT, ACT, 32>(a, q, grid, s);
}

template <int WDT, int ACT, int MG>
hipError_t down_mg(const ExpertArgs& a, int max_units, hipStream_t s) {
    constexpr int U = 4;
    constexpr int R = 4;
    constexpr int RW = 8;
    const int units = ((a.H + kWaves * RW - 1) / (kWaves * RW)) * max_units;
    const int grid = units < 8192 ? units : 8192;
    const size_t lds = (size_t)MG * a.I * sizeof(typename Storage<ACT>::type);
    down_gemv_kernel<WDT, ACT, MG, U, R, RW><<<grid, kThreads, lds, s>>>(a);
    return hipGetLastError();
}

// 16-byte weight vectors per lane in a row of `len` elements (len a multiple
// of 64 vectors): 16 for a bf16 row of 8192, 32 for an fp32 one.
template <int WDT> int row_vecs(int len) { return len / (kWave * vec_elems<WDT>()); }

// ------------------------------------------ one row, combine folded in
//
// Batch 1 with every expert on the GEMV kernels: the down projection of all
// k experts and the weighted combine + residual in one launch.  Workgroup: 8
// waves serving R = 4 consecutive output columns n; wave w takes the choices
// j = w, w + 8 (k <= 16) in turn.  For each, it streams rows n .. n + 3 of
// that expert's down matrix against the expert's row of h, held in
// registers, exactly as down_gemv1_kernel does (same per-lane order, same
// butterfly), so y_j[n] is bit-identical; the k values of each column meet in
// LDS and are combined in the order j = 0, 1, ... with the residual, as
// combine_kernel does: out[n] = x[n] + sum_j w_j y_j[n] in fp32, rounded
// once.  No y workspace is written.  Eight waves (rather than one per choice)
// let two workgroups share a CU at this kernel's register use, so one
// workgroup's start and drain overlap another's stream; this was about 13 us
// faster over the full layer's down projection than 16 waves.  Four columns
// per workgroup streamed faster than 2, 7 or 8 (the wider tiles hold more
// weight registers and leave fewer waves per CU).
constexpr int kFusedMaxK = kFusedCombineMaxK;
constexpr int kFusedCols = 4;
constexpr int kFusedWaves = 8;

template <int WDT, int ACT, int NV>
__global__ __launch_bounds__(kWave * kFusedWaves) void down_combine1_kernel(ExpertArgs p) {
    typedef typename Storage<WDT>::type wt;
    constexpr int VEC = vec_elems<WDT>();
    typedef WOps<WDT> Ops;
    constexpr int R = kFusedCols;
    __shared__ float ys[kFusedMaxK][R];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int H = p.H, I = p.I;
    const int n0 = blockIdx.x * R;
    const int nv = I / (kWave * VEC);
    for (int j = wv; j < p.k; j += kFusedWaves) {
        const int e = p.topk_idx[j];
        const wt* wexp = (const wt*)p.w_down + (int64_t)e * H * I;
        u32x4 v[R][NV];
#pragma unroll
        for (int q = 0; q < R; ++q)
#pragma unroll
            for (int t = 0; t < NV; ++t)
                if (t < nv && n0 + q < H)
                    v[q][t] = load_weights16(wexp + (int64_t)(n0 + q) * I + (t * kWave + lane) * VEC);
        u32x4 hr[NV][act_vecs<WDT>()];
        load_act_row<WDT, ACT, NV>((const char*)p.h + (int64_t)j * I *
                                                          (int64_t)sizeof(typename Storage<ACT>::type),
                                   nv, lane, hr);
#pragma unroll
        for (int q = 0; q < R; ++q) {
            float acc = 0.0f;
#pragma unroll
            for (int t = 0; t < NV; ++t)
                if (t < nv && n0 + q < H) {
                    uint32_t o[Ops::kOps];
                    Ops::unpack(v[q][t], o);
                    acc = Ops::dotr(o, hr[t], acc);
                }
            if (n0 + q < H) {
                const float sd = p.s_d ? p.s_d[(int64_t)e * H + n0 + q] : 1.0f;
                const float yv = wave_sum(acc) * sd;
                if (lane == 0) ys[j][q] = yv;
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < R && n0 + (int)threadIdx.x < H) {
        const int n = n0 + threadIdx.x;
        float acc = 0.0f;
        for (int jj = 0; jj < p.k; ++jj) acc = fmaf(p.topk_w[jj], ys[jj][threadIdx.x], acc);
        store_act<ACT>(p.out, n, load_act<ACT>(p.x, n) + acc);
    }
}

template <int WDT, int ACT, int NV>
hipError_t down_combine_one_row(const ExpertArgs& a, hipStream_t s) {
    const int grid = (a.H + kFusedCols - 1) / kFusedCols;
    const int waves = a.k < kFusedWaves ? a.k : kFusedWaves;
    down_combine1_kernel<WDT, ACT, NV><<<grid, kWave * waves, 0, s>>>(a);
    return hipGetLastError();
}

template <int WDT, int ACT>
hipError_t down_combine_typed(const ExpertArgs& a, hipStream_t s) {
    const int nv = row_vecs<WDT>(a.I);
    if (nv <= 2) return down_combine_one_row<WDT, ACT, 2>(a, s);
    if (nv <= 4) return down_combine_one_row<WDT, ACT, 4>(a, s);
    return hipErrorInvalidValue;  // longer rows: see down_combine_supported
}

// Rows per pass: up to 4 bf16 rows, or 2 fp32 rows, so that the staged
// activations of the widest supported row (8192) fit the 64 KB a block may
// take.
template <int ACT> constexpr int max_pass_rows() { return ACT == DT_F32 ? 2 : 4; }

template <int WDT, int ACT, int NV>
hipError_t down_one_row(const ExpertArgs& a, int max_units, hipStream_t s) {
    constexpr int U = NV < 4 ? NV : 4;
    constexpr int R = 4;
    constexpr int RW = 8;
    const int units = ((a.H + kWaves * RW - 1) / (kWaves * RW)) * max_units;
    const int grid = units < 8192 ? units : 8192;
    down_gemv1_kernel<WDT, ACT, NV, U, R, RW><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

template <int WDT, int ACT>
hipError_t gate_up_typed(const ExpertArgs& a, int max_rows, int max_experts, hipStream_t s) {
    // one-row experts keep the LDS-staged kernel here: holding a whole
    // hidden-size row in registers costs more occupancy than staging saves
    if (max_rows <= 1) return gate_up_mg<WDT, ACT, 1>(a, max_experts, s);
    if (max_rows <= 2) return gate_up_mg<WDT, ACT, 2>(a, max_experts, s);
    return gate_up_mg<WDT, ACT, max_pass_rows<ACT>()>(a, max_experts, s);
}

template <int WDT, int ACT>
hipError_t down_typed(const ExpertArgs& a, int max_rows, int max_experts, hipStream_t s) {
    // the one-row kernel holds a row of h in registers: up to 16 vectors per
    // lane (bf16 / fp8 rows up to 8192, fp32 rows up to 4096); longer rows
    // take the LDS-staged kernel, which walks any row length
    const int nv = row_vecs<WDT>(a.I);
    if (max_rows <= 1 && nv <= 16) {
        if (nv <= 2) return down_one_row<WDT, ACT, 2>(a, max_experts, s);
        if (nv <= 4) return down_one_row<WDT, ACT, 4>(a, max_experts, s);
        if (nv <= 8) return down_one_row<WDT, ACT, 8>(a, max_experts, s);
        return down_one_row<WDT, ACT, 16>(a, max_experts, s);
    }
    if (max_rows <= 2) return down_mg<WDT, ACT, 2>(a, max_experts, s);
    return down_mg<WDT, ACT, max_pass_rows<ACT>()>(a, max_experts, s);
}

}  // namespace

// max_rows: an upper bound on rows per expert in this launch (passes of 4
// rows beyond it).  max_experts: an upper bound on the number of experts the
// GEMV list can hold (sizes the grid).  Supported (wdt, act) pairs:
// (F32, F32), (BF16, BF16), (FP8, BF16).
hipError_t launch_gate_up_gemv(const ExpertArgs& a, int act, int wdt, int max_rows,
                               int max_experts, hipStream_t s) {
    if (wdt == DT_F32) return gate_up_typed<DT_F32, DT_F32>(a, max_rows, max_experts, s);
    if (wdt == DT_BF16) return gate_up_typed<DT_BF16, DT_BF16>(a, max_rows, max_experts, s);
    (void)act;
    return gate_up_typed<DT_FP8, DT_BF16>(a, max_rows, max_experts, s);
}

bool gate_up_select_supported(int E, int k) {
    return E >= 1 && E <= kWave * 32 && k >= 1 && k <= kMaxTopk && k <= E;
}

hipError_t launch_gate_up_select1(const ExpertArgs& a, const SelectArgs& q, int act, int wdt,
                                  int grid, hipStream_t s) {
    if (!gate_up_select_supported(q.E, a.k)) return hipErrorInvalidValue;
    if (wdt == DT_F32) return gate_up_select1_typed<DT_F32, DT_F32>(a, q, grid, s);
    if (wdt == DT_BF16) return gate_up_select1_typed<DT_BF16, DT_BF16>(a, q, grid, s);
    (void)act;
    return gate_up_select1_typed<DT_FP8, DT_BF16>(a, q, grid, s);
}

hipError_t launch_down_gemv(const ExpertArgs& a, int act, int wdt, int max_rows, int max_experts,
                            hipStream_t s) {
    if (wdt == DT_F32) return down_typed<DT_F32, DT_F32>(a, max_rows, max_experts, s);
    if (wdt == DT_BF16) return down_typed<DT_BF16, DT_BF16>(a, max_rows, max_experts, s);
    (void)act;
    return down_typed<DT_FP8, DT_BF16>(a, max_rows, max_experts, s);
}

// Whether launch_down_combine serves this shape: k <= 16 and a down row of at
// most four 16-byte vectors per lane (I <= 2048 bf16, 4096 fp8, 1024 fp32),
// so that a wave's weight loads and its row of h stay in registers.
bool down_combine_supported(int wdt, int I, int k) {
    const int nv = wdt == DT_FP8 ? row_vecs<DT_FP8>(I)
                 : wdt == DT_BF16 ? row_vecs<DT_BF16>(I) : row_vecs<DT_F32>(I);
    return k >= 1 && k <= kFusedMaxK && nv >= 1 && nv <= 4;
}

// Batch 1, every expert on the GEMV kernels: down projection and combine +
// residual in one launch (writes out; no y).
hipError_t launch_down_combine(const ExpertArgs& a, int act, int wdt, hipStream_t s) {
    if (!down_combine_supported(wdt, a.I, a.k)) return hipErrorInvalidValue;
    if (wdt == DT_F32) return down_combine_typed<DT_F32, DT_F32>(a, s);
    if (wdt == DT_BF16) return down_combine_typed<DT_BF16, DT_BF16>(a, s);
    (void)act;
    return down_combine_typed<DT_FP8, DT_BF16>(a, s);
}

}  // namespace moe
