// moe_internal.h -- structures shared by the host runtime and the gfx950
// kernels of libmoe_decode.so (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 2048;
constexpr int kMaxBatch = 64;
constexpr int kMaxTopk = 32;
constexpr int kMaxSlots = kMaxBatch * kMaxTopk;  // rows x selected experts
constexpr int kSlotBits = 11;                    // kMaxSlots == 1 << kSlotBits

enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };
enum { CLS_GEMV = 0, CLS_MFMA = 1 };
enum { PATH_AUTO = 0, PATH_GEMV = 1, PATH_MFMA = 2 };
enum { ROUTER_AUTO = 0, ROUTER_GEMV = 1, ROUTER_MFMA = 2 };
constexpr int kMaxRouterSplits = 4;  // partial-logit slices of the matrix-core router
// Rows of x the bf16 / fp8 GEMV kernels stage per pass: an expert with more
// rows streams its weights once per pass, so AUTO never gives them one.
constexpr int kGemvPassRows = 4;

// The routing plan of one forward, written on the device by the top-k kernel
// (or, above 8 rows, by the bucket kernel) and read by the expert kernels.  The host never
// reads it on the hot path, so grids are sized for the worst case and every
// expert kernel walks the lists that apply to it.
//
// A "slot" is one (row b, choice j) pair, numbered b * k + j.  perm lists the
// slots ordered by (expert, slot), so the rows routed to one expert are
// contiguous: list_start/list_count index into perm.
struct DevPlan {
    int num_slots;              // B * k
    int num_active;             // D, distinct experts selected in the batch
    int n_list[2];              // experts served by GEMV / by MFMA kernels
    int max_rows;               // most rows on one expert
    int pad[3];
    int list_expert[2][kMaxExperts];
    int list_start[2][kMaxExperts];
    int list_count[2][kMaxExperts];
    int perm[kMaxSlots];
};

struct RouterArgs {
    const void* x;       // [B][x_stride] activations
    int64_t x_stride;
    int B, H, E, k, score_fn;
    const float* wr;     // [E][wr_stride]
    int64_t wr_stride;
    const float* bias;   // [E] or null
    double* logits;      // [k_splits][B][E] workspace: partial logits, bias not added
    int k_splits;        // column ranges the router kernel sums separately (set by launch_router)
    int router_mode;     // ROUTER_* (host side: which router kernel)
    int rows_per_stage;  // rows of x staged in LDS per router GEMV pass
    int* topk_idx;       // [B][k] workspace
    float* topk_w;       // [B][k] workspace
    int* user_idx;       // optional copies for the caller
    float* user_w;
    DevPlan* plan;
    int path_mode;
    int mfma_min_rows;
    int mfma_ok;         // weight type has an MFMA kernel
    int logits_only;     // host side: launch the router GEMV only (batch 1, the
                         // gate/up kernel selects the experts itself)
    int logits_ready;    // host side: > 0 when the previous layer's combine +
                         // router kernel already left this many slices of
                         // logits: launch only the top-k (and buckets)
    // the previous layer's combine + residual folded into this router
    // (launch_combine_router): p.x is then the previous layer's input
    const float* comb_y;     // [B * comb_k][H] previous layer's expert outputs
    const float* comb_w;     // [B][comb_k] its routing weights
    int comb_k;
    void* comb_out;          // [B][comb_out_stride] its output (written here)
    int64_t comb_out_stride;
};

struct ExpertArgs {
    const void* x;         // [B][x_stride] activations
    int64_t x_stride;
    int k, H, I;
    const void* w_gate_up; // [E][2I][H]
    const void* w_down;    // [E][H][I]
    const float* s_gu;     // [E][2I] or null
    const float* s_d;      // [E][H] or null
    const DevPlan* plan;
    void* h;               // [slots][I] activation type
    float* y;              // [slots][H]
    float* partial;        // split-K partial sums [split_k][slot_cap][max(2I, H)]
    int slot_cap;          // slots the workspace holds (max_batch * max_topk)
    int split_k;           // K splits of the MFMA kernels (1 = none)
    // down projection with the combine folded in (batch 1) only:
    void* out;             // [1][H] activation type
    const int* topk_idx;   // [k] selected experts, in order
    const float* topk_w;   // [k] routing weights
};

// Batch 1 with the selection taken by the gate/up kernel itself: every
// workgroup selects the top k from the router's logits (fp64, one row, one
// slice) and workgroup 0 also writes the routing outputs and the plan.
struct SelectArgs {
    const double* logits;  // [E]
    const float* bias;     // [E] or null
    int E, score_fn;
    int* topk_idx;         // [k] workspace
    float* topk_w;         // [k] workspace
    int* user_idx;         // optional copies for the caller
    float* user_w;
    DevPlan* plan;         // every expert listed under CLS_GEMV, one row each
};

struct CombineArgs {
    const void* x;
    int64_t x_stride;
    void* out;
    int64_t out_stride;
    int B, H, k;
    const float* topk_w;  // [B][k]
    const float* y;       // [B*k][H]
};

// Launchers (return the launch status).  act/wdt are DT_* codes.
int router_rows_per_stage(int H, int act, int B);
// Router and top-k (and buckets); *kernel receives the router kernel used
// (ROUTER_GEMV / ROUTER_MFMA) and *launches the kernels launched.
hipError_t launch_router(const RouterArgs& a, int act, hipStream_t s, int* kernel, int* launches);
// The previous layer's combine + residual and this layer's router logits in
// one launch, on the matrix cores (a.comb_* set, a.x the previous layer's
// input; batches of up to 16 rows); *splits receives the slices of logits
// left for the top-k.
bool combine_router_supported(int E, int H, int B);
bool router_uses_mfma(int router_mode, int B, int E, int H);
hipError_t launch_combine_router(const RouterArgs& a, int act, hipStream_t s, int* splits);
hipError_t launch_gate_up_gemv(const ExpertArgs& a, int act, int wdt, int max_rows,
                               int max_units, hipStream_t s);
hipError_t launch_down_gemv(const ExpertArgs& a, int act, int wdt, int max_rows, int max_units,
                            hipStream_t s);
// Batch 1: the top-k selection, routing weights and plan, then gate/up +
// SwiGLU of the k selected experts, in one launch (grid: workgroups to use,
// 0 = one per unit).
bool gate_up_select_supported(int E, int k);
hipError_t launch_gate_up_select1(const ExpertArgs& a, const SelectArgs& q, int act, int wdt,
                                  int grid, hipStream_t s);
constexpr int kFusedCombineMaxK = 16;  // experts per row the folded combine serves
bool down_combine_supported(int wdt, int I, int k);
hipError_t launch_down_combine(const ExpertArgs& a, int act, int wdt, hipStream_t s);
hipError_t launch_gate_up_mfma(const ExpertArgs& a, int wdt, int max_rows, int max_experts,
                               hipStream_t s);
hipError_t launch_down_mfma(const ExpertArgs& a, int wdt, int max_rows, int max_experts,
                            hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int act, hipStream_t s);
hipError_t launch_prefetch(const void* const* ptrs, const int64_t* bytes, int n, uint32_t* sink,
                           int grid, hipStream_t s);

}  // namespace moe
