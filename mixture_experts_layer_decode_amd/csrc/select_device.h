// select_device.h -- exact top-k selection of one row of router logits by
// one wave, and the routing weights of the selection (gfx950 device code).
// Used by the top-k kernel and, at batch 1, by the gate/up kernel that
// selects the experts itself.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// (va, ea) ranks before (vb, eb): larger logit, or equal with lower index.
__device__ __forceinline__ bool ranks_before(double va, int ea, double vb, int eb) {
    return va > vb || (va == vb && ea < eb);
}

// Order-preserving 64-bit key of a finite double (larger value, larger key).
__device__ __forceinline__ uint64_t order_key(double d) {
    const uint64_t u = __double_as_longlong(d);
    return (u >> 63) ? ~u : (u | (1ull << 63));
}

// LDS writes of this wave are visible to its other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// The k best (logit, expert) pairs of one row under the order "larger logit,
// then lower index", in that order: lane j < k receives the j-th in
// (sel_v, sel_e).  Lane l holds the logits of experts l, l + 64, ... in v.
//
// Exact threshold method: any L such that at least k lane maxima are >= L is
// a lower bound on the k-th largest logit (those lanes hold k distinct logits
// >= L), so every selected logit is >= L.  L is the largest value whose
// order-preserving key has only its top 24 bits set (sign, exponent, 12
// mantissa bits) and that at least k lane maxima reach; it is found by an
// MSB-first search counting lanes with ballots.  The candidates >= L (about
// 18 of 896 for N(0, 1.7) logits) are written to LDS, each lane at the sum of
// the lower lanes' candidate counts, and ranked by direct comparison, each
// candidate reading the others with readlane.  If more than 64
// logits tie at or above L (degenerate inputs), k rounds of a wave argmax are
// used instead.
template <int PL>
__device__ void select_topk(const double (&v)[PL], int E, int k, double* cv, int* ce,
                            double* sv, int* se, double& sel_v, int& sel_e) {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t key[PL];   // order keys; 0 (below every finite key) past E
    uint64_t lkey = 0;  // the lane's largest
#pragma unroll
    for (int t = 0; t < PL; ++t) {
        key[t] = lane + t * kWave < E ? order_key(v[t]) : 0;
        lkey = key[t] > lkey ? key[t] : lkey;
    }
    uint64_t T = 0;
    for (int bit = 63; bit >= 40; --bit) {
        const uint64_t cand = T | (1ull << bit);
        if (__popcll(__ballot(lkey >= cand)) >= k) T = cand;
    }
    // compact the candidates (key >= T) into cv / ce: each lane counts its
    // own (at most PL < 64), and its first position is the sum of the lower
    // lanes' counts, taken bit by bit with ballots
    int mine = 0;
#pragma unroll
    for (int t = 0; t < PL; ++t) mine += key[t] >= T ? 1 : 0;
    const uint64_t below = (1ull << lane) - 1ull;
    int pos = 0, C = 0;
#pragma unroll
    for (int b = 0; b < 6; ++b) {
        if ((1 << b) > PL) break;
        const uint64_t m = __ballot((mine >> b) & 1);
        pos += __popcll(m & below) << b;
        C += __popcll(m) << b;
    }
#pragma unroll
    for (int t = 0; t < PL; ++t)
        if (key[t] >= T) {
            if (pos < kWave) {
                cv[pos] = v[t];
                ce[pos] = lane + t * kWave;
            }
            ++pos;
        }
    wave_lds_sync();
    if (C <= kWave) {
        // candidate `lane` counts the candidates that rank before it, reading
        // them from the other lanes with readlane (faster here than
        // same-address LDS loads)
        double mv = 0.0;
        int me = 0;
        if (lane < C) {
            mv = cv[lane];
            me = ce[lane];
        }
        const uint64_t mbits = __double_as_longlong(mv);
        const int mlo = (int)(uint32_t)mbits, mhi = (int)(uint32_t)(mbits >> 32);
        int rank = 0;
        for (int j = 0; j < C; ++j) {
            const uint32_t olo = (uint32_t)__builtin_amdgcn_readlane(mlo, j);
            const uint32_t ohi = (uint32_t)__builtin_amdgcn_readlane(mhi, j);
            const int oe = __builtin_amdgcn_readlane(me, j);
            const double ov = __longlong_as_double((long long)(((uint64_t)ohi << 32) | olo));
            rank += ranks_before(ov, oe, mv, me) ? 1 : 0;
        }
        if (lane < C && rank < k) {
            sv[rank] = mv;
            se[rank] = me;
        }
        wave_lds_sync();
        if (lane < k) {
            sel_v = sv[lane];
            sel_e = se[lane];
        }
        return;
    }
    // degenerate ties: k rounds of a wave-wide argmax
    uint32_t avail = 0;
#pragma unroll
    for (int t = 0; t < PL; ++t)
        if (lane + t * kWave < E) avail |= 1u << t;
    for (int j = 0; j < k; ++j) {
        double bv = 0.0;
        int be = 0x7fffffff;  // no candidate
#pragma unroll
        for (int t = 0; t < PL; ++t) {
            const int ee = lane + t * kWave;
            if (((avail >> t) & 1u) && (be == 0x7fffffff || ranks_before(v[t], ee, bv, be))) {
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
}

// Renormalised routing weight of the selection held in lanes 0..k-1 (in
// order), computed in fp64: sigmoid(s_j) / sum sigmoid, or the softmax
// restricted to the selection, exp(s_j - s_0) / sum exp(s - s_0), s_0 being the
// largest selected logit.  Lanes >= k return an unused value.
__device__ __forceinline__ float routing_weight(double sel_v, int k, int score_fn) {
    const int lane = threadIdx.x & (kWave - 1);
    const double top = __shfl(sel_v, 0, kWave);
    double pj = 0.0;
    if (lane < k) pj = score_fn == 1 ? 1.0 / (1.0 + exp(-sel_v)) : exp(sel_v - top);
    const double total = wave_sum(pj);
    return (float)(pj / total);
}

}  // namespace moe
