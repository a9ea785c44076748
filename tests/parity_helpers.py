"""Shared pieces of the GPU parity tests: run the library, run the oracle on
the exact bytes the GPU consumed, and apply the acceptance rules.

Acceptance (per row b of a batch):
  * expert indices equal the oracle's ordered list exactly; a difference is
    excused only when the GPU list is still a valid top-k and every differing
    position swaps experts whose oracle (fp64) logits are within 1e-6;
  * routing weights within 1e-5 of the oracle's.  For an excused row the
    reference is the oracle's weights of the GPU's own selection (its fp64
    logits of those experts, renormalised), and the reference output of that
    row is the oracle's expert FFNs and combine on that selection: an excused
    row is checked like every other row, against the layer it did compute;
  * over the compared rows of out: max |gpu - oracle| <= 2e-2 and
    ||gpu - oracle||_2 / ||oracle||_2 <= 5e-3, against the oracle's unrounded
    fp64 output (the GPU rounds once to the activation type; a bf16 ulp in
    [4, 8) is 0.031, so comparing two rounded values would fail spuriously).
    Where one rounding step of the output type alone exceeds 2e-2 (bf16
    values of magnitude 8 and more, half an ulp 0.031), the bound is 2e-2
    beyond that half ulp: a correctly rounded bf16 output cannot be closer.

Two stricter checks on the expert term, which x dominates in out:
  * rounding excess: the GPU's out is its fp32 value rounded once to the
    activation type, so |out_gpu - out_oracle| <= half an ulp of the output
    plus the GPU's own arithmetic error.  The excess over half an ulp (of the
    larger of the two magnitudes, in the activation type) is a lower bound on
    that arithmetic error; its L2 norm over the rows must stay within 1e-3 of
    the L2 norm of the oracle's delta out - x.  fp32 sums of 7168 products and
    an occasional one-ulp flip of a bf16 rounding of h leave it near 1e-5; a
    1% error in the expert term already exceeds it;
  * with fp32 activations (no coarse output rounding) the relative L2 error of
    the delta itself must stay within 1e-4 (fp32 rounding of out is about
    6e-8 of |out|).
"""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_layer_decode_amd as M
import oracle
import workloads as W

ACT_CODE = {"f32": oracle.F32, "bf16": oracle.BF16}
WDT_CODE = {"f32": oracle.F32, "bf16": oracle.BF16, "fp8": oracle.E4M3}
MOE_W = {"f32": M.F32, "bf16": M.BF16, "fp8": M.FP8_E4M3}
MOE_ACT = {"f32": M.F32, "bf16": M.BF16}
ORACLE_SCORE = {"softmax": oracle.SOFTMAX, "sigmoid": oracle.SIGMOID}
MOE_SCORE = {"softmax": M.SOFTMAX, "sigmoid": M.SIGMOID}

GAP = 1e-6
MAX_ABS = 2e-2
REL_L2 = 5e-3
W_TOL = 1e-5
EXCESS_REL = 1e-3
F32_DELTA_REL = 1e-4
# significand bits of the activation types (binary32: 24, bf16: 8)
ACT_BITS = {"f32": 24, "bf16": 8}


def make_context(w: W.Workload, max_batch=None, max_topk=None) -> M.Context:
    return M.Context(w.E, w.H, w.I, MOE_W[w.wdt], MOE_ACT[w.act],
                     max_batch or w.B, max_topk or w.k)


def gpu_forward(ctx, w, L, x, out=None):
    """One layer on the GPU; returns (idx [B,k], weights [B,k], out tensor)."""
    B = x.shape[0]
    idx = torch.full((B, w.k), -1, dtype=torch.int32, device=x.device)
    wt = torch.zeros((B, w.k), dtype=torch.float32, device=x.device)
    out = torch.empty_like(x) if out is None else out
    ctx.forward(x, L["router_w"], L["w_gate_up"], L["w_down"], w.k, MOE_SCORE[w.score],
                bias=L["bias"], s_gu=L["s_gu"], s_d=L["s_d"], out=out, idx_out=idx,
                weight_out=wt)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), wt.cpu().numpy(), out


def oracle_logits(w, L, x):
    """The oracle's fp64 logits [B,E] of x (bias included)."""
    return oracle.router_logits(W.raw_numpy(x), ACT_CODE[w.act], W.raw_numpy(L["router_w"]),
                                W.raw_numpy(L["bias"]))


def oracle_outputs(w, L, x, sel, wts, rows):
    """The oracle's out [B,H] (NaN outside rows) for the selection sel [B,k]
    with weights wts [B,k]: each selected expert's FFN, then the combine.  Only
    the experts the given rows select are copied to the host, one at a time."""
    x_np = W.raw_numpy(x)
    B = x_np.shape[0]
    act, wdt = ACT_CODE[w.act], WDT_CODE[w.wdt]
    need = {}
    for b in rows:
        for j in range(w.k):
            need.setdefault(int(sel[b, j]), []).append((b, j))
    y = np.zeros((B, w.k, w.H))
    for e in sorted(need):
        gu = W.raw_numpy(L["w_gate_up"][e])
        dn = W.raw_numpy(L["w_down"][e])
        sg = W.raw_numpy(L["s_gu"][e]) if L["s_gu"] is not None else None
        sd = W.raw_numpy(L["s_d"][e]) if L["s_d"] is not None else None
        for b, j in need[e]:
            _, y[b, j] = oracle.expert_ffn(x_np[b], act, gu, dn, wdt, sg, sd)
    out = np.full((B, w.H), np.nan)
    for b in rows:
        out[b] = oracle.combine(x_np[b:b + 1], act, wts[b:b + 1], y[b:b + 1])[0]
    return out


def oracle_layer(w, L, x, rows=None):
    """The oracle on the bytes of the (device or host) tensors L and x.

    Only the outputs of ``rows`` are computed.  Returns
    (logits [B,E], idx [B,k], weights [B,k], out [B,H] with NaN outside rows).
    """
    lg = oracle_logits(w, L, x)
    idx, wts = oracle.topk(lg, w.k, ORACLE_SCORE[w.score])
    rows = list(range(lg.shape[0])) if rows is None else list(rows)
    return lg, idx, wts, oracle_outputs(w, L, x, idx, wts, rows)


def check_routing(lg, idx_o, idx_g, w_o, w_g, score, rows=None):
    """Index and weight parity.  Returns (excused rows, reference selection,
    reference weights): the oracle's own, except on excused rows, where they
    are the GPU's selection and the oracle's weights of it."""
    B, k = idx_o.shape
    E = lg.shape[1]
    rows = range(B) if rows is None else rows
    excused = []
    idx_ref = idx_o.copy()
    w_ref = w_o.copy()
    for b in rows:
        sel = idx_g[b]
        assert len(set(sel.tolist())) == k, f"row {b}: repeated experts {sel}"
        assert sel.min() >= 0 and sel.max() < E
        if not np.array_equal(idx_o[b], sel):
            rest = np.setdiff1d(np.arange(E), sel)
            assert lg[b, sel].min() >= lg[b, rest].max() - GAP, f"row {b}: not a top-{k}"
            for j in np.nonzero(idx_o[b] != sel)[0]:
                gap = abs(lg[b, idx_o[b, j]] - lg[b, sel[j]])
                assert gap < GAP, f"row {b} slot {j}: expert {sel[j]} vs {idx_o[b, j]}, gap {gap}"
            excused.append(b)
            idx_ref[b] = sel
            w_ref[b] = oracle.selection_weights(lg[b:b + 1], sel[None, :], score)[0]
        assert np.max(np.abs(w_g[b] - w_ref[b])) <= W_TOL, (b, w_g[b], w_ref[b])
    return excused, idx_ref, w_ref


def half_ulp(v, act):
    """Half the spacing of the activation type's values at |v| (normal range;
    the smallest normal spacing below it)."""
    bits = ACT_BITS[act]
    _, ex = np.frexp(np.maximum(np.abs(v), np.finfo(np.float32).tiny))
    return np.ldexp(1.0, ex - bits - 1)


def output_stats(out_g, out_o, x, act, rows):
    """Error statistics of the GPU rows against the oracle's unrounded ones."""
    g = out_g.float().cpu().numpy().astype(np.float64) if torch.is_tensor(out_g) else \
        np.asarray(out_g, np.float64)
    xf = x.float().cpu().numpy().astype(np.float64)
    assert rows, "no row to compare"
    assert np.all(np.isfinite(g[rows])), "non-finite GPU output"
    d = g[rows] - out_o[rows]
    delta_o = out_o[rows] - xf[rows]
    dn = max(1e-300, float(np.linalg.norm(delta_o)))
    hu = half_ulp(np.maximum(np.abs(g[rows]), np.abs(out_o[rows])), act)
    excess = np.maximum(0.0, np.abs(d) - hu)
    # the max-abs bound, widened by the output's half ulp where that alone exceeds it
    bound = MAX_ABS + np.where(hu > MAX_ABS, hu, 0.0)
    return dict(max_abs=float(np.abs(d).max()),
                max_abs_over_bound=float((np.abs(d) - bound).max()),
                rel_l2=float(np.linalg.norm(d) / np.linalg.norm(out_o[rows])),
                rel_l2_delta=float(np.linalg.norm(d) / dn),
                rounding_excess_rel=float(np.linalg.norm(excess) / dn),
                rows=len(rows))


def check_output(out_g, out_o, x, act, rows=None):
    """Output parity on rows; returns the statistics."""
    B = out_o.shape[0]
    rows = list(range(B) if rows is None else rows)
    stats = output_stats(out_g, out_o, x, act, rows)
    print(f"[parity] {stats}", flush=True)
    assert stats["max_abs_over_bound"] <= 0.0, stats
    assert stats["rel_l2"] <= REL_L2, stats
    assert stats["rounding_excess_rel"] <= EXCESS_REL, stats
    if act == "f32":
        assert stats["rel_l2_delta"] <= F32_DELTA_REL, stats
    return stats


def check_layer(w, L, x, idx_g, w_g, out_g, rows=None):
    """Every acceptance rule for one layer, given what the GPU returned."""
    lg = oracle_logits(w, L, x)
    idx_o, w_o = oracle.topk(lg, w.k, ORACLE_SCORE[w.score])
    excused, idx_ref, w_ref = check_routing(lg, idx_o, idx_g, w_o, w_g, ORACLE_SCORE[w.score])
    rows = list(range(lg.shape[0])) if rows is None else list(rows)
    out_ref = oracle_outputs(w, L, x, idx_ref, w_ref, rows)
    stats = check_output(out_g, out_ref, x, w.act, rows)
    stats["excused_rows"] = excused
    return stats


def full_check(ctx, w, L, x, rows=None):
    """GPU forward + oracle + all acceptance rules; returns (stats, gpu idx)."""
    idx_g, w_g, out_g = gpu_forward(ctx, w, L, x)
    stats = check_layer(w, L, x, idx_g, w_g, out_g, rows)
    return stats, idx_g, out_g


def run_stack(ctx, w, layers, x, fused, outs=None):
    """A stack through moe_decode_forward_stack, the combine folded into the
    next router or not; returns (idx, weights, outputs per layer, launches of
    the last layer)."""
    ctx.set_fused_next_router(fused)
    n = len(layers)
    idx = [torch.full((x.shape[0], w.k), -1, dtype=torch.int32, device="cuda") for _ in range(n)]
    wts = [torch.zeros((x.shape[0], w.k), dtype=torch.float32, device="cuda") for _ in range(n)]
    outs = ctx.forward_stack(x, layers, w.k, MOE_SCORE[w.score], outs=outs, idx_outs=idx,
                             weight_outs=wts)
    torch.cuda.synchronize()
    return ([i.cpu().numpy() for i in idx], [v.cpu().numpy() for v in wts],
            [o.clone() for o in outs], ctx.last_plan()["launches"])


def same_stack(a, b):
    """Two stacks' results are the same bits, layer by layer."""
    for l in range(len(a[0])):
        assert np.array_equal(a[0][l], b[0][l]), l
        assert np.array_equal(a[1][l], b[1][l]), l
        assert torch.equal(a[2][l], b[2][l]), l
