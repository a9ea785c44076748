"""Shared pieces of the GPU parity tests: run the library, run the oracle on
the exact bytes the GPU consumed, and apply the acceptance rules.

Acceptance (per row b of a batch):
  * expert indices equal the oracle's ordered list exactly; a difference is
    excused only when the GPU list is still a valid top-k and every differing
    position swaps experts whose oracle (fp64) logits are within 1e-6;
  * routing weights within 1e-5 of the oracle's;
  * over the compared rows of out: max |gpu - oracle| <= 2e-2 and
    ||gpu - oracle||_2 / ||oracle||_2 <= 5e-3, against the oracle's unrounded
    fp64 output (the GPU rounds once to the activation type; a bf16 ulp in
    [4, 8) is 0.031, so comparing two rounded values would fail spuriously).
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


def oracle_layer(w, L, x, rows=None):
    """The oracle on the bytes of the (device or host) tensors L and x.

    Only the outputs of ``rows`` are computed, and only the experts those rows
    select are copied to the host (one at a time).  Returns
    (logits [B,E], idx [B,k], weights [B,k], out [B,H] with NaN outside rows).
    """
    x_np = W.raw_numpy(x)
    B = x_np.shape[0]
    act, wdt = ACT_CODE[w.act], WDT_CODE[w.wdt]
    lg = oracle.router_logits(x_np, act, W.raw_numpy(L["router_w"]), W.raw_numpy(L["bias"]))
    idx, wts = oracle.topk(lg, w.k, ORACLE_SCORE[w.score])
    rows = list(range(B)) if rows is None else list(rows)
    need = {}
    for b in rows:
        for j in range(w.k):
            need.setdefault(int(idx[b, j]), []).append((b, j))
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
    return lg, idx, wts, out


def check_routing(lg, idx_o, idx_g, w_o, w_g, rows=None):
    """Index and weight parity; returns the rows excused as near-ties."""
    B, k = idx_o.shape
    E = lg.shape[1]
    rows = range(B) if rows is None else rows
    excused = []
    for b in rows:
        sel = idx_g[b]
        assert len(set(sel.tolist())) == k, f"row {b}: repeated experts {sel}"
        assert sel.min() >= 0 and sel.max() < E
        if np.array_equal(idx_o[b], sel):
            assert np.max(np.abs(w_g[b] - w_o[b])) <= W_TOL, (b, w_g[b], w_o[b])
            continue
        rest = np.setdiff1d(np.arange(E), sel)
        assert lg[b, sel].min() >= lg[b, rest].max() - GAP, f"row {b}: not a top-{k}"
        for j in np.nonzero(idx_o[b] != sel)[0]:
            gap = abs(lg[b, idx_o[b, j]] - lg[b, sel[j]])
            assert gap < GAP, f"row {b} slot {j}: expert {sel[j]} vs {idx_o[b, j]}, gap {gap}"
        excused.append(b)
    return excused


def check_output(out_g, out_o, x, rows=None, exclude=()):
    """Output parity on rows (minus excused ones); returns the statistics."""
    g = out_g.float().cpu().numpy().astype(np.float64)
    xf = x.float().cpu().numpy().astype(np.float64)
    B = g.shape[0]
    rows = [b for b in (range(B) if rows is None else rows) if b not in exclude]
    assert rows, "no row left to compare"
    d = g[rows] - out_o[rows]
    assert np.all(np.isfinite(g[rows])), "non-finite GPU output"
    max_abs = float(np.abs(d).max())
    rel = float(np.linalg.norm(d) / np.linalg.norm(out_o[rows]))
    rel_delta = float(np.linalg.norm(d) / max(1e-300, np.linalg.norm(out_o[rows] - xf[rows])))
    stats = dict(max_abs=max_abs, rel_l2=rel, rel_l2_delta=rel_delta, rows=len(rows))
    print(f"[parity] {stats}", flush=True)
    assert max_abs <= MAX_ABS, stats
    assert rel <= REL_L2, stats
    return stats


def full_check(ctx, w, L, x, rows=None):
    """GPU forward + oracle + all acceptance rules; returns (stats, gpu idx)."""
    idx_g, w_g, out_g = gpu_forward(ctx, w, L, x)
    lg, idx_o, w_o, out_o = oracle_layer(w, L, x, rows)
    excused = check_routing(lg, idx_o, idx_g, w_o, w_g)
    stats = check_output(out_g, out_o, x, rows, exclude=excused)
    stats["excused_rows"] = excused
    return stats, idx_g, out_g
