"""Benchmark of the decode-step MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload full_b1]

A step is one forward of the whole layer (router GEMV + top-k + bucketing,
gate/up + SwiGLU, down, combine + residual) on one decode batch.  Inputs are
synthetic (seeded N(0,1) rows, N(0,0.02) weights), resident in HBM before
the timed region; each step takes the next of 16 pre-generated input batches,
so consecutive steps select different experts (as consecutive decode steps
do) instead of re-reading the same 1.4 GB.

Printed: one JSON line with the headline (microseconds per layer at batch 1
on the full 7168/896/16/2048 bf16 layer), the per-stage times from HIP events
on the library's stream, HBM bandwidth of the expert stream and of the whole
layer against the 8 TB/s MI355X peak, the same at batches 8 and 64, the
roofline of the dominant kernel, and the CPU oracle timed on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_HBM_GBPS = 8000.0
METRIC = "µs per MoE decode layer + achieved HBM GB/s (% of peak), batch 1/8/64"


def _log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="full_b1")
    ap.add_argument("--extra-batches", default="8,64",
                    help="other batch sizes to time on the same layer ('' for none)")
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "mfma"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU-oracle sample budget (0 disables)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("this benchmark runs one GPU: the whole MoE layer is one GPU's share, with no "
               "sharding and no collectives; run it with --gpus 1")
        print(json.dumps({"error": msg, "n_gpus": max(args.gpus, world)}))
        _log(msg)
        return 2

    import numpy as np
    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import mixture_experts_layer_decode_amd as M
    import workloads as W

    if not torch.cuda.is_available():
        _log("no GPU visible")
        return 1
    M.load_library(build_if_missing=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = W.WORKLOADS[args.workload]
    wcode = {"f32": M.F32, "bf16": M.BF16, "fp8": M.FP8_E4M3}[w.wdt]
    acode = {"f32": M.F32, "bf16": M.BF16}[w.act]
    score = M.SIGMOID if w.score == "sigmoid" else M.SOFTMAX
    path = {"auto": M.PATH_AUTO, "gemv": M.PATH_GEMV, "mfma": M.PATH_MFMA}[args.path]

    t0 = time.time()
    L = W.make_layer(w, 0, device=dev)
    torch.cuda.synchronize()
    _log(f"[bench] layer {w.name} generated in {time.time() - t0:.1f}s")

    ctx = M.Context(w.E, w.H, w.I, wcode, acode, max_batch=64, max_topk=w.k)
    ctx.set_path(path)
    n_inputs = 16

    def make_inputs(B, recipe):
        xs = [W.make_x(recipe, 0, step=s, device=dev, B=B) for s in range(n_inputs)]
        idx = [torch.empty((B, w.k), dtype=torch.int32, device=dev) for _ in range(n_inputs)]
        outs = [torch.empty_like(xs[0]) for _ in range(n_inputs)]
        return xs, idx, outs

    def fwd(x, out, idx=None):
        ctx.forward(x, L["router_w"], L["w_gate_up"], L["w_down"], w.k, score, bias=L["bias"],
                    s_gu=L["s_gu"], s_d=L["s_d"], out=out, idx_out=idx)

    def run(B, recipe, steps, warmup):
        xs, idxs, outs = make_inputs(B, recipe)
        for i in range(warmup):
            fwd(xs[i % n_inputs], outs[i % n_inputs], idxs[i % n_inputs])
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(steps):
            fwd(xs[i % n_inputs], outs[i % n_inputs], idxs[i % n_inputs])
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t_start) * 1e3 / steps
        # distinct experts per step (same inputs, same routing)
        d_per_input = [len(torch.unique(t).tolist()) for t in idxs]
        d_mean = float(np.mean([d_per_input[i % n_inputs] for i in range(steps)]))
        # per-stage GPU time from HIP events on the library's stream
        ctx.set_timing(True)
        ctx.get_timing(reset=True)
        for i in range(steps):
            fwd(xs[i % n_inputs], outs[i % n_inputs], idxs[i % n_inputs])
        stage_ms, count = ctx.get_timing(reset=True)
        ctx.set_timing(False)
        stage_us = {k: v * 1e3 / count for k, v in stage_ms.items()}
        return ms, d_mean, stage_us

    def figures(B, ms, d_mean, stage_us):
        expert_bytes = d_mean * w.expert_bytes()
        gu_bytes = d_mean * w.expert_bytes() * 2 / 3 if w.wdt != "fp8" else \
            d_mean * (2 * w.I * w.H + 2 * w.I * 4)
        layer_bytes = expert_bytes + w.router_bytes()
        expert_us = stage_us["gate_up"] + stage_us["down"]
        return dict(
            batch=B, us_per_layer=ms * 1e3, distinct_experts=d_mean,
            algorithmic_bytes=layer_bytes,
            layer_gbps=layer_bytes / (ms * 1e-3) / 1e9,
            layer_pct_of_peak=100 * layer_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            expert_stream_gbps=expert_bytes / (expert_us * 1e-6) / 1e9,
            expert_stream_pct_of_peak=100 * expert_bytes / (expert_us * 1e-6) / 1e9 /
            PEAK_HBM_GBPS,
            stage_us=stage_us, gate_up_bytes=gu_bytes)

    recipe = w
    ms, d_mean, stage_us = run(w.B, recipe, args.steps, args.warmup)
    head = figures(w.B, ms, d_mean, stage_us)
    _log(f"[bench] B={w.B}: {head['us_per_layer']:.1f} us/layer, D={d_mean:.1f}, "
         f"stages {stage_us}")

    extra = {}
    for tok in [t for t in args.extra_batches.split(",") if t.strip()]:
        B = int(tok)
        if B == w.B:
            continue
        rec = W.WORKLOADS["verify_b8"] if (B == 8 and w.name == "full_b1") else \
            W.scaled(w, B=B)
        steps = max(5, min(args.steps, 30 if B >= 32 else args.steps))
        msb, db, sb = run(B, rec, steps, min(args.warmup, 5))
        extra[str(B)] = figures(B, msb, db, sb)
        _log(f"[bench] B={B}: {extra[str(B)]['us_per_layer']:.1f} us/layer, D={db:.1f}")

    # roofline of the dominant kernel: the gate/up projection (2/3 of the bytes)
    gu_us = stage_us["gate_up"]
    achieved = head["gate_up_bytes"] / (gu_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                "kernel": "gate_up (GEMV, SwiGLU epilogue)",
                "bytes_per_launch": head["gate_up_bytes"], "avg_launch_us": round(gu_us, 2)}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, L, dev, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(head["us_per_layer"], 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3 weights, bf16 act", "f32": "f32"}[w.wdt],
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) random-init weights)",
        "config": {"workload": w.name, "batch": w.B, "hidden": w.H, "experts": w.E,
                   "topk": w.k, "inter": w.I, "weights": w.wdt, "score": w.score,
                   "path": args.path},
        "hbm_gbps": round(head["layer_gbps"], 1),
        "pct_of_peak": round(head["layer_pct_of_peak"], 2),
        "expert_stream_gbps": round(head["expert_stream_gbps"], 1),
        "expert_stream_pct_of_peak": round(head["expert_stream_pct_of_peak"], 2),
        "distinct_experts": head["distinct_experts"],
        "stage_us": {k: round(v, 2) for k, v in stage_us.items()},
        "batches": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                        for kk, vv in v.items() if kk != "stage_us"} |
                    {"stage_us": {a: round(b, 2) for a, b in v["stage_us"].items()}}
                    for k, v in extra.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    ctx.close()
    print(json.dumps(line))
    return 0


def cpu_baseline(w, L, dev, budget_s):
    """The CPU oracle on a bounded sample: whole layers at the headline batch,
    repeated until the time budget is spent."""
    import numpy as np
    import torch

    import oracle
    import workloads as W

    act = {"f32": oracle.F32, "bf16": oracle.BF16}[w.act]
    wdt = {"f32": oracle.F32, "bf16": oracle.BF16, "fp8": oracle.E4M3}[w.wdt]
    score = oracle.SIGMOID if w.score == "sigmoid" else oracle.SOFTMAX
    x = W.raw_numpy(W.make_x(w, 0, step=0, device=dev))
    router = W.raw_numpy(L["router_w"])
    bias = W.raw_numpy(L["bias"])
    lg = oracle.router_logits(x, act, router, bias)
    idx, _ = oracle.topk(lg, w.k, score)
    experts = {}
    for e in np.unique(idx):
        experts[int(e)] = (W.raw_numpy(L["w_gate_up"][e]), W.raw_numpy(L["w_down"][e]),
                           W.raw_numpy(L["s_gu"][e]) if L["s_gu"] is not None else None,
                           W.raw_numpy(L["s_d"][e]) if L["s_d"] is not None else None)
    torch.cuda.synchronize()
    reps, t_total = 0, 0.0
    while t_total < budget_s or reps == 0:
        t0 = time.perf_counter()
        lg = oracle.router_logits(x, act, router, bias)
        idx, wts = oracle.topk(lg, w.k, score)
        y = np.zeros((x.shape[0], w.k, w.H))
        for b in range(x.shape[0]):
            for j in range(w.k):
                gu, dn, sg, sd = experts[int(idx[b, j])]
                _, y[b, j] = oracle.expert_ffn(x[b], act, gu, dn, wdt, sg, sd)
        oracle.combine(x, act, wts, y)
        t_total += time.perf_counter() - t0
        reps += 1
    us = t_total / reps * 1e6
    return {"value": round(us, 1), "unit": "us/layer", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{reps} whole layer(s) of {w.name} (batch {w.B}, input step 0), "
                      f"compute only (expert weights copied to host beforehand)"}


if __name__ == "__main__":
    sys.exit(main())
