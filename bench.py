"""Benchmark of the decode-step MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep] [--no-stack]

A step is one forward of the whole layer (router GEMV, top-k + weights +
bucketing, gate/up + SwiGLU, down, combine + residual) on one decode batch.
Inputs are synthetic (seeded N(0,1) rows, N(0,0.02) random-init weights) and
resident in HBM before the timed region; each step takes the next of 16
pre-generated input batches, so consecutive steps select different experts,
as consecutive decode steps do, instead of re-reading the same 1.4 GB.

Printed: one JSON line.  The headline is microseconds per layer at batch 1 on
the full 7168/896/16/2048 bf16 layer (lower is better).  It also carries:
  * per-stage GPU times from HIP events recorded on the library's stream
    during a second pass over the same timed steps;
  * HBM bandwidth of the expert stream and of the whole layer against the
    8 TB/s MI355X peak, also at 8 verify rows and at batch 64, and for verify
    batches of 3 to 6 drafts and of 8 sequences x 8 rows;
  * the roofline of the dominant kernel (gate/up at batch 1), also against
    the read bandwidth of a plain streaming kernel measured in the same run;
  * the 4-layer fp8 stack at batch 16 with and without the next-layer
    prefetch (bandwidth from the distinct experts of every layer);
  * the same steps replayed from a HIP graph, and the launches per layer;
  * per-forward percentiles at batch 1 (HIP events around each forward),
    back to back and with a 512 MB cache scrub before each forward;
  * the small fp32 layer (hidden 512, 64 experts, top-4) at batch 1;
  * the CPU oracle timed beside them on the host's cores (CPU model and core
    count stated): the batch-1 layer on all threads and on one, and batches
    of 8 and 64 rows and one fp8 layer on all threads (the larger ones on a
    sample of their rows, scaled).
With --sweep it also times every expert-kernel choice (GEMV, MFMA, the AUTO
row threshold, split-K factors) at batches 1, 8 and 64.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

PEAK_HBM_GBPS = 8000.0
ROUTER_NAMES = {1: "gemv", 2: "mfma"}
METRIC = "µs per MoE decode layer + achieved HBM GB/s (% of peak), batch 1/8/64"
N_INPUTS = 16
# None: the steps cycle through N_INPUTS input batches (steps 0 .. 15 of the
# workload's recipe); a step number: every forward takes that one batch (for
# counter runs, whose per-dispatch figures then share one set of experts)
INPUT_STEP = None


def _log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Runner:
    """Times forwards of one layer (or a stack) through the C ABI."""

    def __init__(self, M, W, torch, dev, w, layers, router=0):
        self.M, self.W, self.torch, self.dev, self.w = M, W, torch, dev, w
        self.layers = layers
        wcode = {"f32": M.F32, "bf16": M.BF16, "fp8": M.FP8_E4M3}[w.wdt]
        acode = {"f32": M.F32, "bf16": M.BF16}[w.act]
        self.score = M.SIGMOID if w.score == "sigmoid" else M.SOFTMAX
        self.ctx = M.Context(w.E, w.H, w.I, wcode, acode, max_batch=64, max_topk=w.k)
        self.ctx.set_router(router)

    def close(self):
        self.ctx.close()

    def inputs(self, B, recipe):
        torch = self.torch
        steps = range(N_INPUTS) if INPUT_STEP is None else [INPUT_STEP] * N_INPUTS
        xs = [self.W.make_x(recipe, 0, step=s, device=self.dev, B=B) for s in steps]
        # routing of every layer for each input batch (distinct experts per layer)
        idx = [[torch.empty((B, self.w.k), dtype=torch.int32, device=self.dev)
                for _ in self.layers] for _ in range(N_INPUTS)]
        # one output per layer of the stack, for each input batch
        outs = [[torch.empty_like(xs[0]) for _ in self.layers] for _ in range(N_INPUTS)]
        return xs, idx, outs

    def time_graph(self, B, recipe, steps, warmup):
        """ms per step with the steps replayed from one HIP graph that holds
        a forward of each of the N_INPUTS input batches: at least 2 untimed and
        4 timed replays (one replay of 16 forwards is too short a sample: its
        launch and first-replay costs then weigh on every forward)."""
        torch = self.torch
        xs, idxs, outs = self.inputs(B, recipe)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up on a side stream before capture
            for i in range(N_INPUTS):
                self.step(i, xs, idxs, outs, None)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(N_INPUTS):
                self.step(i, xs, idxs, outs, None)
        torch.cuda.synchronize()
        for _ in range(max(2, warmup // N_INPUTS)):
            g.replay()
        torch.cuda.synchronize()
        reps = max(4, steps // N_INPUTS)
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / (reps * N_INPUTS)
        del g
        return ms

    def time_each(self, B, recipe, n, scrub=None):
        """Per-forward GPU times (HIP events on the stream the library runs on,
        around each forward alone): percentiles in us.  With ``scrub``, a
        tensor of at least the last-level cache's size is rewritten before
        each forward, outside the events, so no weight is still cached."""
        torch, np = self.torch, __import__("numpy")
        xs, idxs, outs = self.inputs(B, recipe)
        for i in range(3):
            self.step(i, xs, idxs, outs, None)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i in range(n):
            if scrub is not None:
                scrub.add_(1)
            ev[i][0].record()
            self.step(i, xs, idxs, outs, None)
            ev[i][1].record()
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        return {"p10": round(float(np.percentile(us, 10)), 2),
                "p50": round(float(np.percentile(us, 50)), 2),
                "p90": round(float(np.percentile(us, 90)), 2), "n": n}

    def fwd(self, L, x, out, idx=None):
        self.ctx.forward(x, L["router_w"], L["w_gate_up"], L["w_down"], self.w.k, self.score,
                         bias=L["bias"], s_gu=L["s_gu"], s_d=L["s_d"], out=out, idx_out=idx)

    def step(self, i, xs, idxs, outs, prefetch):
        """One decode step: every layer of the stack in turn (with
        ``prefetch == "stack"``, all layers through one stack call)."""
        x = xs[i % N_INPUTS]
        if prefetch == "stack":
            self.ctx.forward_stack(x, self.layers, self.w.k, self.score, outs=outs[i % N_INPUTS],
                                   idx_outs=idxs[i % N_INPUTS])
            return
        for l, L in enumerate(self.layers):
            if prefetch is not None and prefetch != "stack":
                nxt = self.layers[l + 1] if l + 1 < len(self.layers) else None
                self.ctx.set_prefetch(prefetch(nxt) if nxt is not None else [])
            out = outs[i % N_INPUTS][l]
            self.fwd(L, x, out, idxs[i % N_INPUTS][l])
            x = out

    def time(self, B, recipe, steps, warmup, path=None, min_rows=0, split_k=0, prefetch=None,
             warm_s=0.0):
        """(ms per step, distinct experts of the first layer, per-stage us per layer).
        ``warmup`` untimed steps, then more until ``warm_s`` seconds of them."""
        torch, np = self.torch, __import__("numpy")
        if path is not None:
            self.ctx.set_path(path, min_rows, split_k)
        xs, idxs, outs = self.inputs(B, recipe)
        t_warm = time.perf_counter()
        for i in range(warmup):
            self.step(i, xs, idxs, outs, prefetch)
        torch.cuda.synchronize()
        while time.perf_counter() - t_warm < warm_s:
            for i in range(N_INPUTS):
                self.step(i, xs, idxs, outs, prefetch)
            torch.cuda.synchronize()
        # timed region: exactly `steps` steps, nothing recorded in between
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i, xs, idxs, outs, prefetch)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        # the same steps again, timed per stage by HIP events the library
        # records on its stream between stages (each event adds a little
        # queue overhead, so the headline above is taken without them)
        self.ctx.set_timing(True)
        self.ctx.get_timing(reset=True)
        for i in range(steps):
            self.step(i, xs, idxs, outs, prefetch)
        torch.cuda.synchronize()
        stage_ms, count = self.ctx.get_timing(reset=True)
        self.ctx.set_timing(False)
        if prefetch is not None and prefetch != "stack":
            self.ctx.set_prefetch([])
        stage_us = {k: v * 1e3 / count for k, v in stage_ms.items()}
        # distinct experts of each layer, averaged over the timed steps
        self.d_layers = [float(np.mean([len(torch.unique(idxs[i % N_INPUTS][l]))
                                        for i in range(steps)]))
                         for l in range(len(self.layers))]
        self.plan = self.ctx.last_plan()
        return ms, self.d_layers[0], stage_us


def figures(w, B, ms_per_layer, d_mean, stage_us):
    expert_bytes = d_mean * w.expert_bytes()
    layer_bytes = expert_bytes + w.router_bytes()
    expert_us = stage_us["gate_up"] + stage_us["down"]
    return dict(
        batch=B, us_per_layer=ms_per_layer * 1e3, distinct_experts=d_mean,
        algorithmic_bytes=layer_bytes,
        layer_gbps=layer_bytes / (ms_per_layer * 1e-3) / 1e9,
        layer_pct_of_peak=100 * layer_bytes / (ms_per_layer * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        expert_stream_gbps=expert_bytes / (expert_us * 1e-6) / 1e9,
        expert_stream_pct_of_peak=100 * expert_bytes / (expert_us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
        stage_us=stage_us)


def _round(d):
    if isinstance(d, float):
        return round(d, 3)
    if isinstance(d, dict):
        return {k: _round(v) for k, v in d.items()}
    return d


def gate_up_code_digest(root):
    """SHA-256 of the batch-1 gate/up kernel's sources (expert_gemv.hip, then
    moe_device.h) with comments removed and whitespace collapsed: it changes
    when the code changes, not when a comment does."""
    import hashlib
    import re
    csrc = os.path.join(root, "mixture_experts_layer_decode_amd", "csrc")
    h = hashlib.sha256()
    for name in ("expert_gemv.hip", "moe_device.h"):
        text = open(os.path.join(csrc, name)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
        h.update(b"\0")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes (fetched + written) per launch of the batch-1 gate/up kernel,
    from the committed counter summary, or None when the kernel's code has
    changed since the counters were taken (the summary records its digest)."""
    import re
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        text = open(os.path.join(root, "profiles", "hbm_traffic_full_b1.md")).read()
        nbytes = int(re.search(r"gate_up_traffic_bytes_per_launch = (\d+)", text).group(1))
        want = re.search(r"gate_up_code_sha256 = ([0-9a-f]{64})", text).group(1)
        have = gate_up_code_digest(root)
    except (OSError, AttributeError, ValueError):
        return None
    return nbytes if have == want else None


def read_ceiling(torch, dev, nbytes=4 << 30, grid=16384, reps=10):
    """Read bandwidth of a plain streaming kernel on this card (libmoe_probe.so,
    measurement only): GB/s over `reps` reads of an `nbytes` buffer, timed with
    HIP events on the stream the probe runs on."""
    import ctypes
    from mixture_experts_layer_decode_amd import build as lib_build
    lib = ctypes.CDLL(lib_build.PROBE_LIB)
    fn = lib.moe_probe_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int32
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def read():
        if fn(buf.data_ptr(), nbytes, grid, ctypes.c_void_p(stream.cuda_stream),
              sink.data_ptr()) != 0:
            raise RuntimeError("moe_probe_stream_read failed")

    for _ in range(3):
        read()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        read()
    b.record(stream)
    torch.cuda.synchronize()
    gbps = nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del buf, sink
    return {"gbps": round(gbps, 1), "bytes": nbytes, "grid": grid,
            "kernel": "stream_read_kernel (libmoe_probe.so): contiguous share per workgroup, "
                      "16 non-temporal 16-byte loads per lane in flight"}


def gate_up_bytes(w, d_mean):
    """Algorithmic bytes of the gate/up projections of d_mean experts."""
    per = 2 * w.I * w.H * (1 if w.wdt == "fp8" else 2 if w.wdt == "bf16" else 4)
    if w.wdt == "fp8":
        per += 2 * w.I * 4
    return d_mean * per


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--extra", default="verify_b8,full_b64,verify_d3,verify_d4,verify_d5,"
                                       "verify_d6,verify_8x8",
                    help="other workloads of the same layer to time ('' for none)")
    ap.add_argument("--extra-batches", dest="extra",
                    help="the same as --extra (kept for the recorded profiling commands)")
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "mfma"])
    ap.add_argument("--router", default="auto", choices=["auto", "gemv", "mfma"],
                    help="router kernel: AUTO (GEMV at one row, matrix cores above), or forced")
    ap.add_argument("--sweep", action="store_true",
                    help="also time every expert-kernel choice at batches 1, 8, 64")
    ap.add_argument("--no-stack", action="store_true", help="skip the 4-layer fp8 stack")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the timings of the same steps replayed from a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU-oracle sample budget (0 disables)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device to device 5 times (reference for HBM counters)")
    ap.add_argument("--input-step", type=int, default=None,
                    help="every timed forward takes this one input batch instead of cycling "
                         "through 16 (for counter runs)")
    args = ap.parse_args()
    global INPUT_STEP
    INPUT_STEP = args.input_step

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("this benchmark runs on one GPU: the whole MoE layer is one GPU's share, with "
               "no sharding and no collectives; run it with --gpus 1")
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
    M.load_library(build_if_missing=False)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch,
        # against 1 GiB, scales the same counters taken on the layer's kernels
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "copies": 5}))
        return 0
    path = {"auto": M.PATH_AUTO, "gemv": M.PATH_GEMV, "mfma": M.PATH_MFMA}[args.path]
    router = {"auto": M.ROUTER_AUTO, "gemv": M.ROUTER_GEMV, "mfma": M.ROUTER_MFMA}[args.router]

    w = W.WORKLOADS["full_b1"]
    t0 = time.time()
    L = W.make_layer(w, 0, device=dev)
    torch.cuda.synchronize()
    _log(f"[bench] layer {w.name} generated in {time.time() - t0:.1f}s")
    run = Runner(M, W, torch, dev, w, [L], router)

    ms, d_mean, stage_us = run.time(1, w, args.steps, args.warmup, path=path)
    head = figures(w, 1, ms, d_mean, stage_us)
    # what a kernel that only reads reaches on this card, right after the
    # headline steps (the roofline's peak stays the 8 TB/s specification)
    ceiling = read_ceiling(torch, dev)
    _log(f"[bench] plain streaming read: {ceiling['gbps']:.1f} GB/s")
    head.update(launches=run.plan["launches"], router=ROUTER_NAMES[run.plan["router"]])
    if not args.no_graph:
        head["graph_us_per_layer"] = run.time_graph(1, w, args.steps, args.warmup) * 1e3
    # per-forward distribution: back to back (warm), and with 512 MB rewritten
    # between forwards (cold: more than the 256 MB last-level cache)
    scrub = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    per_forward = {"warm": run.time_each(1, w, args.steps),
                   "cold_512MB_scrub": run.time_each(1, w, args.steps, scrub)}
    del scrub
    # the per-forward medians as layer bandwidth (the cold one is the figure
    # with nothing of the layer left in any cache)
    for v in per_forward.values():
        v["layer_gbps_p50"] = round(head["algorithmic_bytes"] / (v["p50"] * 1e-6) / 1e9, 1)
        v["pct_of_peak_p50"] = round(100 * v["layer_gbps_p50"] / PEAK_HBM_GBPS, 2)
    _log(f"[bench] B=1 per forward: {per_forward}")
    _log(f"[bench] B=1: {head['us_per_layer']:.1f} us/layer "
         f"(graph {head.get('graph_us_per_layer', 0):.1f}), D={d_mean:.1f}, stages {stage_us}")

    extra = {}
    for name in [t.strip() for t in args.extra.split(",") if t.strip()]:
        rec = W.WORKLOADS[name]
        B = rec.B
        steps = max(5, min(args.steps, 30 if B >= 32 else args.steps))
        # at least 0.2 s of untimed steps first: a short batch right after the
        # batch-1 passes otherwise starts before the card is back at speed
        msb, db, sb = run.time(B, rec, steps, min(args.warmup, 5), path=path, warm_s=0.2)
        extra[name] = figures(w, B, msb, db, sb)
        extra[name].update(launches=run.plan["launches"],
                           router=ROUTER_NAMES[run.plan["router"]])
        if not args.no_graph:
            extra[name]["graph_us_per_layer"] = run.time_graph(B, rec, steps, 5) * 1e3
        _log(f"[bench] {name} (B={B}): {extra[name]['us_per_layer']:.1f} us/layer "
             f"(graph {extra[name].get('graph_us_per_layer', 0):.1f}), D={db:.1f}, stages {sb}")

    # the small fp32 layer (hidden 512, 64 experts, top-4, softmax): its own
    # context; its 6.4 MB stay in the caches, so its bandwidth is not HBM's
    tiny = W.WORKLOADS["tiny_b1"]
    Lt = W.make_layer(tiny, 0, device=dev)
    rt = Runner(M, W, torch, dev, tiny, [Lt], router)
    mst, dt, st = rt.time(1, tiny, args.steps, args.warmup, path=path, warm_s=0.2)
    extra["tiny_b1"] = figures(tiny, 1, mst, dt, st)
    extra["tiny_b1"].update(launches=rt.plan["launches"], router=ROUTER_NAMES[rt.plan["router"]])
    if not args.no_graph:
        extra["tiny_b1"]["graph_us_per_layer"] = rt.time_graph(1, tiny, args.steps, 5) * 1e3
    rt.close()
    _log(f"[bench] tiny_b1 (B=1): {extra['tiny_b1']['us_per_layer']:.2f} us/layer, stages {st}")

    sweep = None
    if args.sweep:
        sweep = []
        choices = [("gemv", M.PATH_GEMV, 0, 0), ("mfma", M.PATH_MFMA, 0, 1),
                   ("mfma_split2", M.PATH_MFMA, 0, 2), ("mfma_split4", M.PATH_MFMA, 0, 4)] + \
                  [(f"auto_min{r}", M.PATH_AUTO, r, 1) for r in (2, 3, 4, 6, 8)]
        for B, rec in ((1, w), (8, W.WORKLOADS["verify_b8"]), (64, W.scaled(w, B=64))):
            for name, p, r, sk in choices:
                if B == 1 and name.startswith("auto"):
                    continue
                steps = 20 if B < 64 else 8
                msb, db, sb = run.time(B, rec, steps, 3, path=p, min_rows=r, split_k=sk)
                sweep.append({"batch": B, "choice": name, "us_per_layer": round(msb * 1e3, 1),
                              "stage_us": _round(sb)})
                _log(f"[sweep] B={B} {name}: {msb * 1e3:.1f} us/layer, stages {_round(sb)}")
        run.ctx.set_path(path, 1, 0)

    # roofline of the dominant kernel: gate/up (2/3 of the bytes) at batch 1.
    # A stage time runs from one HIP event to the next and so includes what
    # recording the closing event costs on the GPU (a timed event writes back
    # the caches); at batch 1 the combine stage holds no kernel (the combine
    # is folded into the down projection), so its time is that cost alone and
    # is taken off the gate/up stage
    event_us = stage_us["combine"] if head["launches"] <= 4 else 0.0
    gu_us = stage_us["gate_up"] - event_us
    gu_b = gate_up_bytes(w, d_mean)
    achieved = gu_b / (gu_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": measured_traffic() if args.path != "mfma" else None,
                "kernel": "gate_up_gemv_kernel (batch 1)", "bytes_per_launch": gu_b,
                "avg_launch_us": round(gu_us, 2),
                "stage_us_with_event": round(stage_us["gate_up"], 2),
                "event_us": round(event_us, 2),
                "frac_of_read_ceiling": round(achieved / ceiling["gbps"], 4)}

    cpu = None
    if args.cpu_seconds > 0:
        gpu_us = {"full_b1": head["us_per_layer"]}
        gpu_us.update({k: v["us_per_layer"] for k, v in extra.items()})
        cpu = cpu_baseline(w, L, dev, args.cpu_seconds, gpu_us)
        cpu["per_config"]["tiny_b1"] = oracle_time(tiny, Lt, W.make_x(tiny, 0, device=dev),
                                                   min(1.0, 0.05 * args.cpu_seconds))
        cpu["per_config"]["tiny_b1"]["gpu_us_per_layer"] = round(extra["tiny_b1"]["us_per_layer"], 2)
        cpu["one_thread"]["tiny_b1"] = oracle_time(tiny, Lt, W.make_x(tiny, 0, device=dev),
                                                   min(0.5, 0.025 * args.cpu_seconds), threads=1)
        _log(f"[bench] cpu oracle: {cpu}")
    del Lt
    run.close()
    del run, L
    gc.collect()
    torch.cuda.empty_cache()

    stack = None
    if not args.no_stack:
        stack = time_stack(M, W, torch, dev, args, router, cpu)

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
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) random-init weights)",
        "config": {"workload": w.name, "batch": 1, "hidden": w.H, "experts": w.E,
                   "topk": w.k, "inter": w.I, "weights": w.wdt, "score": w.score,
                   "path": args.path, "router": args.router},
        "hbm_gbps": round(head["layer_gbps"], 1),
        "pct_of_peak": round(head["layer_pct_of_peak"], 2),
        "expert_stream_gbps": round(head["expert_stream_gbps"], 1),
        "expert_stream_pct_of_peak": round(head["expert_stream_pct_of_peak"], 2),
        "expert_stream_pct_of_read_ceiling": round(
            100 * head["expert_stream_gbps"] / ceiling["gbps"], 2),
        "read_ceiling": ceiling,
        "distinct_experts": head["distinct_experts"],
        "launches_per_layer": head["launches"],
        "router": head["router"],
        "graph_us_per_layer": (round(head["graph_us_per_layer"], 2)
                               if "graph_us_per_layer" in head else None),
        "per_forward_us": per_forward,
        "stage_us": _round(stage_us),
        "workloads": {k: _round(v) for k, v in extra.items()},
        "stack4_fp8_b16": stack,
        "sweep": sweep,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))
    return 0


def time_stack(M, W, torch, dev, args, router, cpu=None):
    """4 consecutive fp8 layers at batch 16: layer by layer, with and without
    prefetching each next layer's router while a layer runs, and through the
    stack call, with and without each layer's combine folded into the next
    layer's router launch.  With ``cpu`` (the CPU
    baseline's record) the oracle is also timed on the first layer, on 4 of
    its 16 rows, and added to it."""
    w = W.WORKLOADS["stack4_fp8_b16"]
    t0 = time.time()
    layers = [W.make_layer(w, 0, layer=l, device=dev) for l in range(w.layers)]
    torch.cuda.synchronize()
    _log(f"[bench] stack {w.name} generated in {time.time() - t0:.1f}s")
    run = Runner(M, W, torch, dev, w, layers, router)
    res = {}
    steps = max(5, min(args.steps, 20))
    modes = (("no_prefetch", None, False), ("prefetch_router", lambda n: [n["router_w"]], False),
             ("stack_call", "stack", False), ("stack_call_folded_next_router", "stack", True))
    for name, pf, folded in modes:
        run.ctx.set_fused_next_router(folded)
        ms, d, st = run.time(w.B, w, steps, min(args.warmup, 5), path=M.PATH_AUTO, prefetch=pf)
        per_layer = ms / w.layers
        # each layer selects its own experts (later layers more of them: their
        # inputs have grown by the earlier layers' outputs), so the bytes of a
        # step are summed over the layers
        d_layers = run.d_layers
        step_bytes = sum(dl * w.expert_bytes() + w.router_bytes() for dl in d_layers)
        expert_bytes = sum(d_layers) * w.expert_bytes()
        expert_us = (st["gate_up"] + st["down"]) * w.layers
        res[name] = {"us_per_layer": round(per_layer * 1e3, 2),
                     "distinct_experts_per_layer": [round(dl, 1) for dl in d_layers],
                     "stack_gbps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                     "stack_pct_of_peak": round(100 * step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
                     "expert_stream_gbps": round(expert_bytes / (expert_us * 1e-6) / 1e9, 1),
                     "stage_us_per_layer": _round(st),
                     "launches_last_layer": run.plan["launches"]}
        _log(f"[bench] stack {name}: {per_layer * 1e3:.1f} us/layer, D per layer "
             f"{[round(dl, 1) for dl in d_layers]}, {res[name]['stack_gbps']} GB/s, stages {st}")
    if cpu is not None:
        e = oracle_time(w, layers[0], W.make_x(w, 0, device=dev), 0.2 * args.cpu_seconds,
                        sample_rows=4)
        e["gpu_us_per_layer"] = res["no_prefetch"]["us_per_layer"]
        e["sample"] += " (layer 0 of the stack)"
        cpu["per_config"]["stack4_fp8_b16_layer"] = e
        e1 = oracle_time(w, layers[0], W.make_x(w, 0, device=dev), 0.05 * args.cpu_seconds,
                         sample_rows=1, threads=1)
        e1["sample"] += " (layer 0 of the stack)"
        cpu["one_thread"]["stack4_fp8_b16_layer"] = e1
        _log(f"[bench] cpu oracle, one fp8 layer: {e}; one thread: {e1}")
    run.close()
    del run, layers
    gc.collect()
    torch.cuda.empty_cache()
    return res


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo), its logical CPUs and the ones
    this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def oracle_time(w, L, x, budget_s, sample_rows=None, threads=None):
    """The CPU oracle, unchanged, on whole layers of ``w`` (router, top-k and
    weights, each selected expert's FFN, combine) over the input x, repeated
    until ``budget_s`` seconds are spent (at least once).  With
    ``sample_rows`` only the first that many rows of x are computed and the
    time is scaled by B / sample_rows (every row costs the same: its logits,
    its k experts and its combine).  The selected experts' weights are copied
    to the host before the clock starts, so the figure is compute only.
    Returns a dict with us per layer and what was sampled."""
    import numpy as np

    import oracle
    import workloads as W

    act = {"f32": oracle.F32, "bf16": oracle.BF16}[w.act]
    wdt = {"f32": oracle.F32, "bf16": oracle.BF16, "fp8": oracle.E4M3}[w.wdt]
    score = oracle.SIGMOID if w.score == "sigmoid" else oracle.SOFTMAX
    B = x.shape[0]
    n = B if sample_rows is None else min(B, sample_rows)
    xs = W.raw_numpy(x)[:n]
    router = W.raw_numpy(L["router_w"])
    bias = W.raw_numpy(L["bias"])
    idx, _ = oracle.topk(oracle.router_logits(xs, act, router, bias), w.k, score)
    experts = {}
    for e in np.unique(idx):
        experts[int(e)] = (W.raw_numpy(L["w_gate_up"][e]), W.raw_numpy(L["w_down"][e]),
                           W.raw_numpy(L["s_gu"][e]) if L["s_gu"] is not None else None,
                           W.raw_numpy(L["s_d"][e]) if L["s_d"] is not None else None)
    prev = oracle.max_threads()
    if threads is not None:
        oracle.set_threads(threads)
    used = oracle.max_threads()
    try:
        reps, t_total = 0, 0.0
        while t_total < budget_s or reps == 0:
            t0 = time.perf_counter()
            lg = oracle.router_logits(xs, act, router, bias)
            idx, wts = oracle.topk(lg, w.k, score)
            y = np.zeros((n, w.k, w.H))
            for b in range(n):
                for j in range(w.k):
                    gu, dn, sg, sd = experts[int(idx[b, j])]
                    _, y[b, j] = oracle.expert_ffn(xs[b], act, gu, dn, wdt, sg, sd)
            oracle.combine(xs, act, wts, y)
            t_total += time.perf_counter() - t0
            reps += 1
    finally:
        oracle.set_threads(prev)
    us = t_total / reps * 1e6 * B / n
    sample = f"{reps} pass(es) over {n} of {B} rows of {w.name}"
    if n < B:
        sample += f", scaled by {B}/{n}"
    return {"us_per_layer": round(us, 1), "threads": used, "distinct_experts": len(experts),
            "sample": sample}


def cpu_baseline(w, L, dev, budget_s, gpu_us):
    """The CPU oracle timed beside the GPU figures: the batch-1 layer on all of
    the host's threads (the headline figure) and on one thread, and batches
    of 8 and 64 rows of the same layer on all threads (64 rows sampled on 4 of
    them) and on one thread (one row sampled, scaled to the batch).
    ``budget_s`` is split between the entries; gpu_us holds the GPU's us per
    layer of each workload, reported beside the oracle's."""
    import torch

    import workloads as W

    shares = {"full_b1": 0.3, "full_b1_1thread": 0.2, "verify_b8": 0.2, "full_b64": 0.2,
              "rows_1thread": 0.05}
    x1 = W.make_x(w, 0, step=0, device=dev)
    entries = {}
    entries["full_b1"] = oracle_time(w, L, x1, budget_s * shares["full_b1"])
    one = {"full_b1": oracle_time(w, L, x1, budget_s * shares["full_b1_1thread"], threads=1)}
    for name, rows in (("verify_b8", None), ("full_b64", 4)):
        rec = W.WORKLOADS[name]
        xr = W.make_x(rec, 0, step=0, device=dev)
        entries[name] = oracle_time(rec, L, xr, budget_s * shares[name], sample_rows=rows)
        one[name] = oracle_time(rec, L, xr, budget_s * shares["rows_1thread"], sample_rows=1,
                                threads=1)
    torch.cuda.synchronize()
    for name, e in entries.items():
        if name in gpu_us:
            e["gpu_us_per_layer"] = round(gpu_us[name], 2)
    head = entries["full_b1"]
    cpu = host_cpu()
    return {"value": head["us_per_layer"], "unit": "us/layer", "cores": head["threads"],
            "kind": "oracle",
            "sample": f"{head['sample']} (batch 1, input step 0), compute only (the selected "
                      f"experts copied to host beforehand), on {head['threads']} OpenMP threads",
            "cpu_model": cpu["model"], "host_logical_cpus": cpu["logical_cpus"],
            "host_usable_cpus": cpu["usable_cpus"],
            "one_thread": one,
            "per_config": entries}


if __name__ == "__main__":
    sys.exit(main())
