"""Seeded synthetic inputs for the decode-step MoE layer.

This module holds only input recipes (shapes, value distributions, storage
types); it does none of the layer's arithmetic.  Both the GPU path's tests
and the CPU oracle consume what it produces: the oracle always reads back the
exact bytes the GPU was given.

Recipes (all values drawn from torch's seeded generators):
  * weights ~ N(0, 0.02) (0.02 is the standard deviation), drawn in fp32 and
    rounded once, nearest-even, to the storage type;
  * fp8 weights: per output row, scale = max|w| / 448 and
    code = RNE(w / scale) in OCP e4m3 (torch.float8_e4m3fn), so every row
    uses the full e4m3 range; the fp32 scale is stored beside it;
  * router ~ N(0, 0.02) in fp32;
  * x ~ N(0, 1) drawn in fp32, rounded once to the activation type;
  * correlated rows (speculative-verify shape): one shared base N(0,1) row plus
    an independent 0.3 * N(0,1) per row, summed in fp32, rounded once; with
    several sequences in one batch, each group of `group` consecutive rows
    (one sequence's token and drafts) has its own base;
  * Zipf(1.1) expert bias: bias[e] = -1.1 * ln(1 + pi(e)) with pi a seeded
    permutation of 0..E-1, one per layer; it adds s^-1.1 popularity to the
    expert of popularity rank s.

The decode shape is the one the pages give for Kimi K3: every token picks 16
of 896 experts (ailookout.news, "vLLM speeds up Kimi K3 up to 1.9x on NVIDIA
GB300 with agent-assisted kernels", section "How the specialised decode path
works").  The pages publish neither the hidden nor the expert width; 7168 and
2048 stand in for them.  Decode batches run from 1 to 64 (spectrumweb.co,
"vLLM and NVIDIA use coding agents to nearly double Kimi K3 decode speed, then
rethink how to review it");
the 8-row verify shape is 1 token + 7 draft tokens (same page, DSpark with
seven draft tokens).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch

ACT_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}
W_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
FP8_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int           # rows (tokens) in the decode batch
    H: int           # hidden width
    E: int           # experts
    k: int           # experts per token
    I: int           # expert SwiGLU intermediate width
    act: str         # activation storage: "f32" | "bf16"
    wdt: str         # expert weight storage: "f32" | "bf16" | "fp8"
    score: str       # "softmax" | "sigmoid"
    x_kind: str = "normal"          # "normal" | "correlated"
    group: int = 0                  # correlated: rows per sequence (0: all rows)
    bias: Optional[str] = None      # None | "zipf"
    layers: int = 1
    w_std: float = 0.02

    def expert_bytes(self) -> int:
        """Bytes of one expert's weights (and fp8 scales)."""
        if self.wdt == "fp8":
            return 3 * self.H * self.I + (2 * self.I + self.H) * 4
        return 3 * self.H * self.I * (4 if self.wdt == "f32" else 2)

    def router_bytes(self) -> int:
        return self.E * self.H * 4


_FULL = dict(H=7168, E=896, k=16, I=2048, act="bf16", wdt="bf16", score="sigmoid")

WORKLOADS = {
    # small layer, fp32 everywhere, softmax routing
    "tiny_b1": Workload("tiny_b1", B=1, H=512, E=64, k=4, I=256, act="f32", wdt="f32",
                        score="softmax"),
    # full-size layer, batch 1 (the headline decode shape)
    "full_b1": Workload("full_b1", B=1, **_FULL),
    # speculative verify: 1 token + 7 drafts of one sequence, correlated rows
    "verify_b8": Workload("verify_b8", B=8, x_kind="correlated", **_FULL),
    # 64 independent tokens
    "full_b64": Workload("full_b64", B=64, **_FULL),
    # speculative verify with 3 to 7 draft tokens: 1 + d correlated rows
    **{f"verify_d{d}": Workload(f"verify_d{d}", B=1 + d, x_kind="correlated", **_FULL)
       for d in range(3, 8)},
    # 8 sequences verified together, 1 token + 7 drafts each (64 rows)
    "verify_8x8": Workload("verify_8x8", B=64, x_kind="correlated", group=8, **_FULL),
    # 4 consecutive layers, fp8 e4m3 experts with per-row scales, Zipf bias
    "stack4_fp8_b16": Workload("stack4_fp8_b16", B=16, layers=4, bias="zipf",
                               **{**_FULL, "wdt": "fp8"}),
}


def scaled(w: Workload, **kw) -> Workload:
    """The same recipe at other sizes (for oracle-sized parity cases)."""
    return replace(w, **kw)


def _seed(seed: int, layer: int, tensor: int) -> int:
    return (seed * 1_000_003 + layer * 10_007 + tensor) & 0x7FFF_FFFF_FFFF


def _gen(device, seed: int, layer: int, tensor: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, layer, tensor))
    return g


def make_x(w: Workload, seed: int, step: int = 0, device="cpu", B: Optional[int] = None):
    """Input rows [B, H] in the activation type.  ``step`` picks another batch
    of the same recipe (a new decode step)."""
    B = w.B if B is None else B
    g = _gen("cpu", seed, 1000 + step, 1)
    if w.x_kind == "correlated":
        group = w.group if w.group > 0 else B
        n_seq = (B + group - 1) // group
        base = torch.randn(n_seq, w.H, generator=g, dtype=torch.float32)
        noise = torch.randn(B, w.H, generator=g, dtype=torch.float32)
        seq = torch.arange(B) // group
        xf = base[seq] + 0.3 * noise
    else:
        xf = torch.randn(B, w.H, generator=g, dtype=torch.float32)
    return xf.to(ACT_TORCH[w.act]).to(device)


def _fill_normal(dst: torch.Tensor, g: torch.Generator, std: float, chunk_rows: int):
    """dst[e] = N(0, std) rounded to dst's type, generated chunk by chunk."""
    E = dst.shape[0]
    for e0 in range(0, E, chunk_rows):
        e1 = min(E, e0 + chunk_rows)
        t = torch.randn((e1 - e0,) + tuple(dst.shape[1:]), generator=g, device=dst.device,
                        dtype=torch.float32)
        t.mul_(std)
        dst[e0:e1].copy_(t.to(dst.dtype))
        del t


def _fill_fp8(codes: torch.Tensor, scales: torch.Tensor, g: torch.Generator, std: float,
              chunk_rows: int):
    """codes[e] = e4m3(w / scale), scales[e] = max|w_row| / 448 per output row."""
    E = codes.shape[0]
    for e0 in range(0, E, chunk_rows):
        e1 = min(E, e0 + chunk_rows)
        t = torch.randn((e1 - e0,) + tuple(codes.shape[1:]), generator=g, device=codes.device,
                        dtype=torch.float32)
        t.mul_(std)
        s = t.abs().amax(dim=-1) / FP8_MAX
        q = (t / s.unsqueeze(-1)).to(torch.float8_e4m3fn).view(torch.uint8)
        codes[e0:e1].copy_(q)
        scales[e0:e1].copy_(s)
        del t, q


def make_layer(w: Workload, seed: int, layer: int = 0, device="cpu", expert_device=None):
    """One layer's parameters.

    router_w [E,H] f32 and bias [E] f32 (or None) are drawn on the CPU and moved
    to ``device``; the expert weights are drawn directly on ``expert_device``
    (default: ``device``) because the full layer is tens of GB.

    Returns a dict: router_w, bias, w_gate_up [E,2I,H], w_down [E,H,I],
    s_gu [E,2I] / s_d [E,H] (fp8 only, else None).  Rows 0..I-1 of each
    w_gate_up[e] are the gate projection, rows I..2I-1 the up projection.
    fp8 weights are raw uint8 e4m3 codes.
    """
    expert_device = device if expert_device is None else expert_device
    g = _gen("cpu", seed, layer, 2)
    router = (torch.randn(w.E, w.H, generator=g, dtype=torch.float32) * w.w_std).to(device)
    bias = None
    if w.bias == "zipf":
        gp = _gen("cpu", seed, layer, 3)
        pi = torch.randperm(w.E, generator=gp).to(torch.float64)
        bias = (-1.1 * torch.log1p(pi)).to(torch.float32).to(device)

    per_expert = 2 * w.I * w.H * (4 if w.wdt == "f32" else 2 if w.wdt == "bf16" else 1)
    chunk = max(1, min(w.E, (1 << 30) // max(1, per_expert)))
    gu = torch.empty((w.E, 2 * w.I, w.H), dtype=W_TORCH[w.wdt], device=expert_device)
    dn = torch.empty((w.E, w.H, w.I), dtype=W_TORCH[w.wdt], device=expert_device)
    s_gu = s_d = None
    g_gu = _gen(expert_device, seed, layer, 4)
    g_dn = _gen(expert_device, seed, layer, 5)
    if w.wdt == "fp8":
        s_gu = torch.empty((w.E, 2 * w.I), dtype=torch.float32, device=expert_device)
        s_d = torch.empty((w.E, w.H), dtype=torch.float32, device=expert_device)
        _fill_fp8(gu, s_gu, g_gu, w.w_std, chunk)
        _fill_fp8(dn, s_d, g_dn, w.w_std, chunk)
    else:
        _fill_normal(gu, g_gu, w.w_std, chunk)
        _fill_normal(dn, g_dn, w.w_std, chunk)
    return dict(router_w=router, bias=bias, w_gate_up=gu, w_down=dn, s_gu=s_gu, s_d=s_d)


def raw_numpy(t: Optional[torch.Tensor]):
    """Host numpy copy of a tensor's raw storage (bf16 as uint16 bits)."""
    if t is None:
        return None
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def gib(nbytes: int) -> float:
    return nbytes / math.pow(2, 30)
