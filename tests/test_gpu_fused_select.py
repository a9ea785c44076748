"""GPU tests of the top-k selection taken inside the batch-1 gate/up kernel:
every gate/up workgroup selects the k experts from the router's logits and
workgroup 0 writes the routing outputs and the plan.  The result must be the
separate top-k kernel's bit for bit (same selection code, same weights, the
same gate/up arithmetic), with one launch fewer, for every weight type,
expert counts off the 64-lane grid, k from 1 to 32, a router bias, and tied
logits (more candidates than lanes); and it must pass the oracle check."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_decode_amd as M
import workloads as W
from parity_helpers import full_check, gpu_forward, make_context

pytestmark = pytest.mark.gpu

CASES = {
    "bf16": W.scaled(W.WORKLOADS["full_b1"], H=1024, E=64, k=16, I=2048),
    "bf16_E100_k1": W.scaled(W.WORKLOADS["full_b1"], H=1024, E=100, k=1, I=512),
    "bf16_E300_k32": W.scaled(W.WORKLOADS["full_b1"], H=512, E=300, k=32, I=512),
    "fp8_bias": W.scaled(W.WORKLOADS["stack4_fp8_b16"], B=1, H=1024, E=200, k=16, I=1024,
                         layers=1),
    "f32": W.WORKLOADS["tiny_b1"],
}


def layer(w, seed):
    return {k: (v.cuda() if v is not None else None) for k, v in W.make_layer(w, seed).items()}


def both(ctx, w, L, x):
    ctx.set_fused_select(False)
    a = gpu_forward(ctx, w, L, x)
    na = ctx.last_plan()
    ctx.set_fused_select(True)
    b = gpu_forward(ctx, w, L, x)
    nb = ctx.last_plan()
    assert nb["launches"] == na["launches"] - 1, (na, nb)
    assert nb["distinct"] == na["distinct"] == w.k and nb["gemv"] == w.k
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert torch.equal(a[2], b[2])
    return b


@pytest.mark.parametrize("name", sorted(CASES))
def test_selection_in_gate_up_is_bit_identical_and_matches_the_oracle(name):
    w = CASES[name]
    L = layer(w, 71)
    ctx = make_context(w)
    for step in range(3):
        x = W.make_x(w, 71, step=step, device="cuda")
        both(ctx, w, L, x)
        stats, _, _ = full_check(ctx, w, L, x)
        assert ctx.last_plan()["launches"] == (3 if w.k <= 16 else 4)


def test_all_tied_logits_take_the_lowest_indices():
    # a zero router ties all 300 logits: more candidates than lanes, so the
    # selection takes its wave-argmax rounds
    w = CASES["bf16_E300_k32"]
    L = layer(w, 72)
    L["router_w"].zero_()
    x = W.make_x(w, 72, device="cuda")
    ctx = make_context(w)
    idx, wt, _ = both(ctx, w, L, x)
    assert np.array_equal(idx[0], np.arange(w.k, dtype=np.int32))
    assert np.all(wt == np.float32(1.0 / w.k))


def test_matrix_core_router_keeps_the_top_k_launch():
    # the matrix-core router leaves several partial slices; the selecting
    # gate/up kernel reads one, so a forced matrix-core router at batch 1 runs
    # the separate top-k kernel
    w = CASES["bf16"]
    L = layer(w, 73)
    x = W.make_x(w, 73, device="cuda")
    ctx = make_context(w)
    ctx.set_fused_select(True)
    ctx.set_router(M.ROUTER_MFMA)
    full_check(ctx, w, L, x)
    plan = ctx.last_plan()
    assert plan["router"] == M.ROUTER_MFMA and plan["launches"] == 4, plan
