"""GPU parity on the fp8 stack at full size: 4 consecutive layers of 896
experts (hidden 7168, top-16, SwiGLU width 2048) with OCP e4m3 weights and
per-output-row fp32 scales, a Zipf(1.1) router bias, batch 16.  Each layer
is checked against the oracle on the GPU's own input to that layer (the
previous layer's GPU output)."""
import gc

import numpy as np
import pytest
import torch

import workloads as W
from parity_helpers import full_check, make_context

pytestmark = pytest.mark.gpu

STACK = W.WORKLOADS["stack4_fp8_b16"]


@pytest.fixture(scope="module")
def stack():
    layers = [W.make_layer(STACK, 0, layer=l, device="cuda") for l in range(STACK.layers)]
    torch.cuda.synchronize()
    yield layers
    for L in layers:
        L.clear()
    layers.clear()
    gc.collect()
    torch.cuda.empty_cache()


def test_fp8_stack_teacher_forced(stack):
    ctx = make_context(STACK, max_batch=64, max_topk=16)
    x = W.make_x(STACK, 0, device="cuda")
    for l, L in enumerate(stack):
        # while layer l runs, warm the cache with layer l+1's router
        nxt = stack[l + 1] if l + 1 < len(stack) else None
        ctx.set_prefetch([nxt["router_w"]] if nxt is not None else [])
        stats, idx, out = full_check(ctx, STACK, L, x, rows=[0, 7, 15])
        plan = ctx.last_plan()
        print(f"[fp8 layer {l}] plan {plan} stats {stats}", flush=True)
        assert plan["distinct"] == len(np.unique(idx))
        x = out
    ctx.close()
