"""GPU tests of the combine folded into the down projection at batch 1: the
folded kernel must give the separate kernels' output bit for bit (same
per-lane order, same butterfly, same combine order), for every weight type,
with out aliasing x, and must pass the oracle check; shapes it does not serve
fall back to the separate kernels."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_decode_amd as M
import workloads as W
from parity_helpers import full_check, gpu_forward, make_context

pytestmark = pytest.mark.gpu

CASES = {
    "bf16": W.scaled(W.WORKLOADS["full_b1"], H=1024, E=64, k=16, I=2048),
    "bf16_k8": W.scaled(W.WORKLOADS["full_b1"], H=1536, E=64, k=8, I=1024),
    "fp8": W.scaled(W.WORKLOADS["stack4_fp8_b16"], B=1, H=1024, E=64, k=16, I=2048, layers=1),
    "f32": W.WORKLOADS["tiny_b1"],
}


def layer(w, seed):
    return {k: (v.cuda() if v is not None else None) for k, v in W.make_layer(w, seed).items()}


def context(w):
    # the top-k stays its own launch here, so that the launch counts below
    # count the combine alone
    ctx = make_context(w)
    ctx.set_fused_select(False)
    return ctx


@pytest.mark.parametrize("name", sorted(CASES))
def test_folded_combine_is_bit_identical_and_matches_the_oracle(name):
    w = CASES[name]
    L = layer(w, 61)
    ctx = context(w)
    for step in range(3):
        x = W.make_x(w, 61, step=step, device="cuda")
        ctx.set_fused_combine(False)
        a = gpu_forward(ctx, w, L, x)
        assert ctx.last_plan()["launches"] == 5
        ctx.set_fused_combine(True)
        b = gpu_forward(ctx, w, L, x)
        assert ctx.last_plan()["launches"] == 4
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert torch.equal(a[2], b[2]), (name, step)
    full_check(ctx, w, L, x)


def test_folded_combine_with_out_aliasing_x():
    w = CASES["bf16"]
    L = layer(w, 62)
    x = W.make_x(w, 62, device="cuda")
    ctx = context(w)
    want = gpu_forward(ctx, w, L, x.clone())[2]
    y = x.clone()
    gpu_forward(ctx, w, L, y, out=y)
    assert torch.equal(y, want)


@pytest.mark.parametrize("shape", [dict(k=32, E=64), dict(I=4096)])
def test_shapes_the_folded_kernel_does_not_serve_fall_back(shape):
    # k above 16, or a bf16 down row longer than 2048: separate kernels
    w = W.scaled(CASES["bf16"], **shape)
    L = layer(w, 63)
    x = W.make_x(w, 63, device="cuda")
    ctx = context(w)
    full_check(ctx, w, L, x)
    assert ctx.last_plan()["launches"] == 5
