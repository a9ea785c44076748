"""Consecutive layers through moe_decode_forward_stack, with and without the
combine folded into the next layer's router launch.  Both must give the same
bits as separate forwards (the folded combine runs the combine kernel's
operations in its order), every layer must pass the oracle check on its GPU
input (teacher forcing), and the folded stack must launch one kernel fewer
per folded layer boundary."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_decode_amd as M
import workloads as W
from parity_helpers import check_layer, gpu_forward, make_context, run_stack, same_stack

pytestmark = pytest.mark.gpu

SMALL = W.scaled(W.WORKLOADS["full_b64"], H=1024, E=64, k=8, I=512)
SMALL_FP8 = W.scaled(W.WORKLOADS["stack4_fp8_b16"], H=1024, E=64, k=8, I=1024)
N_LAYERS = 3


def stack_layers(w, seed, n=N_LAYERS):
    return [{k: (v.cuda() if v is not None else None)
             for k, v in W.make_layer(w, seed, layer=l).items()} for l in range(n)]


@pytest.mark.parametrize("recipe,B,router", [
    (SMALL, 16, M.ROUTER_AUTO), (SMALL, 8, M.ROUTER_AUTO), (SMALL, 3, M.ROUTER_AUTO),
    (SMALL_FP8, 16, M.ROUTER_AUTO),     # fp8 weights with the Zipf router bias
    (SMALL, 2, M.ROUTER_MFMA),          # two rows with the matrix-core router: folded
    (SMALL, 2, M.ROUTER_AUTO),          # two rows, GEMV router: not folded
    (SMALL, 1, M.ROUTER_AUTO),          # combine folded into down instead
    (SMALL, 24, M.ROUTER_AUTO),         # beyond one 16-row tile: not folded
])
def test_stack_matches_separate_forwards_and_the_oracle(recipe, B, router):
    w = W.scaled(recipe, B=B, layers=N_LAYERS)
    layers = stack_layers(w, 81 + B)
    x = W.make_x(w, 81 + B, device="cuda")
    ctx = make_context(w)
    ctx.set_router(router)
    plain = run_stack(ctx, w, layers, x, False)
    folded = run_stack(ctx, w, layers, x, True)
    same_stack(plain, folded)
    foldable = 2 <= B <= 16 and (router == M.ROUTER_MFMA or B >= 3)
    # the last layer's router was computed by the previous layer's combine
    assert folded[3] == plain[3] - (1 if foldable else 0), (plain[3], folded[3])
    # separate forwards, layer by layer, give the same bits
    xin = x
    for l, L in enumerate(layers):
        g = gpu_forward(ctx, w, L, xin)
        assert np.array_equal(g[0], plain[0][l]) and torch.equal(g[2], plain[2][l]), l
        xin = g[2]
    # every layer against the oracle on its GPU input
    for l, L in enumerate(layers):
        xin = x if l == 0 else folded[2][l - 1]
        check_layer(w, L, xin, folded[0][l], folded[1][l], folded[2][l])


def test_stack_in_place_and_overlapping_outputs():
    # every layer written over its own input (out == x): the folded kernel
    # would read rows other workgroups overwrite, so those boundaries keep the
    # separate launches; the result is the same
    w = W.scaled(SMALL, B=16, layers=N_LAYERS)
    layers = stack_layers(w, 91)
    x = W.make_x(w, 91, device="cuda")
    ctx = make_context(w)
    plain = run_stack(ctx, w, layers, x, False)
    buf = x.clone()
    folded = run_stack(ctx, w, layers, buf, True, outs=[buf] * N_LAYERS)
    assert torch.equal(folded[2][-1], plain[2][-1])
    assert folded[3] == plain[3]


def test_stack_checks_every_layer_before_any_work():
    w = W.scaled(SMALL, B=8, layers=N_LAYERS)
    layers = stack_layers(w, 92)
    layers[2] = dict(layers[2])
    layers[2]["router_w"] = layers[2]["router_w"][:, :512]  # wrong width
    x = W.make_x(w, 92, device="cuda")
    ctx = make_context(w)
    outs = [torch.full_like(x, 7.0) for _ in range(N_LAYERS)]
    with pytest.raises(M.MoeError) as err:
        ctx.forward_stack(x, layers, w.k, M.SIGMOID, outs=outs)
    assert "layer 2" in str(err.value)
    torch.cuda.synchronize()
    assert all(bool((o == 7.0).all()) for o in outs)
