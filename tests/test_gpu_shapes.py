"""GPU parity on less common shapes and layouts: one expert (the layer is then
a dense SwiGLU FFN with routing weight exactly 1), top-1 routing, expert
counts that are not multiples of the 16-expert router tile or of the 64-lane
wave, and activation / output rows with a stride larger than the row."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_decode_amd as M
import workloads as W
from parity_helpers import full_check, gpu_forward, make_context

pytestmark = pytest.mark.gpu

SMALL_BF16 = W.scaled(W.WORKLOADS["full_b64"], H=1024, E=64, k=8, I=512)
ROUTERS = {"gemv": M.ROUTER_GEMV, "mfma": M.ROUTER_MFMA}


def layer(w, seed):
    return {k: (v.cuda() if v is not None else None) for k, v in W.make_layer(w, seed).items()}


@pytest.mark.parametrize("B,path", [(1, M.PATH_AUTO), (7, M.PATH_AUTO), (33, M.PATH_GEMV),
                                    (33, M.PATH_MFMA)])
def test_one_expert_is_a_dense_ffn(B, path):
    w = W.scaled(SMALL_BF16, B=B, E=1, k=1)
    L = layer(w, 81)
    x = W.make_x(w, 81, device="cuda")
    ctx = make_context(w)
    ctx.set_path(path)
    _, idx, _ = full_check(ctx, w, L, x, rows=sorted({0, B - 1}))
    assert np.all(idx == 0)
    wt = gpu_forward(ctx, w, L, x)[1]
    assert np.all(wt == np.float32(1.0))


@pytest.mark.parametrize("router", sorted(ROUTERS))
@pytest.mark.parametrize("E,k", [(33, 1), (100, 3), (100, 7), (17, 16)])
@pytest.mark.parametrize("B", [1, 9, 40])
def test_expert_counts_off_the_tiles(router, E, k, B):
    w = W.scaled(SMALL_BF16, B=B, E=E, k=k)
    L = layer(w, 82)
    x = W.make_x(w, 82, device="cuda")
    ctx = make_context(w)
    ctx.set_router(ROUTERS[router])
    full_check(ctx, w, L, x, rows=sorted({0, B // 2, B - 1}))


@pytest.mark.parametrize("E,B,path", [(16, 1, M.PATH_AUTO), (16, 5, M.PATH_MFMA), (32, 3, M.PATH_GEMV),
                                      (32, 64, M.PATH_AUTO)])
def test_every_expert_selected(E, B, path):
    # k = E: every row selects all experts, in logit order, and the weights
    # are the normalised scores of all of them
    w = W.scaled(SMALL_BF16, B=B, E=E, k=E)
    L = layer(w, 84)
    x = W.make_x(w, 84, device="cuda")
    ctx = make_context(w)
    ctx.set_path(path)
    _, idx, _ = full_check(ctx, w, L, x, rows=sorted({0, B // 2, B - 1}))
    assert all(sorted(row) == list(range(E)) for row in idx.tolist())
    plan = ctx.last_plan()
    assert plan["distinct"] == E and plan["max_rows"] == B


@pytest.mark.parametrize("B", [1, 6, 24])
def test_strided_rows_give_the_contiguous_result(B):
    w = W.scaled(SMALL_BF16, B=B)
    L = layer(w, 83)
    x = W.make_x(w, 83, device="cuda")
    ctx = make_context(w)
    want = gpu_forward(ctx, w, L, x)
    pad = 512
    xs = torch.zeros((B, w.H + pad), dtype=x.dtype, device="cuda")
    xs[:, :w.H] = x
    outs = torch.full((B, w.H + pad), 7.0, dtype=x.dtype, device="cuda")
    got = gpu_forward(ctx, w, L, xs[:, :w.H], out=outs[:, :w.H])
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    assert torch.equal(outs[:, :w.H], want[2])
    assert torch.all(outs[:, w.H:] == 7.0)  # nothing written past the rows
