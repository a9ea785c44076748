"""The layer captured in a HIP graph: a forward enqueues only kernel launches
on the caller's stream (no allocation, no host synchronisation, no memset), so
it can be recorded once and replayed.  Each replay must reproduce, bit for
bit, the eager forward of the same input, with eager forwards of other inputs
and host synchronisations in between, and the replayed results must pass the
oracle check."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_decode_amd as M
import workloads as W
from parity_helpers import check_layer, gpu_forward, make_context

pytestmark = pytest.mark.gpu

SMALL_BF16 = W.scaled(W.WORKLOADS["full_b64"], H=1024, E=64, k=8, I=512)


def layer(w, seed):
    return {k: (v.cuda() if v is not None else None) for k, v in W.make_layer(w, seed).items()}


@pytest.mark.parametrize("B,path", [(1, M.PATH_AUTO), (8, M.PATH_AUTO), (64, M.PATH_AUTO),
                                    (24, M.PATH_GEMV)])
def test_graph_replays_match_eager_forwards(B, path):
    w = W.scaled(SMALL_BF16, B=B)
    L = layer(w, 51)
    xs = [W.make_x(w, 51, step=s, device="cuda") for s in range(3)]
    ctx = make_context(w)
    ctx.set_path(path)
    eager = [gpu_forward(ctx, w, L, x) for x in xs]

    x_static = xs[0].clone()
    out_static = torch.empty_like(x_static)
    idx_static = torch.full((B, w.k), -1, dtype=torch.int32, device="cuda")
    wt_static = torch.zeros((B, w.k), dtype=torch.float32, device="cuda")

    def fwd():
        ctx.forward(x_static, L["router_w"], L["w_gate_up"], L["w_down"], w.k, M.SIGMOID,
                    bias=L["bias"], out=out_static, idx_out=idx_static, weight_out=wt_static)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    torch.cuda.synchronize()

    for rep in range(2):
        for i, x in enumerate(xs):
            x_static.copy_(x)
            out_static.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            want_idx, want_w, want_out = eager[i]
            assert np.array_equal(idx_static.cpu().numpy(), want_idx), (rep, i)
            assert np.array_equal(wt_static.cpu().numpy(), want_w), (rep, i)
            assert torch.equal(out_static, want_out), (rep, i)
            # eager work of another input between replays
            gpu_forward(ctx, w, L, xs[(i + 1) % len(xs)])

    # the replayed result of the last input against the oracle
    x_static.copy_(xs[2])
    g.replay()
    torch.cuda.synchronize()
    rows = sorted({0, B - 1})
    check_layer(w, L, xs[2], idx_static.cpu().numpy(), wt_static.cpu().numpy(), out_static,
                rows=rows)
