"""Stream semantics of the boundary: a forward is queued on the caller's
current stream and ordered with the caller's own work there; two contexts are
independent (each has its own workspace), so forwards of both may be in
flight at once on two streams; destroying a context waits for the work it
queued."""
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


def queue(ctx, w, L, x, out, idx):
    ctx.forward(x, L["router_w"], L["w_gate_up"], L["w_down"], w.k, M.SIGMOID, bias=L["bias"],
                out=out, idx_out=idx)


def test_forward_is_ordered_with_the_callers_side_stream():
    w = W.scaled(SMALL_BF16, B=8)
    L = layer(w, 91)
    x0 = W.make_x(w, 91, device="cuda")
    ctx = make_context(w)
    want = gpu_forward(ctx, w, L, x0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        # the input is produced on the side stream, and the output is read
        # there, with no synchronisation in between
        x = torch.empty_like(x0)
        x.copy_(x0)
        out = torch.empty_like(x0)
        idx = torch.full((w.B, w.k), -1, dtype=torch.int32, device="cuda")
        queue(ctx, w, L, x, out, idx)
        got = out.clone()
    torch.cuda.synchronize()
    assert torch.equal(got, want[2])
    assert np.array_equal(idx.cpu().numpy(), want[0])


def test_two_contexts_in_flight_on_two_streams():
    wa = W.scaled(SMALL_BF16, B=8)
    wb = W.scaled(SMALL_BF16, B=1, k=4, E=32)
    La, Lb = layer(wa, 92), layer(wb, 93)
    xa = [W.make_x(wa, 92, step=s, device="cuda") for s in range(4)]
    xb = [W.make_x(wb, 93, step=s, device="cuda") for s in range(4)]
    ca, cb = make_context(wa), make_context(wb)
    res_a = [gpu_forward(ca, wa, La, x) for x in xa]
    want_a = [r[2] for r in res_a]
    want_b = [gpu_forward(cb, wb, Lb, x)[2] for x in xb]
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    outs_a = [torch.empty_like(x) for x in xa]
    outs_b = [torch.empty_like(x) for x in xb]
    for i in range(4):
        with torch.cuda.stream(sa):
            queue(ca, wa, La, xa[i], outs_a[i], None)
        with torch.cuda.stream(sb):
            queue(cb, wb, Lb, xb[i], outs_b[i], None)
    torch.cuda.synchronize()
    for i in range(4):
        assert torch.equal(outs_a[i], want_a[i]), i
        assert torch.equal(outs_b[i], want_b[i]), i
    # and the last ones against the oracle
    check_layer(wa, La, xa[3], res_a[3][0], res_a[3][1], outs_a[3])


def test_close_waits_for_the_work_it_queued():
    w = W.scaled(SMALL_BF16, B=16)
    L = layer(w, 94)
    x = W.make_x(w, 94, device="cuda")
    ref_ctx = make_context(w)
    want = gpu_forward(ref_ctx, w, L, x)[2]
    ref_ctx.close()
    ctx = make_context(w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out = torch.empty_like(x)
        for _ in range(3):
            queue(ctx, w, L, x, out, None)
    ctx.close()  # frees the workspace only after the queued forwards ran
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    ctx.close()  # a second close is a no-op
    with pytest.raises(M.MoeError):
        ctx.set_timing(True)  # the handle is gone


def test_one_context_alternating_two_streams_stays_ordered():
    # one context (one workspace) fed from two streams in turn, with no
    # synchronisation by the caller: each switch orders the new stream after
    # the work queued on the old one, so every output equals the serial run
    w = W.scaled(SMALL_BF16, B=16)
    L = layer(w, 95)
    xs = [W.make_x(w, 95, step=s, device="cuda") for s in range(8)]
    ctx = make_context(w)
    want = [gpu_forward(ctx, w, L, x) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [torch.empty_like(x) for x in xs]
    idxs = [torch.full((w.B, w.k), -1, dtype=torch.int32, device="cuda") for _ in xs]
    for rnd in range(3):
        for i, x in enumerate(xs):
            with torch.cuda.stream(streams[i % 2]):
                queue(ctx, w, L, x, outs[i], idxs[i])
        torch.cuda.synchronize()
        for i in range(len(xs)):
            assert torch.equal(outs[i], want[i][2]), (rnd, i)
            assert np.array_equal(idxs[i].cpu().numpy(), want[i][0]), (rnd, i)
    ctx.close()


def test_close_after_a_stream_switch_waits_for_both_streams():
    w = W.scaled(SMALL_BF16, B=16)
    L = layer(w, 96)
    x = W.make_x(w, 96, device="cuda")
    ref_ctx = make_context(w)
    want = gpu_forward(ref_ctx, w, L, x)[2]
    ref_ctx.close()
    ctx = make_context(w)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    out_a, out_b = torch.empty_like(x), torch.empty_like(x)
    with torch.cuda.stream(sa):
        for _ in range(3):
            queue(ctx, w, L, x, out_a, None)
    with torch.cuda.stream(sb):
        queue(ctx, w, L, x, out_b, None)
    ctx.close()  # waits on sb, which waits for what sa had queued
    torch.cuda.synchronize()
    assert torch.equal(out_a, want) and torch.equal(out_b, want)
