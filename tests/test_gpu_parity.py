"""GPU parity at oracle-sized shapes: the HIP path through the C ABI against
the CPU oracle, element by element, plus edge cases and error paths."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_layer_decode_amd as M
import workloads as W
from mixture_experts_layer_decode_amd import binding
from parity_helpers import MOE_SCORE, check_layer, full_check, gpu_forward, make_context

pytestmark = pytest.mark.gpu

TINY = W.WORKLOADS["tiny_b1"]
# the full layer's recipe at sizes the oracle finishes in seconds
SMALL_BF16 = W.scaled(W.WORKLOADS["full_b64"], H=1024, E=64, k=8, I=512)
SMALL_VERIFY = W.scaled(W.WORKLOADS["verify_b8"], H=1024, E=64, k=8, I=512)
SMALL_FP8 = W.scaled(W.WORKLOADS["stack4_fp8_b16"], H=1024, E=64, k=8, I=1024, layers=1)


def layer(w, seed, layer_id=0):
    return {k: (v.cuda() if v is not None else None)
            for k, v in W.make_layer(w, seed, layer_id).items()}


@pytest.mark.parametrize("seed", range(5))
def test_tiny_b1(seed):
    L = layer(TINY, seed)
    x = W.make_x(TINY, seed, device="cuda")
    ctx = make_context(TINY)
    stats, idx, _ = full_check(ctx, TINY, L, x)
    assert stats["excused_rows"] == []


@pytest.mark.parametrize("B", [2, 5, 64])
def test_tiny_recipe_batches(B):
    w = W.scaled(TINY, B=B)
    L = layer(w, 11)
    x = W.make_x(w, 11, device="cuda")
    ctx = make_context(w)
    full_check(ctx, w, L, x)


@pytest.mark.parametrize("B", [1, 2, 3, 8, 17, 64])
def test_bf16_small_batches(B):
    w = W.scaled(SMALL_BF16, B=B)
    L = layer(w, 3)
    x = W.make_x(w, 3, device="cuda")
    ctx = make_context(w)
    full_check(ctx, w, L, x)
    plan = ctx.last_plan()
    assert 1 <= plan["distinct"] <= min(B * w.k, w.E)
    assert plan["gemv"] + plan["mfma"] == plan["distinct"]


def test_verify_rows_correlated():
    L = layer(SMALL_VERIFY, 4)
    x = W.make_x(SMALL_VERIFY, 4, device="cuda")
    ctx = make_context(SMALL_VERIFY)
    _, idx, _ = full_check(ctx, SMALL_VERIFY, L, x)
    # correlated rows share experts: far fewer than B*k distinct
    assert len(np.unique(idx)) < SMALL_VERIFY.B * SMALL_VERIFY.k


@pytest.mark.parametrize("B", [1, 16])
def test_fp8_small_zipf(B):
    w = W.scaled(SMALL_FP8, B=B)
    L = layer(w, 5)
    x = W.make_x(w, 5, device="cuda")
    ctx = make_context(w)
    full_check(ctx, w, L, x)


def test_rerun_is_bitwise_deterministic():
    w = W.scaled(SMALL_BF16, B=17)
    L = layer(w, 6)
    x = W.make_x(w, 6, device="cuda")
    ctx = make_context(w)
    a = gpu_forward(ctx, w, L, x)
    b = gpu_forward(ctx, w, L, x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert torch.equal(a[2], b[2])


def test_rows_alone_match_rows_in_a_batch():
    w = W.scaled(SMALL_BF16, B=8)
    L = layer(w, 7)
    x = W.make_x(w, 7, device="cuda")
    ctx = make_context(w)
    ctx.set_path(M.PATH_GEMV)
    idx_all, w_all, out_all = gpu_forward(ctx, w, L, x)
    for b in (0, 3, 7):
        xb = x[b:b + 1].contiguous()
        idx1, w1, out1 = gpu_forward(ctx, w, L, xb)
        assert np.array_equal(idx1[0], idx_all[b])
        assert np.array_equal(w1[0], w_all[b])
        # the same per-row arithmetic on the GEMV kernels: identical bits
        assert torch.equal(out1[0], out_all[b])


def test_out_may_alias_x():
    w = W.scaled(SMALL_BF16, B=4)
    L = layer(w, 8)
    x = W.make_x(w, 8, device="cuda")
    ctx = make_context(w)
    _, _, ref = gpu_forward(ctx, w, L, x)
    xin = x.clone()
    gpu_forward(ctx, w, L, xin, out=xin)
    assert torch.equal(xin, ref)


def test_duplicate_router_rows_tie_to_lower_index():
    w = W.scaled(SMALL_BF16, B=4)
    L = layer(w, 9)
    x = W.make_x(w, 9, device="cuda")
    ctx = make_context(w)
    idx0, _, _ = gpu_forward(ctx, w, L, x)
    # copy each row's top expert onto a higher and a lower index: exact ties
    r = L["router_w"]
    top = int(idx0[0, 0])
    for other in [e for e in (top - 1, top + 1, top + 2) if 0 <= e < w.E][:2]:
        r[other] = r[top]
    idx_g, w_g, out_g = gpu_forward(ctx, w, L, x)
    stats = check_layer(w, L, x, idx_g, w_g, out_g)
    assert stats["excused_rows"] == []


def test_forward_without_routing_outputs_and_bound_context():
    w = W.scaled(SMALL_BF16, B=3)
    L = layer(w, 10)
    x = W.make_x(w, 10, device="cuda")
    ctx = make_context(w)
    _, _, ref = gpu_forward(ctx, w, L, x)
    out = torch.empty_like(x)
    ctx.bind()
    ctx.forward(x, L["router_w"], L["w_gate_up"], L["w_down"], w.k, MOE_SCORE[w.score],
                out=out, use_bound=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_errors_are_reported_before_any_work():
    w = W.scaled(SMALL_BF16, B=4)
    L = layer(w, 12)
    x = W.make_x(w, 12, device="cuda")
    ctx = make_context(w)
    sentinel = torch.full_like(x, 7.0)

    def call(**kw):
        args = dict(x=x, router_w=L["router_w"], w_gate_up=L["w_gate_up"], w_down=L["w_down"],
                    k=w.k, score_fn=M.SIGMOID, out=sentinel)
        args.update(kw)
        with pytest.raises(M.MoeError) as ei:
            ctx.forward(**args)
        return ei.value.status

    big = W.make_x(w, 12, device="cuda", B=5)           # beyond the context's max_batch
    assert call(x=big, out=torch.empty_like(big)) == binding.ERR_UNSUPPORTED
    empty = x[:0]                                        # an empty batch
    assert call(x=empty, out=torch.empty_like(empty)) == binding.ERR_UNSUPPORTED
    assert call(k=w.k + 1) == binding.ERR_UNSUPPORTED    # beyond max_topk
    assert call(score_fn=5) == binding.ERR_INVALID_ARG
    assert call(x=x.float(), out=sentinel.float()) == binding.ERR_UNSUPPORTED
    assert call(out=x[1:]) == binding.ERR_INVALID_ARG     # wrong shape
    wide = torch.zeros(4, w.H + 8, dtype=x.dtype, device="cuda")
    assert call(x=wide[:, 1:w.H + 1]) == binding.ERR_INVALID_ARG  # misaligned rows
    buf = torch.zeros(5, w.H, dtype=x.dtype, device="cuda")
    buf[:4] = x
    assert call(x=buf[:4], out=buf[1:5]) == binding.ERR_INVALID_ARG  # partial overlap
    s_fake = torch.ones(w.E, 2 * w.I, device="cuda")
    assert call(s_gu=s_fake, s_d=s_fake) == binding.ERR_INVALID_ARG  # scales without fp8
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)                      # nothing was queued


def test_timing_and_plan_counters():
    w = W.scaled(SMALL_BF16, B=8)
    L = layer(w, 13)
    x = W.make_x(w, 13, device="cuda")
    ctx = make_context(w)
    ctx.set_timing(True)
    for _ in range(3):
        gpu_forward(ctx, w, L, x)
    ms, n = ctx.get_timing(reset=True)
    assert n == 3 and all(v > 0 for v in ms.values()), ms
    idx, _, _ = gpu_forward(ctx, w, L, x)
    plan = ctx.last_plan()
    assert plan["distinct"] == len(np.unique(idx))
    counts = np.bincount(idx.ravel(), minlength=w.E)
    assert plan["max_rows"] == counts.max()
