"""GPU parity of the two router kernels (vector-unit GEMV and fp64 matrix
cores): each forced on its own against the CPU oracle, at batch sizes that
give one, several and ragged 16-row tiles, for bf16 and fp32 activations and
for a wide router; both against each other; and dyadic inputs whose logits are
exact in any summation order, so that the selection, ties included, must be
the oracle's exactly."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_decode_amd as M
import workloads as W
from parity_helpers import check_layer, full_check, gpu_forward, make_context, oracle_layer

pytestmark = pytest.mark.gpu

SMALL_BF16 = W.scaled(W.WORKLOADS["full_b64"], H=1024, E=64, k=8, I=512)
ROUTERS = {"gemv": M.ROUTER_GEMV, "mfma": M.ROUTER_MFMA}


def layer(w, seed, layer_id=0):
    return {k: (v.cuda() if v is not None else None)
            for k, v in W.make_layer(w, seed, layer_id).items()}


@pytest.mark.parametrize("router", sorted(ROUTERS))
@pytest.mark.parametrize("B", [1, 2, 5, 16, 17, 40, 64])
def test_router_kernels_match_the_oracle(router, B):
    w = W.scaled(SMALL_BF16, B=B)
    L = layer(w, 41)
    x = W.make_x(w, 41, device="cuda")
    ctx = make_context(w)
    ctx.set_router(ROUTERS[router])
    full_check(ctx, w, L, x, rows=sorted({0, B // 2, B - 1}))


@pytest.mark.parametrize("router", sorted(ROUTERS))
def test_fp32_activations_and_softmax(router):
    w = W.scaled(W.WORKLOADS["tiny_b1"], B=9)
    L = layer(w, 42)
    x = W.make_x(w, 42, device="cuda")
    ctx = make_context(w)
    ctx.set_router(ROUTERS[router])
    full_check(ctx, w, L, x)


def test_wide_router_on_matrix_cores():
    w = W.scaled(SMALL_BF16, B=21, E=2048, k=32, H=512, I=512)
    L = layer(w, 43)
    x = W.make_x(w, 43, device="cuda")
    ctx = make_context(w)
    ctx.set_router(M.ROUTER_MFMA)
    full_check(ctx, w, L, x, rows=[0, 20])


def test_router_kernels_agree_with_each_other():
    w = W.scaled(SMALL_BF16, B=64)
    L = layer(w, 44)
    x = W.make_x(w, 44, device="cuda")
    ctx = make_context(w)
    ctx.set_router(M.ROUTER_GEMV)
    a = gpu_forward(ctx, w, L, x)
    ctx.set_router(M.ROUTER_MFMA)
    b = gpu_forward(ctx, w, L, x)
    # fp64 sums in two orders: equal selections unless two logits lie within
    # a few fp64 ulps, which these random inputs never produce
    assert np.array_equal(a[0], b[0])
    assert np.max(np.abs(a[1] - b[1])) <= 1e-6
    if np.array_equal(a[1], b[1]):
        assert torch.equal(a[2], b[2])


def dyadic_layer(w, seed):
    """Router weights n / 1024 with |n| < 256 and activations in {-2..2}: every
    product and partial sum is a multiple of 2^-10 below 2^10, exact in fp64
    in any order, and logits tie often."""
    L = layer(w, seed)
    g = torch.Generator().manual_seed(seed)
    n = torch.randint(-255, 256, (w.E, w.H), generator=g, dtype=torch.int32)
    # duplicate some router rows onto other experts: exact ties between
    # different expert indices
    n[1::7] = n[0::7][: n[1::7].shape[0]]
    L["router_w"] = (n.to(torch.float32) / 1024.0).cuda()
    xi = torch.randint(-2, 3, (w.B, w.H), generator=g, dtype=torch.int32)
    x = xi.to(torch.bfloat16).cuda()
    return L, x


@pytest.mark.parametrize("router", sorted(ROUTERS))
def test_dyadic_logits_select_exactly_the_oracles_experts(router):
    w = W.scaled(SMALL_BF16, B=33)
    L, x = dyadic_layer(w, 45)
    ctx = make_context(w)
    ctx.set_router(ROUTERS[router])
    idx, wt, out = gpu_forward(ctx, w, L, x)
    lg, idx_o, w_o, _ = oracle_layer(w, L, x, rows=[])
    assert np.array_equal(idx, idx_o)
    assert np.max(np.abs(wt - w_o)) <= 1e-6
    check_layer(w, L, x, idx, wt, out, rows=[0, 16, 32])


def test_dyadic_routing_is_identical_on_both_kernels():
    w = W.scaled(SMALL_BF16, B=64)
    L, x = dyadic_layer(w, 46)
    ctx = make_context(w)
    ctx.set_router(M.ROUTER_GEMV)
    a = gpu_forward(ctx, w, L, x)
    ctx.set_router(M.ROUTER_MFMA)
    b = gpu_forward(ctx, w, L, x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert torch.equal(a[2], b[2])


def test_set_router_rejects_unknown_kernels():
    w = W.scaled(SMALL_BF16, B=2)
    ctx = make_context(w)
    for bad in (-1, 3):
        with pytest.raises(M.MoeError) as ei:
            ctx.set_router(bad)
        assert ei.value.status == M.binding.ERR_INVALID_ARG


@pytest.mark.parametrize("B,split,router,launches", [(1, 0, M.ROUTER_GEMV, 4),
                                                     (2, 0, M.ROUTER_GEMV, 5),
                                                     (3, 0, M.ROUTER_MFMA, 5),
                                                     (8, 0, M.ROUTER_MFMA, 5),
                                                     (24, 0, M.ROUTER_MFMA, 6),
                                                     (24, 2, M.ROUTER_MFMA, 8)])
def test_last_plan_reports_router_and_launch_count(B, split, router, launches):
    # AUTO: GEMV router at one and two rows, matrix cores above; top-k with the
    # buckets in one kernel up to 8 rows, a separate bucket kernel above; one
    # kernel per expert stage, two with split-K; then the combine, which at
    # one row is folded into the down projection
    w = W.scaled(SMALL_BF16, B=B)
    L = layer(w, 47)
    x = W.make_x(w, 47, device="cuda")
    ctx = make_context(w)
    ctx.set_path(M.PATH_AUTO, split_k=split)
    gpu_forward(ctx, w, L, x)
    plan = ctx.last_plan()
    assert plan["router"] == router and plan["launches"] == launches, plan


@pytest.mark.parametrize("wl", ["full_b64", "tiny_b1"])
def test_one_row_router_kernel_matches_the_multi_row_kernel_bitwise(wl):
    # batch 1 runs its own GEMV router kernel; a batch of two identical rows
    # runs the multi-row one.  Same arithmetic order, so the same logits:
    # identical experts and bit-identical routing weights.
    base = W.WORKLOADS[wl]
    w = W.scaled(SMALL_BF16, B=1) if wl == "full_b64" else W.scaled(base, B=1)
    L = layer(w, 48)
    x1 = W.make_x(w, 48, device="cuda")
    ctx = make_context(w, max_batch=2)
    ctx.set_router(M.ROUTER_GEMV)
    a = gpu_forward(ctx, w, L, x1)
    w2 = W.scaled(w, B=2)
    b = gpu_forward(ctx, w2, L, x1.expand(2, w.H).contiguous())
    assert np.array_equal(a[0][0], b[0][0]) and np.array_equal(a[1][0], b[1][0])
    assert np.array_equal(b[0][0], b[0][1]) and np.array_equal(b[1][0], b[1][1])
