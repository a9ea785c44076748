"""GPU parity of the split-K MFMA expert kernels and of the exact top-k, at
oracle-sized shapes: every expert forced onto the matrix-core kernels, with
and without K splits, against the CPU oracle; GEMV and MFMA paths on the same
inputs; experts with more than one 16-row M tile; degenerate routing ties."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_decode_amd as M
import workloads as W
from parity_helpers import check_layer, full_check, gpu_forward, make_context

pytestmark = pytest.mark.gpu

# the full layer's recipe at sizes the oracle finishes in seconds: several
# 128-wide K blocks, several 32-row N blocks, ragged per-expert row counts
SMALL_BF16 = W.scaled(W.WORKLOADS["full_b64"], H=1024, E=64, k=8, I=512)
SMALL_FP8 = W.scaled(W.WORKLOADS["stack4_fp8_b16"], H=1024, E=64, k=8, I=1024, layers=1)


def layer(w, seed, layer_id=0):
    return {k: (v.cuda() if v is not None else None)
            for k, v in W.make_layer(w, seed, layer_id).items()}


@pytest.mark.parametrize("B", [1, 3, 17, 64])
@pytest.mark.parametrize("split_k", [1, 2, 3, 7])
def test_bf16_all_experts_on_mfma(B, split_k):
    w = W.scaled(SMALL_BF16, B=B)
    L = layer(w, 21)
    x = W.make_x(w, 21, device="cuda")
    ctx = make_context(w)
    ctx.set_path(M.PATH_MFMA, split_k=split_k)
    full_check(ctx, w, L, x)
    plan = ctx.last_plan()
    assert plan["gemv"] == 0 and plan["mfma"] == plan["distinct"], plan


@pytest.mark.parametrize("B", [1, 5, 16])
@pytest.mark.parametrize("split_k", [1, 4])
def test_fp8_all_experts_on_mfma(B, split_k):
    w = W.scaled(SMALL_FP8, B=B)
    L = layer(w, 22)
    x = W.make_x(w, 22, device="cuda")
    ctx = make_context(w)
    ctx.set_path(M.PATH_MFMA, split_k=split_k)
    full_check(ctx, w, L, x)
    plan = ctx.last_plan()
    assert plan["gemv"] == 0


@pytest.mark.parametrize("B", [1, 2, 3])
def test_auto_runs_gemv_at_one_row_and_mfma_from_two(B):
    w = W.scaled(SMALL_BF16, B=B)
    L = layer(w, 24)
    x = W.make_x(w, 24, device="cuda")
    ctx = make_context(w)
    full_check(ctx, w, L, x)
    plan = ctx.last_plan()
    kind = "gemv" if B == 1 else "mfma"
    assert plan[kind] == plan["distinct"], plan


@pytest.mark.parametrize("min_rows", [1, 2, 3, 5, 8, 64])
def test_auto_threshold_splits_experts_between_kernels(min_rows):
    # AUTO: an expert goes to the MFMA kernels from min_rows rows, and from
    # five rows whatever min_rows (the GEMV kernels stage four rows of x per
    # pass and would stream an expert's weights once per pass)
    w = W.scaled(SMALL_BF16, B=24)
    L = layer(w, 23)
    x = W.make_x(w, 23, device="cuda")
    ctx = make_context(w)
    ctx.set_path(M.PATH_AUTO, mfma_min_rows=min_rows)
    _, idx, _ = full_check(ctx, w, L, x)
    plan = ctx.last_plan()
    counts = np.bincount(idx.ravel(), minlength=w.E)
    assert counts.max() > 4  # the cap matters for this batch
    to_mfma = (counts >= min_rows) | (counts > 4)
    assert plan["mfma"] == int(to_mfma.sum()), (plan, min_rows)
    assert plan["gemv"] == int(((counts > 0) & ~to_mfma).sum())


def test_auto_never_gives_gemv_an_expert_beyond_one_pass():
    # correlated verify rows share experts (up to 8 rows each): with the MFMA
    # threshold above the batch, only experts of at most four rows stay on GEMV
    w = W.scaled(W.WORKLOADS["verify_b8"], H=1024, E=64, k=8, I=512)
    L = layer(w, 29)
    x = W.make_x(w, 29, device="cuda")
    ctx = make_context(w)
    ctx.set_path(M.PATH_AUTO, mfma_min_rows=64)
    _, idx, _ = full_check(ctx, w, L, x)
    plan = ctx.last_plan()
    counts = np.bincount(idx.ravel(), minlength=w.E)
    assert counts.max() > 4
    assert plan["mfma"] == int((counts > 4).sum()) > 0, plan
    assert plan["gemv"] == int(((counts > 0) & (counts <= 4)).sum()), plan


def test_gemv_and_mfma_paths_agree():
    w = W.scaled(SMALL_BF16, B=12)
    L = layer(w, 24)
    x = W.make_x(w, 24, device="cuda")
    ctx = make_context(w)
    ctx.set_path(M.PATH_GEMV)
    idx_g, w_g, out_g = gpu_forward(ctx, w, L, x)
    ctx.set_path(M.PATH_MFMA)
    idx_m, w_m, out_m = gpu_forward(ctx, w, L, x)
    assert np.array_equal(idx_g, idx_m) and np.array_equal(w_g, w_m)
    # both within the oracle tolerance, and close to each other (fp32 sums in
    # different orders, h rounded to bf16 on both sides)
    check_layer(w, L, x, idx_g, w_g, out_g)
    check_layer(w, L, x, idx_m, w_m, out_m)
    d = (out_g.float() - out_m.float()).abs().max().item()
    assert d <= 2e-2, d


def test_many_rows_on_one_expert():
    # every row of the batch is the same token: each of its k experts gets all
    # 40 rows, i.e. three 16-row M tiles (16 + 16 + 8)
    w = W.scaled(SMALL_BF16, B=40)
    L = layer(w, 25)
    x1 = W.make_x(w, 25, device="cuda", B=1)
    x = x1.expand(w.B, w.H).contiguous()
    ctx = make_context(w)
    for split_k in (1, 2):
        ctx.set_path(M.PATH_MFMA, split_k=split_k)
        _, idx, out = full_check(ctx, w, L, x, rows=[0, 17, 39])
        plan = ctx.last_plan()
        assert plan["distinct"] == w.k and plan["max_rows"] == w.B, plan
        # identical rows give identical outputs
        assert torch.equal(out[0], out[39]) and torch.equal(out[0], out[17])


def test_fp8_many_rows_on_one_expert():
    w = W.scaled(SMALL_FP8, B=20)
    L = layer(w, 26)
    x = W.make_x(w, 26, device="cuda", B=1).expand(w.B, w.H).contiguous()
    ctx = make_context(w)
    ctx.set_path(M.PATH_AUTO, mfma_min_rows=2)
    full_check(ctx, w, L, x, rows=[0, 19])
    assert ctx.last_plan()["mfma"] == w.k


def test_split_k_results_are_deterministic():
    w = W.scaled(SMALL_BF16, B=33)
    L = layer(w, 27)
    x = W.make_x(w, 27, device="cuda")
    ctx = make_context(w)
    ctx.set_path(M.PATH_MFMA, split_k=5)
    a = gpu_forward(ctx, w, L, x)
    b = gpu_forward(ctx, w, L, x)
    assert torch.equal(a[2], b[2])


def test_all_logits_tied_take_the_lowest_indices():
    # a zero router ties every logit at 0: the selection must be experts
    # 0..k-1 in order with equal weights (more than 64 tied candidates)
    w = W.scaled(SMALL_BF16, B=3)
    L = layer(w, 28)
    L["router_w"].zero_()
    x = W.make_x(w, 28, device="cuda")
    ctx = make_context(w)
    idx, wt, out = gpu_forward(ctx, w, L, x)
    assert np.array_equal(idx, np.tile(np.arange(w.k, dtype=np.int32), (w.B, 1)))
    assert np.all(wt == np.float32(1.0 / w.k))
    stats = check_layer(w, L, x, idx, wt, out)
    assert stats["excused_rows"] == []


def test_wide_router_2048_experts_top32():
    w = W.scaled(SMALL_BF16, B=5, E=2048, k=32, H=512, I=512)
    L = layer(w, 29)
    x = W.make_x(w, 29, device="cuda")
    ctx = make_context(w)
    full_check(ctx, w, L, x)


def test_ramp_router_many_near_ties():
    # logits e * 2^-20 apart: every gap is exact in fp64 and far below 1e-6,
    # so the GPU must order them exactly (largest indices first)
    w = W.scaled(SMALL_BF16, B=2)
    L = layer(w, 30)
    x = torch.zeros((w.B, w.H), dtype=torch.bfloat16, device="cuda")
    x[:, 0] = 1.0
    r = torch.zeros((w.E, w.H), dtype=torch.float32, device="cuda")
    r[:, 0] = torch.arange(w.E, dtype=torch.float32, device="cuda") * 2.0 ** -20
    L["router_w"] = r
    ctx = make_context(w)
    idx, _, _ = gpu_forward(ctx, w, L, x)
    want = np.arange(w.E - 1, w.E - 1 - w.k, -1, dtype=np.int32)
    assert np.array_equal(idx, np.tile(want, (w.B, 1)))


def test_prefetch_leaves_results_unchanged_and_checks_arguments():
    w = W.scaled(SMALL_BF16, B=8)
    L = layer(w, 31)
    nxt = layer(w, 32, layer_id=1)
    x = W.make_x(w, 31, device="cuda")
    ctx = make_context(w)
    ref = gpu_forward(ctx, w, L, x)
    ctx.set_prefetch([nxt["router_w"], nxt["w_gate_up"][:3], nxt["w_down"][:3]])
    for _ in range(3):
        got = gpu_forward(ctx, w, L, x)
        assert np.array_equal(got[0], ref[0]) and torch.equal(got[2], ref[2])
    with pytest.raises(M.MoeError) as ei:
        ctx.set_prefetch([nxt["router_w"]] * 9)
    assert ei.value.status == M.binding.ERR_INVALID_ARG
    flat = nxt["router_w"].view(-1)
    with pytest.raises(M.MoeError) as ei:
        ctx.set_prefetch([flat[1:]])        # not 16-byte aligned
    assert ei.value.status == M.binding.ERR_INVALID_ARG
    ctx.set_prefetch([])                     # off again
    got = gpu_forward(ctx, w, L, x)
    assert torch.equal(got[2], ref[2])


@pytest.mark.parametrize("B", [1, 8])
def test_prefetch_with_the_forward_leaves_results_unchanged(B):
    # the warm-up started with the forward's first launch, on a wide grid,
    # over the experts this forward then reads
    w = W.scaled(SMALL_BF16, B=B)
    L = layer(w, 34)
    x = W.make_x(w, 34, device="cuda")
    ctx = make_context(w)
    ref = gpu_forward(ctx, w, L, x)
    hot = [int(e) for e in ref[0][0][:3]]
    ctx.set_prefetch_mode(1, 1024)
    ctx.set_prefetch([L["w_gate_up"][e] for e in hot] + [L["router_w"]])
    for _ in range(3):
        got = gpu_forward(ctx, w, L, x)
        assert np.array_equal(got[0], ref[0]) and torch.equal(got[2], ref[2])
    assert ctx.last_plan()["launches"] == (5 if B == 1 else 6)  # the warm-up counted
    for bad in ((2, 0), (-1, 0), (0, -1), (0, 65537)):
        with pytest.raises(M.MoeError) as ei:
            ctx.set_prefetch_mode(*bad)
        assert ei.value.status == M.binding.ERR_INVALID_ARG


@pytest.mark.parametrize("path", [M.PATH_AUTO, M.PATH_GEMV])
def test_all_2048_slots_bucketed(path):
    # 64 rows x top-32 of 2048 experts: every slot the plan can hold, grouped
    # by the counting sort; the plan's counters must match the selection
    w = W.scaled(SMALL_BF16, B=64, E=2048, k=32, H=512, I=512)
    L = layer(w, 33)
    x = W.make_x(w, 33, device="cuda")
    ctx = make_context(w)
    ctx.set_path(path)
    _, idx, _ = full_check(ctx, w, L, x, rows=[0, 31, 63])
    plan = ctx.last_plan()
    counts = np.bincount(idx.ravel(), minlength=w.E)
    assert plan["distinct"] == int((counts > 0).sum()), plan
    assert plan["max_rows"] == int(counts.max()), plan
