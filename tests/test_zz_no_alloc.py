"""The entry point that allocates nothing (moe_decode_forward_noalloc): its
workspace is the library's fixed scratch array.  Through the C ABI, two calls
in a row, the second with a smaller batch, each checked against the context
entry point (moe_decode_forward_ctx, the same kernels: bit for bit) and
against the oracle."""
import gc

import numpy as np
import pytest
import torch

import mixture_experts_layer_decode_amd as M
import workloads as W
from parity_helpers import MOE_SCORE, check_layer, gpu_forward, make_context

pytestmark = pytest.mark.gpu

SMALL_BF16 = W.scaled(W.WORKLOADS["full_b64"], H=1024, E=64, k=8, I=512)
SMALL_FP8 = W.scaled(W.WORKLOADS["stack4_fp8_b16"], H=1024, E=64, k=8, I=1024, layers=1)
TINY = W.WORKLOADS["tiny_b1"]


def layer(w, seed):
    return {k: (v.cuda() if v is not None else None) for k, v in W.make_layer(w, seed).items()}


def noalloc_forward(w, L, x):
    B = x.shape[0]
    idx = torch.full((B, w.k), -1, dtype=torch.int32, device="cuda")
    wt = torch.zeros((B, w.k), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    M.forward_noalloc(x, L["router_w"], L["w_gate_up"], L["w_down"], w.k, MOE_SCORE[w.score],
                      bias=L["bias"], s_gu=L["s_gu"], s_d=L["s_d"], out=out, idx_out=idx,
                      weight_out=wt)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), wt.cpu().numpy(), out


def same_as_context(w, L, x, oracle_rows=None):
    ctx = make_context(w, max_batch=x.shape[0])
    want = gpu_forward(ctx, w, L, x)
    ctx.close()
    got = noalloc_forward(w, L, x)
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1], want[1])
    assert torch.equal(got[2], want[2])
    stats = check_layer(w, L, x, got[0], got[1], got[2], rows=oracle_rows)
    print(f"[noalloc] {w.name} B={x.shape[0]}: {stats}", flush=True)


@pytest.mark.parametrize("recipe,batches,seed", [
    (SMALL_BF16, (16, 3), 61),   # MFMA path, then fewer rows
    (SMALL_FP8, (8, 2), 62),
    (TINY, (2, 1), 63),          # fp32, then batch 1 with the combine folded in
    (SMALL_BF16, (5, 1), 64),    # MFMA path, then the GEMV path at batch 1
])
def test_noalloc_matches_the_context_entry_point(recipe, batches, seed):
    L = layer(recipe, seed)
    for step, B in enumerate(batches):
        w = W.scaled(recipe, B=B)
        x = W.make_x(w, seed, step=step, device="cuda")
        same_as_context(w, L, x)


def test_noalloc_full_layer_largest_batch_then_batch_one():
    # the full layer at 64 rows fills most of the scratch array; the batch-1
    # call after it runs on what the first one left there
    w64 = W.WORKLOADS["full_b64"]
    L = W.make_layer(w64, 0, device="cuda")
    same_as_context(w64, L, W.make_x(w64, 0, device="cuda"), oracle_rows=[0, 31, 63])
    w1 = W.WORKLOADS["full_b1"]
    same_as_context(w1, L, W.make_x(w1, 0, step=1, device="cuda"))
    L.clear()
    gc.collect()
    torch.cuda.empty_cache()


def test_noalloc_refuses_a_batch_beyond_the_array():
    # H 8192, I 8192, top-32 of 64 experts at 64 rows: 64 MiB of y alone.  The
    # refusal comes before any device work: the (uninitialised) tensors are
    # never read, and out keeps its contents
    E, H, I, k, B = 64, 8192, 8192, 32, 64
    x = torch.zeros((B, H), dtype=torch.bfloat16, device="cuda")
    r = torch.zeros((E, H), dtype=torch.float32, device="cuda")
    gu = torch.empty((E, 2 * I, H), dtype=torch.bfloat16, device="cuda")
    dn = torch.empty((E, H, I), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(x, 3.0)
    with pytest.raises(M.MoeError) as err:
        M.forward_noalloc(x, r, gu, dn, k, M.SIGMOID, out=out)
    assert err.value.status == M.binding.ERR_UNSUPPORTED and "scratch array" in str(err.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    del gu, dn
    torch.cuda.empty_cache()
