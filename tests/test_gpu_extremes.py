"""GPU parity at the extremes of the supported shapes: hidden and intermediate
widths at their largest (8192) and smallest for every weight type, on the
GEMV and the MFMA kernels, against the CPU oracle.  Large rows
change the kernel variants used (the widest router split, 16-vector weight
rows, the separate combine instead of the folded one)."""
import pytest

import mixture_experts_layer_decode_amd as M
import workloads as W
from parity_helpers import full_check, make_context

pytestmark = pytest.mark.gpu

BASE = {
    "bf16": W.WORKLOADS["full_b64"],
    "fp8": W.scaled(W.WORKLOADS["stack4_fp8_b16"], layers=1),
    "f32": W.scaled(W.WORKLOADS["full_b64"], act="f32", wdt="f32"),
}


def layer_on_gpu(w, seed):
    return W.make_layer(w, seed, device="cuda")


@pytest.mark.parametrize("wdt", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("B,path", [(1, M.PATH_AUTO), (5, M.PATH_AUTO), (20, M.PATH_GEMV)])
def test_largest_hidden_and_intermediate(wdt, B, path):
    # weights N(0, 0.01): with 4x the full layer's widths this keeps the
    # output at the full layer's magnitude (|out| < 8), where the 2e-2 bound
    # holds for an output rounded once to bf16 (its spacing is 0.0625 from 8)
    w = W.scaled(BASE[wdt], B=B, H=8192, I=8192, E=8, k=2, w_std=0.01)
    L = layer_on_gpu(w, 71)
    x = W.make_x(w, 71, device="cuda")
    ctx = make_context(w)
    ctx.set_path(path)
    full_check(ctx, w, L, x, rows=sorted({0, B - 1}))


# the narrowest widths each weight type supports: rows of one 16-byte vector
# per lane (bf16 512, fp8 1024, fp32 256 elements) and a hidden width of at
# least one 512-column router chunk
SMALLEST = {"bf16": (512, 512), "fp8": (1024, 1024), "f32": (512, 256)}


@pytest.mark.parametrize("wdt", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("B", [1, 64])
def test_smallest_hidden_and_intermediate(wdt, B):
    H, I = SMALLEST[wdt]
    w = W.scaled(BASE[wdt], B=B, H=H, I=I, E=32, k=8)
    L = layer_on_gpu(w, 72)
    x = W.make_x(w, 72, device="cuda")
    ctx = make_context(w)
    full_check(ctx, w, L, x, rows=sorted({0, B // 2, B - 1}))
