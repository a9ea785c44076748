"""The seeded input recipes (CPU only): shapes, storage types and the row
structure of the verify workloads."""
import numpy as np
import torch

import workloads as W


def _corr(x):
    return np.corrcoef(x.float().numpy())


def test_verify_rows_share_one_base_per_sequence():
    x = W.make_x(W.WORKLOADS["verify_8x8"], 0)
    assert x.shape == (64, 7168) and x.dtype == torch.bfloat16
    c = _corr(x)
    seq = np.arange(64) // 8
    same = c[seq[:, None] == seq[None, :]]
    other = c[seq[:, None] != seq[None, :]]
    # base N(0,1) + 0.3 N(0,1): correlation 1 / 1.09 within a sequence, 0 across
    assert same.min() > 0.85
    assert np.abs(other).max() < 0.1


def test_single_sequence_verify_shapes():
    for d in range(3, 8):
        w = W.WORKLOADS[f"verify_d{d}"]
        x = W.make_x(w, 0)
        assert x.shape == (1 + d, 7168)
        assert _corr(x).min() > 0.85
    # seven drafts is the 8-row verify shape
    assert torch.equal(W.make_x(W.WORKLOADS["verify_d7"], 0), W.make_x(W.WORKLOADS["verify_b8"], 0))


def test_independent_rows_are_uncorrelated_and_standard_normal():
    x = W.make_x(W.WORKLOADS["full_b64"], 0).float().numpy()
    c = _corr(torch.from_numpy(x))
    off = c[~np.eye(64, dtype=bool)]
    assert np.abs(off).max() < 0.1
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01


def test_steps_and_seeds_give_new_inputs():
    w = W.WORKLOADS["full_b1"]
    a, b, c = W.make_x(w, 0, step=0), W.make_x(w, 0, step=1), W.make_x(w, 1, step=0)
    assert not torch.equal(a, b) and not torch.equal(a, c)
    assert torch.equal(a, W.make_x(w, 0, step=0))


def test_small_layer_weights_follow_the_recipe():
    w = W.scaled(W.WORKLOADS["stack4_fp8_b16"], H=1024, E=8, I=1024, layers=1)
    L = W.make_layer(w, 0)
    assert L["w_gate_up"].dtype == torch.uint8 and L["w_gate_up"].shape == (8, 2048, 1024)
    # per-row scale = max |w| / 448, so every row reaches the largest e4m3 code
    codes = L["w_gate_up"].view(torch.float8_e4m3fn).float().abs()
    assert torch.all(codes.amax(dim=-1) == 448.0)
    # Zipf bias: -1.1 ln(1 + rank), one rank per expert
    ranks = torch.exp(-L["bias"].double() / 1.1) - 1.0
    assert torch.allclose(torch.sort(ranks).values, torch.arange(8, dtype=torch.float64), atol=1e-4)
    w16 = W.scaled(W.WORKLOADS["full_b1"], H=512, E=4, I=512)
    L16 = W.make_layer(w16, 0)
    assert abs(float(L16["w_gate_up"].float().std()) - 0.02) < 0.001
    assert abs(float(L16["router_w"].std()) - 0.02) < 0.001
