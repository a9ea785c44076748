"""Pins of the CPU oracle against things other than itself (CPU only).

Each test pins one step of the layer with an independent source: a library
routine (torch's bf16 / OCP-e4m3 conversions, numpy matmul, scipy's
expit/softmax, itertools enumeration), exact integer arithmetic, a hand-worked
example (tests/golden/), or a structural invariant of the method.  They are
chosen so that a dropped term, a swapped gate/up, a transposed weight, a wrong
scale index or a wrong tie-break fails at least one of them.
"""
import itertools
import os

import numpy as np
import pytest
import scipy.special as sp
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(a):
    """float32 array -> bf16 storage bits via torch (RNE from float32)."""
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def bf16_to_f64(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def e4m3_to_f64(codes):
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ------------------------------------------------------------ input decode

def test_e4m3_all_codes_match_library():
    codes = np.arange(256, dtype=np.uint8)
    ref = e4m3_to_f64(codes)
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # S.1111.111 only (OCP e4m3 has no infinities)
    assert np.array_equal(got[~nan], ref[~nan])
    # format constants: largest finite, smallest normal / subnormal, one
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0xB8) == -1.0


def test_bf16_decode_all_patterns_match_library():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bf16_to_f64(bits)
    finite = np.isfinite(ref)
    got = np.array([oracle.bf16_value(int(b)) for b in bits[finite][::7]])
    assert np.array_equal(got, ref[finite][::7])


def test_bf16_rounding_ties_and_single_step():
    one = 0x3F80
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == one            # tie -> even (down)
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == one + 2    # tie -> even (up)
    assert oracle.round_bf16(-(1.0 + 2.0 ** -8)) == 0x8000 | one
    # above the tie by less than float32's resolution: one rounding step goes up,
    # rounding through float32 first would land on the tie and go down
    assert oracle.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == one + 1
    assert oracle.round_bf16(0.0) == 0


def test_bf16_rounding_matches_library_on_float32_values():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(20000) * rng.choice([1e-3, 1.0, 30.0], 20000)).astype(np.float32)
    ref = bf16_bits(v)
    got = np.array([oracle.round_bf16(float(t)) for t in v], np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ router

def test_router_one_hot_x_reads_a_column_plus_bias():
    rng = np.random.default_rng(1)
    E, H = 24, 64
    wr = rng.standard_normal((E, H)).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    x = np.zeros((3, H), np.float32)
    cols = [0, 17, 63]
    for r, c in enumerate(cols):
        x[r, c] = 1.0
    lg = oracle.router_logits(x, oracle.F32, wr, bias)
    for r, c in enumerate(cols):
        assert np.array_equal(lg[r], wr[:, c].astype(np.float64) + bias.astype(np.float64))


def test_router_dyadic_integers_exact():
    rng = np.random.default_rng(2)
    B, E, H = 4, 32, 512
    xi = rng.integers(-8, 9, (B, H))
    wi = rng.integers(-64, 65, (E, H))
    x = bf16_bits(xi.astype(np.float32))          # small integers: exact in bf16
    wr = (wi / 4.0).astype(np.float32)             # quarters: exact in fp32
    ref = (xi @ wi.T) / 4.0                        # exact integer arithmetic
    lg = oracle.router_logits(x, oracle.BF16, wr)
    assert np.array_equal(lg, ref)


# ------------------------------------------------------------------- top-k

def _order_key(s, e):
    return (-s, e)


def _brute_force_topk(s, k):
    """The unique k-set whose members all rank before every non-member."""
    E = len(s)
    winners = []
    for comb in itertools.combinations(range(E), k):
        inside = set(comb)
        if all(_order_key(s[a], a) < _order_key(s[b], b)
               for a in inside for b in range(E) if b not in inside):
            winners.append(inside)
    assert len(winners) == 1
    return winners[0]


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    for E, k in [(8, 1), (10, 3), (12, 4), (16, 4)]:
        # values from a small set so that ties are frequent
        s = rng.choice(np.array([-1.0, -0.25, 0.0, 0.5, 0.5, 2.0]), size=(5, E))
        idx, w = oracle.topk(s, k, oracle.SIGMOID)
        for b in range(5):
            assert set(idx[b].tolist()) == _brute_force_topk(s[b], k)
            want_order = sorted(idx[b].tolist(), key=lambda e: _order_key(s[b][e], e))
            assert idx[b].tolist() == want_order


def test_topk_duplicate_rows_lower_index_wins():
    rng = np.random.default_rng(3)
    E, H = 16, 64
    wr = rng.standard_normal((E, H)).astype(np.float32)
    wr[9] = wr[2]     # experts 2 and 9 always tie
    wr[12] = wr[5]
    x = rng.standard_normal((1, H)).astype(np.float32)
    lg = oracle.router_logits(x, oracle.F32, wr)
    assert lg[0, 2] == lg[0, 9] and lg[0, 5] == lg[0, 12]
    order = np.argsort(-lg[0], kind="stable")     # library stable sort: lower index first
    for k in range(1, E + 1):
        idx, _ = oracle.topk(lg, k, oracle.SIGMOID)
        assert idx[0].tolist() == order[:k].tolist()


def test_topk_ramp_picks_largest_indices():
    E, k = 896, 16
    s = (np.arange(E) * 1e-3)[None, :]
    idx, _ = oracle.topk(s, k, oracle.SIGMOID)
    assert idx[0].tolist() == list(range(E - 1, E - 1 - k, -1))


# ----------------------------------------------------------------- weights

def test_sigmoid_weights_closed_form_two_experts():
    a, b = 1.3, -0.4
    s = np.array([[b, a, -5.0]])
    idx, w = oracle.topk(s, 2, oracle.SIGMOID)
    assert idx[0].tolist() == [1, 0]
    pa, pb = sp.expit(a), sp.expit(b)
    np.testing.assert_allclose(w[0], [pa / (pa + pb), pb / (pa + pb)], rtol=1e-14)


def test_softmax_weights_equal_full_softmax_then_renorm():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((6, 64)) * 2
    idx, w = oracle.topk(s, 4, oracle.SOFTMAX)
    full = sp.softmax(s, axis=1)
    for b in range(6):
        sel = full[b, idx[b]]
        np.testing.assert_allclose(w[b], sel / sel.sum(), rtol=1e-13)


def test_softmax_weights_stay_finite_for_large_logits():
    # exp(800) overflows a double: the weights must come from shifted logits
    # and exp(-800) underflows to zero: both signs need the shift
    for sign in (1.0, -1.0):
        s = sign * 800.0 + np.array([[0.0, -1.0, -10.0, -803.0, -1.5]])
        idx, w = oracle.topk(s, 3, oracle.SOFTMAX)
        assert idx[0].tolist() == [0, 1, 4]
        sel = sp.softmax(s[0])[[0, 1, 4]]
        np.testing.assert_allclose(w[0], sel / sel.sum(), rtol=1e-13)


def test_weights_sum_to_one_positive_and_equal_on_ties():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((8, 896)) * 1.7
    for fn in (oracle.SIGMOID, oracle.SOFTMAX):
        idx, w = oracle.topk(s, 16, fn)
        assert np.all(w > 0)
        assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 1e-12
        assert all(len(set(r.tolist())) == 16 for r in idx)
    flat = np.full((1, 32), 0.7)
    _, w = oracle.topk(flat, 8, oracle.SIGMOID)
    # p / (p + ... + p): the sequential sum of eight equal terms rounds, so 1/k
    # holds to a couple of ulps
    assert np.max(np.abs(w - 0.125)) <= 4 * np.finfo(np.float64).eps * 0.125


def test_selection_weights_of_any_selection_match_closed_forms():
    # the weights of a selection that is not the top-k, listed in an
    # arbitrary order: sigmoid renormalised over exactly those experts, and
    # the full softmax restricted to them and renormalised
    rng = np.random.default_rng(6)
    s = rng.standard_normal((5, 96)) * 1.7
    sel = np.stack([rng.permutation(96)[:7] for _ in range(5)]).astype(np.int32)
    w = oracle.selection_weights(s, sel, oracle.SIGMOID)
    p = sp.expit(np.take_along_axis(s, sel, axis=1))
    np.testing.assert_allclose(w, p / p.sum(axis=1, keepdims=True), rtol=1e-14)
    w = oracle.selection_weights(s, sel, oracle.SOFTMAX)
    full = np.take_along_axis(sp.softmax(s, axis=1), sel, axis=1)
    np.testing.assert_allclose(w, full / full.sum(axis=1, keepdims=True), rtol=1e-13)


def test_selection_weights_follow_the_selection_order():
    # swapping two chosen experts swaps their weights and nothing else
    s = np.array([[0.3, -1.2, 2.5, 0.9, -0.1]])
    a = oracle.selection_weights(s, np.array([[2, 3, 0]], np.int32), oracle.SIGMOID)
    b = oracle.selection_weights(s, np.array([[3, 2, 0]], np.int32), oracle.SIGMOID)
    np.testing.assert_allclose(b[0], a[0][[1, 0, 2]], rtol=1e-15)


# ------------------------------------------------------------- expert FFN

def _read_golden():
    rows = {}
    with open(os.path.join(GOLDEN, "swiglu_hand_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            act, h, o0, o1 = line.split()
            rows[act] = (float(h), float(o0), float(o1))
    return rows


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_hand_example_single_expert(act):
    h_want, o0, o1 = _read_golden()[act]
    x = np.array([[1.0, 0.5]], np.float32)
    gu = np.array([[[30.0, 0.0], [1.015625, 0.0]]], np.float32)
    dn = np.array([[[1.0], [-2.0]]], np.float32)
    wr = np.zeros((1, 2), np.float32)
    if act == "bf16":
        xa, ad = bf16_bits(x), oracle.BF16
        gw, dw, wd_ = bf16_bits(gu), bf16_bits(dn), oracle.BF16
    else:
        xa, ad, gw, dw, wd_ = x, oracle.F32, gu, dn, oracle.F32
    idx, w, out = oracle.moe_forward(xa, ad, wr, None, 1, oracle.SIGMOID, gw, dw, wd_)
    assert idx.tolist() == [[0]] and w.tolist() == [[1.0]]
    h, _ = oracle.expert_ffn(xa[0], ad, gw[0], dw[0], wd_)
    assert h.tolist() == [h_want]
    np.testing.assert_allclose(out[0], [o0, o1], rtol=0, atol=1e-9)


def _dense_swiglu(x, wg, wu, wd, round_h):
    g = wg @ x
    u = wu @ x
    a = g * sp.expit(g) * u
    return wd @ round_h(a)


def test_single_expert_equals_dense_swiglu_f32():
    rng = np.random.default_rng(6)
    H, I = 96, 40
    x = rng.standard_normal((1, H)).astype(np.float32)
    gu = (rng.standard_normal((1, 2 * I, H)) * 0.2).astype(np.float32)
    dn = (rng.standard_normal((1, H, I)) * 0.2).astype(np.float32)
    wr = rng.standard_normal((1, H)).astype(np.float32)
    idx, w, out = oracle.moe_forward(x, oracle.F32, wr, None, 1, oracle.SIGMOID, gu, dn,
                                     oracle.F32)
    assert w[0, 0] == 1.0
    ref = _dense_swiglu(x[0].astype(np.float64), gu[0, :I].astype(np.float64),
                        gu[0, I:].astype(np.float64), dn[0].astype(np.float64),
                        lambda a: a.astype(np.float32).astype(np.float64))
    np.testing.assert_allclose(out[0] - x[0], ref, rtol=1e-12, atol=1e-12)


def test_forward_equals_its_steps_recomposed_in_numpy():
    # k = 3 of E = 8 with distinct weights: the whole layer recomputed from
    # numpy pieces (logits by matmul, order by argsort, sigmoid by scipy, each
    # selected expert as a dense SwiGLU), so that pairing a routing weight
    # with another choice's expert output, or a wrong slot order, fails
    rng = np.random.default_rng(12)
    B, H, I, E, k = 3, 64, 24, 8, 3
    x = rng.standard_normal((B, H)).astype(np.float32)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    gu = (rng.standard_normal((E, 2 * I, H)) * 0.2).astype(np.float32)
    dn = (rng.standard_normal((E, H, I)) * 0.2).astype(np.float32)
    idx, w, out = oracle.moe_forward(x, oracle.F32, wr, None, k, oracle.SIGMOID, gu, dn,
                                     oracle.F32)
    lg = x.astype(np.float64) @ wr.astype(np.float64).T
    for b in range(B):
        order = np.argsort(-lg[b], kind="stable")[:k]
        assert np.array_equal(idx[b], order)
        p = sp.expit(lg[b, order])
        np.testing.assert_allclose(w[b], p / p.sum(), rtol=1e-12)
        assert len(set(np.round(w[b], 6).tolist())) == k  # distinct weights
        ref = x[b].astype(np.float64).copy()
        for j in range(k):
            e = order[j]
            ref += (p[j] / p.sum()) * _dense_swiglu(
                x[b].astype(np.float64), gu[e, :I].astype(np.float64),
                gu[e, I:].astype(np.float64), dn[e].astype(np.float64),
                lambda a: a.astype(np.float32).astype(np.float64))
        np.testing.assert_allclose(out[b], ref, rtol=1e-11, atol=1e-11)


def test_single_expert_equals_dense_swiglu_bf16():
    rng = np.random.default_rng(7)
    H, I = 128, 64
    x = bf16_bits(rng.standard_normal((1, H)))
    gu = bf16_bits(rng.standard_normal((1, 2 * I, H)) * 0.1)
    dn = bf16_bits(rng.standard_normal((1, H, I)) * 0.1)
    wr = rng.standard_normal((1, H)).astype(np.float32)
    h, y = oracle.expert_ffn(x[0], oracle.BF16, gu[0], dn[0], oracle.BF16)
    xf, g64, d64 = bf16_to_f64(x[0]), bf16_to_f64(gu[0]), bf16_to_f64(dn[0])
    g = g64[:I] @ xf
    u = g64[I:] @ xf
    a = g * sp.expit(g) * u
    # h is a rounded to bf16: within half a bf16 spacing, and representable
    spacing = 2.0 ** (np.floor(np.log2(np.abs(a))) - 7)
    assert np.all(np.abs(h - a) <= spacing / 2 * (1 + 1e-9))
    assert np.array_equal(bf16_to_f64(bf16_bits(h.astype(np.float32))), h)
    np.testing.assert_allclose(y, d64 @ h, rtol=1e-12, atol=1e-12)


def test_fp8_scales_index_rows_of_gate_up_and_down():
    rng = np.random.default_rng(8)
    H, I = 64, 32
    x = bf16_bits(rng.standard_normal(H))
    gu_c = rng.integers(0, 256, (2 * I, H), dtype=np.uint8)
    dn_c = rng.integers(0, 256, (H, I), dtype=np.uint8)
    gu_c[(gu_c & 0x7F) == 0x7F] = 0x3F   # no NaN codes
    dn_c[(dn_c & 0x7F) == 0x7F] = 0x3F
    s_gu = rng.uniform(0.5, 2.0, 2 * I).astype(np.float32) * 1e-3
    s_d = rng.uniform(0.5, 2.0, H).astype(np.float32) * 1e-2
    h, y = oracle.expert_ffn(x, oracle.BF16, gu_c, dn_c, oracle.E4M3, s_gu, s_d)
    deq_gu = e4m3_to_f64(gu_c) * s_gu.astype(np.float64)[:, None]
    deq_dn = e4m3_to_f64(dn_c) * s_d.astype(np.float64)[:, None]
    xf = bf16_to_f64(x)
    g = deq_gu[:I] @ xf
    u = deq_gu[I:] @ xf
    a = g * sp.expit(g) * u
    spacing = 2.0 ** (np.floor(np.log2(np.abs(a))) - 7)
    assert np.all(np.abs(h - a) <= spacing / 2 * (1 + 1e-9))
    np.testing.assert_allclose(y, deq_dn @ h, rtol=1e-12, atol=1e-15)


def test_silu_identities_through_the_ffn():
    # gate rows give g = z and g = -z with u = 1: h0 - h1 = silu(z) - silu(-z) = z
    H, I = 2, 3
    z = 0.8125
    x = np.array([1.0, 0.0], np.float32)
    gu = np.array([[z, 0], [-z, 0], [0, 0], [1, 0], [1, 0], [1, 0]], np.float32)
    dn = np.zeros((H, I), np.float32)
    h, y = oracle.expert_ffn(x, oracle.F32, gu, dn, oracle.F32)
    assert abs((h[0] - h[1]) - z) < 1e-7
    assert h[2] == 0.0    # silu(0) = 0
    assert np.all(y == 0.0)


# ---------------------------------------------------------------- combine

def _small_layer(seed, B=3, H=64, E=12, k=4, I=32, act="f32", wdt="f32"):
    w = W.Workload("t", B=B, H=H, E=E, k=k, I=I, act=act, wdt=wdt, score="sigmoid",
                   w_std=0.2)
    L = W.make_layer(w, seed)
    x = W.make_x(w, seed)
    ad = oracle.F32 if act == "f32" else oracle.BF16
    wd_ = {"f32": oracle.F32, "bf16": oracle.BF16, "fp8": oracle.E4M3}[wdt]
    return (W.raw_numpy(x), ad, W.raw_numpy(L["router_w"]), W.raw_numpy(L["w_gate_up"]),
            W.raw_numpy(L["w_down"]), wd_, W.raw_numpy(L["s_gu"]), W.raw_numpy(L["s_d"]))


def test_zero_experts_leave_x_unchanged():
    x, ad, wr, gu, dn, wd_, _, _ = _small_layer(0)
    idx, w, out = oracle.moe_forward(x, ad, wr, None, 4, oracle.SIGMOID, np.zeros_like(gu),
                                     dn, wd_)
    assert np.array_equal(out, x.astype(np.float64))


def test_down_scale_by_power_of_two_scales_delta_exactly():
    # 4 * Wd scales every product, hence every sum, by 4 without rounding; the
    # weighted combine with a zero residual scales the same way
    x, ad, wr, gu, dn, wd_, _, _ = _small_layer(1)
    _, y1 = oracle.expert_ffn(x[0], ad, gu[3], dn[3], wd_)
    _, y4 = oracle.expert_ffn(x[0], ad, gu[3], dn[3] * 4.0, wd_)
    assert np.any(y1 != 0) and np.array_equal(y4, 4.0 * y1)
    w = np.array([[0.25, 0.75]])
    zero = np.zeros((1, y1.size), np.float32)
    c1 = oracle.combine(zero, oracle.F32, w, np.stack([y1, -y1])[None])
    c4 = oracle.combine(zero, oracle.F32, w, np.stack([y4, -y4])[None])
    assert np.array_equal(c4, 4.0 * c1)


def test_combine_is_weighted_sum_plus_residual():
    rng = np.random.default_rng(9)
    B, k, H = 2, 3, 5
    x = rng.standard_normal((B, H)).astype(np.float32)
    w = rng.uniform(size=(B, k))
    y = rng.standard_normal((B, k, H))
    out = oracle.combine(x, oracle.F32, w, y)
    np.testing.assert_allclose(out, x + np.einsum("bk,bkh->bh", w, y), rtol=1e-14)


# -------------------------------------------------------------- structure

def test_expert_permutation_equivariance():
    x, ad, wr, gu, dn, wd_, _, _ = _small_layer(2)
    idx, w, out = oracle.moe_forward(x, ad, wr, None, 4, oracle.SIGMOID, gu, dn, wd_)
    perm = np.random.default_rng(10).permutation(wr.shape[0])   # new expert p <- old perm[p]
    inv = np.argsort(perm)
    idx2, w2, out2 = oracle.moe_forward(x, ad, np.ascontiguousarray(wr[perm]), None, 4,
                                        oracle.SIGMOID, np.ascontiguousarray(gu[perm]),
                                        np.ascontiguousarray(dn[perm]), wd_)
    assert np.array_equal(idx2, inv[idx])
    assert np.array_equal(w2, w)
    assert np.array_equal(out2, out)


def test_batch_invariance_rows_are_independent():
    x, ad, wr, gu, dn, wd_, _, _ = _small_layer(3, B=5)
    idx, w, out = oracle.moe_forward(x, ad, wr, None, 4, oracle.SIGMOID, gu, dn, wd_)
    for b in range(5):
        i1, w1, o1 = oracle.moe_forward(np.ascontiguousarray(x[b:b + 1]), ad, wr, None, 4,
                                        oracle.SIGMOID, gu, dn, wd_)
        assert np.array_equal(i1[0], idx[b]) and np.array_equal(w1[0], w[b])
        assert np.array_equal(o1[0], out[b])


def test_routing_invariants_on_a_realistic_recipe():
    w = W.scaled(W.WORKLOADS["full_b64"], H=512, I=64, E=128, k=16, B=6)
    L = W.make_layer(w, 0)
    x = W.make_x(w, 0)
    lg = oracle.router_logits(W.raw_numpy(x), oracle.BF16, W.raw_numpy(L["router_w"]))
    idx, wt = oracle.topk(lg, 16, oracle.SIGMOID)
    for b in range(6):
        assert len(set(idx[b].tolist())) == 16
        assert abs(wt[b].sum() - 1.0) <= 1e-12
        # the selected logits dominate the rest
        rest = np.setdiff1d(np.arange(128), idx[b])
        assert lg[b, idx[b]].min() >= lg[b, rest].max()


def test_thread_count_does_not_change_results():
    x, ad, wr, gu, dn, wd_, _, _ = _small_layer(4, B=2, H=128, I=64)
    oracle.set_threads(1)
    r1 = oracle.moe_forward(x, ad, wr, None, 4, oracle.SIGMOID, gu, dn, wd_)
    oracle.set_threads(max(2, oracle.max_threads()))
    r2 = oracle.moe_forward(x, ad, wr, None, 4, oracle.SIGMOID, gu, dn, wd_)
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)
