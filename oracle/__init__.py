"""CPU oracle of the decode-step MoE layer (test infrastructure only).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg
import this package.  The GPU library never links, loads or calls it, and
it shares no code with the GPU path.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision); this
module only builds it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16, E4M3 = 0, 1, 2
SOFTMAX, SIGMOID = 0, 1

_lib = None


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, d = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = d
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = d
    lib.oracle_round_bf16.argtypes = [d]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_router_logits.argtypes = [P, i32, i64, i32, i32, P, i32, P, P]
    lib.oracle_router_logits.restype = None
    lib.oracle_topk.argtypes = [P, i32, i32, i32, i32, P, P]
    lib.oracle_topk.restype = None
    lib.oracle_selection_weights.argtypes = [P, i32, i32, i32, i32, P, P]
    lib.oracle_selection_weights.restype = None
    lib.oracle_expert_ffn.argtypes = [P, i32, i32, i32, P, P, i32, P, P, P, P]
    lib.oracle_expert_ffn.restype = None
    lib.oracle_combine.argtypes = [P, i32, i64, i32, i32, i32, P, P, P]
    lib.oracle_combine.restype = None
    lib.oracle_moe_forward.argtypes = [P, i32, i32, i32, P, P, i32, i32, i32,
                                       P, P, i32, P, P, i32, P, P, P]
    lib.oracle_moe_forward.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_set_threads.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    _lib = lib
    return lib


# ------------------------------------------------------------------ helpers

_NP_OF = {F32: np.float32, BF16: np.uint16, E4M3: np.uint8}


def _raw(a: np.ndarray, dtype_code: int) -> np.ndarray:
    """Check that ``a`` holds raw storage of ``dtype_code`` and is C-contiguous."""
    want = _NP_OF[dtype_code]
    if a.dtype != want:
        raise TypeError(f"expected raw {np.dtype(want).name} storage, got {a.dtype}")
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def bf16_value(bits: int) -> float:
    return float(_load().oracle_bf16_value(int(bits)))


def e4m3_value(code: int) -> float:
    return float(_load().oracle_e4m3_value(int(code)))


def round_bf16(v: float) -> int:
    return int(_load().oracle_round_bf16(float(v)))


def router_logits(x, act, router_w, bias=None):
    """x: [B,H] raw act storage; router_w: [E,H] float32; bias: [E] or None."""
    x = _raw(x, act)
    router_w = _raw(router_w, F32)
    B, H = x.shape
    E = router_w.shape[0]
    assert router_w.shape[1] == H
    if bias is not None:
        bias = _raw(bias, F32)
    out = np.empty((B, E), np.float64)
    _load().oracle_router_logits(_ptr(x), act, H, B, H, _ptr(router_w), E,
                                 _ptr(bias), _ptr(out))
    return out


def topk(logits, k, score_fn):
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    B, E = logits.shape
    idx = np.empty((B, k), np.int32)
    w = np.empty((B, k), np.float64)
    _load().oracle_topk(_ptr(logits), B, E, k, score_fn, _ptr(idx), _ptr(w))
    return idx, w


def selection_weights(logits, idx, score_fn):
    """Renormalised weights of a given selection idx [B,k] (k distinct experts
    per row, any order) from logits [B,E]; the weights ``topk`` returns for its
    own selection."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, E = logits.shape
    k = idx.shape[1]
    assert idx.shape[0] == B and idx.min() >= 0 and idx.max() < E
    w = np.empty((B, k), np.float64)
    _load().oracle_selection_weights(_ptr(logits), B, E, k, score_fn, _ptr(idx), _ptr(w))
    return w


def expert_ffn(x_row, act, w_gate_up, w_down, wdt, s_gu=None, s_d=None):
    """One token through one expert.  w_gate_up: [2I,H], w_down: [H,I] raw."""
    x_row = _raw(x_row, act)
    w_gate_up = _raw(w_gate_up, wdt)
    w_down = _raw(w_down, wdt)
    two_i, H = w_gate_up.shape
    I = two_i // 2
    assert w_down.shape == (H, I) and x_row.shape == (H,)
    if s_gu is not None:
        s_gu = _raw(s_gu, F32)
        s_d = _raw(s_d, F32)
    h = np.empty(I, np.float64)
    y = np.empty(H, np.float64)
    _load().oracle_expert_ffn(_ptr(x_row), act, H, I, _ptr(w_gate_up), _ptr(w_down),
                              wdt, _ptr(s_gu), _ptr(s_d), _ptr(h), _ptr(y))
    return h, y


def combine(x, act, w, y):
    """x: [B,H] raw act; w: [B,k]; y: [B,k,H] -> out [B,H] float64."""
    x = _raw(x, act)
    B, H = x.shape
    k = w.shape[1]
    w = np.ascontiguousarray(w, np.float64)
    y = np.ascontiguousarray(y, np.float64)
    assert y.shape == (B, k, H)
    out = np.empty((B, H), np.float64)
    _load().oracle_combine(_ptr(x), act, H, B, H, k, _ptr(w), _ptr(y), _ptr(out))
    return out


def moe_forward(x, act, router_w, bias, k, score_fn, w_gate_up, w_down, wdt,
                s_gu=None, s_d=None):
    """Whole layer.  w_gate_up: [E,2I,H], w_down: [E,H,I] raw storage.

    Returns (idx [B,k] int32, w [B,k] float64, out [B,H] float64).
    """
    x = _raw(x, act)
    router_w = _raw(router_w, F32)
    w_gate_up = _raw(w_gate_up, wdt)
    w_down = _raw(w_down, wdt)
    B, H = x.shape
    E, two_i, H2 = w_gate_up.shape
    I = two_i // 2
    assert H2 == H and w_down.shape == (E, H, I) and router_w.shape == (E, H)
    if bias is not None:
        bias = _raw(bias, F32)
    if s_gu is not None:
        s_gu = _raw(s_gu, F32)
        s_d = _raw(s_d, F32)
        assert s_gu.shape == (E, 2 * I) and s_d.shape == (E, H)
    idx = np.empty((B, k), np.int32)
    w = np.empty((B, k), np.float64)
    out = np.empty((B, H), np.float64)
    rc = _load().oracle_moe_forward(_ptr(x), act, B, H, _ptr(router_w), _ptr(bias), E, k,
                                    score_fn, _ptr(w_gate_up), _ptr(w_down), wdt, _ptr(s_gu),
                                    _ptr(s_d), I, _ptr(idx), _ptr(w), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_moe_forward: size out of range")
    return idx, w, out
