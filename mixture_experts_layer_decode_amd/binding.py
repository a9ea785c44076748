"""ctypes binding of libmoe_decode.so (include/moe_decode.h).

Argument marshalling only: torch tensors provide device memory and the HIP
stream; every step of the layer runs in the library's kernels.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch  # loads the HIP runtime that the library then shares

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_decode.so")

# moe_status
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_DEVICE, ERR_NO_CONTEXT = 0, -1, -2, -3, -4
# moe_dtype
F32, BF16, FP8_E4M3 = 0, 1, 2
# moe_score_fn
SOFTMAX, SIGMOID = 0, 1
# moe_path
PATH_AUTO, PATH_GEMV, PATH_MFMA = 0, 1, 2
# moe_router_kernel
ROUTER_AUTO, ROUTER_GEMV, ROUTER_MFMA = 0, 1, 2
# moe_stage
STAGES = ("router", "gate_up", "down", "combine")

_STATUS_NAMES = {OK: "MOE_OK", ERR_INVALID_ARG: "MOE_ERR_INVALID_ARG",
                 ERR_UNSUPPORTED: "MOE_ERR_UNSUPPORTED", ERR_DEVICE: "MOE_ERR_DEVICE",
                 ERR_NO_CONTEXT: "MOE_ERR_NO_CONTEXT"}

# Names the header declares (the CPU test checks the library exports each).
EXPORTS = (
    "moe_check_config", "moe_context_create", "moe_context_set_stream",
    "moe_context_set_path", "moe_context_set_router", "moe_context_set_fused_combine",
    "moe_context_set_fused_select", "moe_context_set_fused_next_router",
    "moe_decode_forward_stack",
    "moe_context_set_prefetch", "moe_context_set_prefetch_mode",
    "moe_context_set_timing",
    "moe_context_get_timing", "moe_context_last_plan", "moe_context_bind",
    "moe_decode_forward", "moe_decode_forward_ctx", "moe_decode_forward_noalloc",
    "moe_context_destroy", "moe_last_error",
)


class MoeMat(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("row_stride", ctypes.c_int64)]


class MoeExperts(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("scale_gate_up", ctypes.c_void_p), ("scale_down", ctypes.c_void_p)]


class MoeTopk(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("score_fn", ctypes.c_int32), ("bias", ctypes.c_void_p),
                ("idx_out", ctypes.c_void_p), ("weight_out", ctypes.c_void_p)]


class MoeConfig(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_topk", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH, build_if_missing: bool = True):
    """Load libmoe_decode.so (building it first only if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        if not build_if_missing:
            raise RuntimeError(f"{path} is not built")
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "moe_check_config": ([P], i32),
        "moe_context_create": ([P, P, ctypes.POINTER(P)], i32),
        "moe_context_set_stream": ([P, P], i32),
        "moe_context_set_path": ([P, i32, i32, i32], i32),
        "moe_context_set_router": ([P, i32], i32),
        "moe_context_set_fused_combine": ([P, i32], i32),
        "moe_context_set_fused_select": ([P, i32], i32),
        "moe_context_set_fused_next_router": ([P, i32], i32),
        "moe_decode_forward_stack": ([P, P, i32, P, P, P, P], i32),
        "moe_context_set_prefetch": ([P, P, P, i32], i32),
        "moe_context_set_prefetch_mode": ([P, i32, i32], i32),
        "moe_context_set_timing": ([P, i32], i32),
        "moe_context_get_timing": ([P, P, P, i32], i32),
        "moe_context_last_plan": ([P, P], i32),
        "moe_context_bind": ([P], i32),
        "moe_decode_forward": ([P, P, P, P, P], i32),
        "moe_decode_forward_ctx": ([P, P, P, P, P, P], i32),
        "moe_decode_forward_noalloc": ([P, P, P, P, P, P], i32),
        "moe_context_destroy": ([P], i32),
        "moe_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().moe_last_error().decode()


def _check(status: int) -> None:
    if status != OK:
        raise MoeError(status, last_error())


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _dev_ptr(t: Optional[torch.Tensor], name: str) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _mat(t: torch.Tensor, name: str) -> MoeMat:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    return MoeMat(_dev_ptr(t, name), dtype_code(t), t.shape[0], t.shape[1], t.stride(0))


def check_forward_tensors(x, w_gate_up, w_down, k, bias=None, s_gu=None, s_d=None,
                          idx_out=None, weight_out=None) -> None:
    """Shapes and dtypes of the tensors whose sizes the C ABI cannot see (it
    takes their data pointers only): the library would read or write past a
    tensor that is too small.  Raises ValueError; touches no device."""
    if w_gate_up.dim() != 3 or w_down.dim() != 3:
        raise ValueError("w_gate_up must be [E, 2I, H] and w_down [E, H, I]")
    E, two_i, H = w_gate_up.shape
    if two_i % 2 or tuple(w_down.shape) != (E, H, two_i // 2):
        raise ValueError(f"w_down {tuple(w_down.shape)} does not match w_gate_up "
                         f"{tuple(w_gate_up.shape)} (expected [E, H, I])")
    if w_gate_up.dtype != w_down.dtype:
        raise ValueError("w_gate_up and w_down must have the same dtype")
    for name, t in (("w_gate_up", w_gate_up), ("w_down", w_down)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    # x and out travel with their shapes and strides, which the library checks
    if x.dim() != 2:
        raise ValueError("x must be [B, H]")
    B = x.shape[0]
    wants = (("bias", bias, torch.float32, (E,)),
             ("s_gu", s_gu, torch.float32, (E, two_i)),
             ("s_d", s_d, torch.float32, (E, H)),
             ("idx_out", idx_out, torch.int32, (B, k)),
             ("weight_out", weight_out, torch.float32, (B, k)))
    for name, t, dt, shape in wants:
        if t is None:
            continue
        if t.dtype != dt:
            raise ValueError(f"{name} must be {dt}, got {t.dtype}")
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def make_config(E: int, H: int, I: int, weight_dtype: int, act_dtype: int, max_batch: int,
                max_topk: int) -> MoeConfig:
    return MoeConfig(E, H, I, weight_dtype, act_dtype, max_batch, max_topk)


def check_config(cfg: MoeConfig) -> int:
    """Host-only support check; returns the moe_status (no exception)."""
    return int(load_library().moe_check_config(ctypes.byref(cfg)))


class Context:
    """A moe_context on the current device (workspace allocated once)."""

    def __init__(self, E: int, H: int, I: int, weight_dtype: int, act_dtype: int,
                 max_batch: int = 64, max_topk: int = 16, stream=None):
        lib = load_library()
        self._lib = lib
        self.cfg = make_config(E, H, I, weight_dtype, act_dtype, max_batch, max_topk)
        handle = ctypes.c_void_p()
        s = torch.cuda.current_stream() if stream is None else stream
        _check(lib.moe_context_create(ctypes.byref(self.cfg), ctypes.c_void_p(s.cuda_stream),
                                      ctypes.byref(handle)))
        self._h = handle

    @property
    def handle(self):
        return self._h

    def close(self) -> None:
        # the handle is dropped first: the library frees the context even when
        # it reports a failure, so it must never be passed again
        h, self._h = self._h, None
        if h:
            _check(self._lib.moe_context_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_path(self, path: int, mfma_min_rows: int = 0, split_k: int = 0) -> None:
        _check(self._lib.moe_context_set_path(self._h, path, mfma_min_rows, split_k))

    def set_router(self, kernel: int) -> None:
        _check(self._lib.moe_context_set_router(self._h, kernel))

    def set_fused_combine(self, enable: bool) -> None:
        _check(self._lib.moe_context_set_fused_combine(self._h, 1 if enable else 0))

    def set_fused_next_router(self, enable: bool) -> None:
        _check(self._lib.moe_context_set_fused_next_router(self._h, 1 if enable else 0))

    def forward_stack(self, x: torch.Tensor, layers: Sequence[dict], k: int, score_fn: int,
                      outs: Optional[Sequence[torch.Tensor]] = None,
                      idx_outs: Optional[Sequence[Optional[torch.Tensor]]] = None,
                      weight_outs: Optional[Sequence[Optional[torch.Tensor]]] = None):
        """Queue len(layers) consecutive layers on torch's current stream
        (moe_decode_forward_stack); each layer is a dict with router_w,
        w_gate_up, w_down and optionally bias, s_gu, s_d.  Returns the
        outputs (layer l's output is layer l+1's input)."""
        n = len(layers)
        if n < 1:
            raise ValueError("at least one layer")
        outs = [torch.empty_like(x) for _ in range(n)] if outs is None else list(outs)
        idx_outs = [None] * n if idx_outs is None else list(idx_outs)
        weight_outs = [None] * n if weight_outs is None else list(weight_outs)
        if not (len(outs) == len(idx_outs) == len(weight_outs) == n):
            raise ValueError("one output (and routing output) per layer")
        mats_r = (MoeMat * n)()
        exps = (MoeExperts * n)()
        tks = (MoeTopk * n)()
        mats_o = (MoeMat * n)()
        for l, L in enumerate(layers):
            xin = x if l == 0 else outs[l - 1]
            check_forward_tensors(xin, L["w_gate_up"], L["w_down"], k, L.get("bias"),
                                  L.get("s_gu"), L.get("s_d"), idx_outs[l], weight_outs[l])
            E, two_i, H = L["w_gate_up"].shape
            mats_r[l] = _mat(L["router_w"], "router_w")
            exps[l] = MoeExperts(E, H, two_i // 2, dtype_code(L["w_gate_up"]),
                                 _dev_ptr(L["w_gate_up"], "w_gate_up"),
                                 _dev_ptr(L["w_down"], "w_down"), _dev_ptr(L.get("s_gu"), "s_gu"),
                                 _dev_ptr(L.get("s_d"), "s_d"))
            tks[l] = MoeTopk(k, score_fn, _dev_ptr(L.get("bias"), "bias"),
                             _dev_ptr(idx_outs[l], "idx_out"), _dev_ptr(weight_outs[l], "weight_out"))
            mats_o[l] = _mat(outs[l], "out")
        xm = _mat(x, "x")
        s = torch.cuda.current_stream(x.device)
        _check(self._lib.moe_context_set_stream(self._h, ctypes.c_void_p(s.cuda_stream)))
        _check(self._lib.moe_decode_forward_stack(self._h, ctypes.byref(xm), n, mats_r, exps, tks,
                                                  mats_o))
        return outs

    def set_fused_select(self, enable: bool) -> None:
        _check(self._lib.moe_context_set_fused_select(self._h, 1 if enable else 0))

    def set_prefetch(self, tensors: Sequence[torch.Tensor]) -> None:
        n = len(tensors)
        ptrs = (ctypes.c_void_p * max(1, n))(*[_dev_ptr(t, "prefetch") for t in tensors])
        nbytes = (ctypes.c_int64 * max(1, n))(*[t.numel() * t.element_size() for t in tensors])
        self._keep_prefetch = list(tensors)
        _check(self._lib.moe_context_set_prefetch(self._h, ptrs, nbytes, n))

    def set_prefetch_mode(self, start: int = 0, grid: int = 0) -> None:
        """When the warm-up starts (0: after routing, 1: with the forward) and
        its kernel's workgroups (0: the default)."""
        _check(self._lib.moe_context_set_prefetch_mode(self._h, start, grid))

    def set_timing(self, enable: bool) -> None:
        _check(self._lib.moe_context_set_timing(self._h, 1 if enable else 0))

    def get_timing(self, reset: bool = False):
        """(per-stage milliseconds summed over timed forwards, their count)."""
        ms = (ctypes.c_double * len(STAGES))()
        count = ctypes.c_int64()
        _check(self._lib.moe_context_get_timing(self._h, ms, ctypes.byref(count),
                                                1 if reset else 0))
        return dict(zip(STAGES, list(ms))), int(count.value)

    def last_plan(self):
        """Routing-plan counters of the last forward (synchronises the stream)."""
        out = (ctypes.c_int32 * 6)()
        _check(self._lib.moe_context_last_plan(self._h, out))
        return dict(distinct=out[0], gemv=out[1], mfma=out[2], max_rows=out[3], launches=out[4],
                    router=out[5])

    def bind(self) -> None:
        _check(self._lib.moe_context_bind(self._h))

    def forward(self, x: torch.Tensor, router_w: torch.Tensor, w_gate_up: torch.Tensor,
                w_down: torch.Tensor, k: int, score_fn: int, bias=None, s_gu=None, s_d=None,
                out: Optional[torch.Tensor] = None, idx_out: Optional[torch.Tensor] = None,
                weight_out: Optional[torch.Tensor] = None, use_bound: bool = False):
        """Queue one layer on torch's current stream; returns out."""
        check_forward_tensors(x, w_gate_up, w_down, k, bias, s_gu, s_d, idx_out, weight_out)
        if out is None:
            out = torch.empty_like(x)
        E, two_i, H = w_gate_up.shape
        xm, rm, om = _mat(x, "x"), _mat(router_w, "router_w"), _mat(out, "out")
        ex = MoeExperts(E, H, two_i // 2, dtype_code(w_gate_up), _dev_ptr(w_gate_up, "w_gate_up"),
                        _dev_ptr(w_down, "w_down"), _dev_ptr(s_gu, "s_gu"), _dev_ptr(s_d, "s_d"))
        tk = MoeTopk(k, score_fn, _dev_ptr(bias, "bias"), _dev_ptr(idx_out, "idx_out"),
                     _dev_ptr(weight_out, "weight_out"))
        s = torch.cuda.current_stream(x.device)
        _check(self._lib.moe_context_set_stream(self._h, ctypes.c_void_p(s.cuda_stream)))
        if use_bound:
            st = self._lib.moe_decode_forward(ctypes.byref(xm), ctypes.byref(rm), ctypes.byref(ex),
                                              ctypes.byref(tk), ctypes.byref(om))
        else:
            st = self._lib.moe_decode_forward_ctx(self._h, ctypes.byref(xm), ctypes.byref(rm),
                                                  ctypes.byref(ex), ctypes.byref(tk),
                                                  ctypes.byref(om))
        _check(st)
        return out


def forward_noalloc(x: torch.Tensor, router_w: torch.Tensor, w_gate_up: torch.Tensor,
                    w_down: torch.Tensor, k: int, score_fn: int, bias=None, s_gu=None, s_d=None,
                    out: Optional[torch.Tensor] = None, idx_out: Optional[torch.Tensor] = None,
                    weight_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Queue one layer on torch's current stream through
    moe_decode_forward_noalloc (no context; the library's fixed scratch
    array as workspace); returns out.  ``out`` is allocated here when not
    given: pass it to keep the call allocation-free."""
    lib = load_library()
    check_forward_tensors(x, w_gate_up, w_down, k, bias, s_gu, s_d, idx_out, weight_out)
    if out is None:
        out = torch.empty_like(x)
    E, two_i, H = w_gate_up.shape
    xm, rm, om = _mat(x, "x"), _mat(router_w, "router_w"), _mat(out, "out")
    ex = MoeExperts(E, H, two_i // 2, dtype_code(w_gate_up), _dev_ptr(w_gate_up, "w_gate_up"),
                    _dev_ptr(w_down, "w_down"), _dev_ptr(s_gu, "s_gu"), _dev_ptr(s_d, "s_d"))
    tk = MoeTopk(k, score_fn, _dev_ptr(bias, "bias"), _dev_ptr(idx_out, "idx_out"),
                 _dev_ptr(weight_out, "weight_out"))
    s = torch.cuda.current_stream(x.device)
    _check(lib.moe_decode_forward_noalloc(ctypes.byref(xm), ctypes.byref(rm), ctypes.byref(ex),
                                          ctypes.byref(tk), ctypes.byref(om),
                                          ctypes.c_void_p(s.cuda_stream)))
    return out
