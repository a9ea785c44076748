"""The C-ABI library on the CPU: it loads, exports what the header declares,
and its host-only checks answer without touching a GPU."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_decode_amd as M
from mixture_experts_layer_decode_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")


def declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", src, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert "moe_decode_forward" in names and "moe_decode_forward_ctx" in names
    assert set(names) == set(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = M.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_probe_library_exports_its_declared_symbol_and_checks_arguments():
    # measurement only: the streaming-read probe the benchmark compares with
    from mixture_experts_layer_decode_amd import build
    names = declared_functions(os.path.join(ROOT, "include", "moe_probe.h"))
    assert names == ["moe_probe_stream_read"]
    lib = ctypes.CDLL(build.PROBE_LIB)
    fn = lib.moe_probe_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int32
    # bad arguments are refused before any HIP call
    assert fn(None, 1 << 20, 16, None, None) == -1
    assert fn(16, 1 << 20, 0, None, 16) == -1
    assert fn(16, (1 << 20) + 16, 16, None, 16) == -1  # not whole 64 KB steps per workgroup
    assert fn(8, 1 << 20, 16, None, 16) == -1          # unaligned buffer


FULL = dict(E=896, H=7168, I=2048, weight_dtype=M.BF16, act_dtype=M.BF16, max_batch=64,
            max_topk=16)


def cfg(**kw):
    d = dict(FULL)
    d.update(kw)
    return M.make_config(d["E"], d["H"], d["I"], d["weight_dtype"], d["act_dtype"],
                         d["max_batch"], d["max_topk"])


@pytest.mark.parametrize("kw", [
    {},                                                     # full bf16 layer
    dict(weight_dtype=M.FP8_E4M3),                          # fp8 experts, bf16 activations
    dict(E=64, H=512, I=256, weight_dtype=M.F32, act_dtype=M.F32, max_batch=1, max_topk=4),
    dict(max_batch=1, max_topk=1),
    dict(E=2048, max_topk=32),
])
def test_supported_configs(kw):
    assert M.check_config(cfg(**kw)) == binding.OK, M.last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(max_batch=65), binding.ERR_UNSUPPORTED),          # beyond decode batches
    (dict(max_batch=0), binding.ERR_UNSUPPORTED),
    (dict(max_topk=33), binding.ERR_UNSUPPORTED),
    (dict(E=8, max_topk=9), binding.ERR_UNSUPPORTED),        # k > E
    (dict(H=7000), binding.ERR_UNSUPPORTED),
    (dict(H=512, weight_dtype=M.FP8_E4M3), binding.ERR_UNSUPPORTED),   # fp8 rows: 1024 multiple
    (dict(I=300), binding.ERR_UNSUPPORTED),
    (dict(E=4096), binding.ERR_UNSUPPORTED),
    (dict(weight_dtype=M.BF16, act_dtype=M.F32), binding.ERR_UNSUPPORTED),
    (dict(weight_dtype=7), binding.ERR_INVALID_ARG),
])
def test_unsupported_configs_are_refused(kw, status):
    assert M.check_config(cfg(**kw)) == status
    assert M.last_error() != ""


def test_null_config_is_invalid():
    lib = M.load_library()
    assert lib.moe_check_config(None) == binding.ERR_INVALID_ARG


def test_calls_without_a_context():
    lib = M.load_library()
    assert lib.moe_context_bind(None) == binding.OK
    assert lib.moe_decode_forward(None, None, None, None, None) == binding.ERR_NO_CONTEXT
    assert "no context" in M.last_error()
    assert lib.moe_decode_forward_ctx(None, None, None, None, None, None) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_set_path(None, 0, 0, 0) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_set_timing(None, 1) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_destroy(None) == binding.OK
    out = ctypes.c_void_p(1)
    assert lib.moe_context_create(None, None, ctypes.byref(out)) == binding.ERR_INVALID_ARG
    assert out.value is None


def test_last_error_is_per_thread_and_never_null():
    import threading
    M.check_config(cfg(H=7000))
    seen = {}

    def other():
        seen["msg"] = M.last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "hidden" in M.last_error()


def _noalloc_args(B, H, E, I, k, wdt=M.BF16, act=M.BF16):
    """moe_decode_forward_noalloc arguments with made-up (aligned, never
    dereferenced) device addresses: every check before the device work is
    host-only."""
    fake = 1 << 20
    es = {M.F32: 4, M.BF16: 2}[act]
    x = binding.MoeMat(fake, act, B, H, H)
    out = binding.MoeMat(fake + (1 << 30), act, B, H, H)
    r = binding.MoeMat(fake + (2 << 30), M.F32, E, H, H)
    ex = binding.MoeExperts(E, H, I, wdt, fake + (3 << 30), fake + (4 << 30),
                            (fake + (5 << 30)) if wdt == M.FP8_E4M3 else None,
                            (fake + (6 << 30)) if wdt == M.FP8_E4M3 else None)
    tk = binding.MoeTopk(k, M.SIGMOID, None, None, None)
    assert es * H % 16 == 0
    return [ctypes.byref(x), ctypes.byref(r), ctypes.byref(ex), ctypes.byref(tk), ctypes.byref(out),
            None]


def test_noalloc_refuses_a_workspace_beyond_its_scratch_array_before_device_work():
    lib = M.load_library()
    # 64 rows x top-32 of a 8192 / 8192 layer: 64 MiB of y alone
    assert lib.moe_decode_forward_noalloc(*_noalloc_args(64, 8192, 64, 8192, 32)) == \
        binding.ERR_UNSUPPORTED
    assert "scratch array" in M.last_error()


def test_noalloc_checks_its_arguments_on_the_host():
    lib = M.load_library()
    assert lib.moe_decode_forward_noalloc(None, None, None, None, None, None) == \
        binding.ERR_INVALID_ARG
    # 65 rows: beyond the decode batches
    assert lib.moe_decode_forward_noalloc(*_noalloc_args(65, 7168, 896, 2048, 16)) == \
        binding.ERR_UNSUPPORTED
    # fp8 weights without their scales
    args = _noalloc_args(4, 7168, 896, 2048, 16, wdt=M.FP8_E4M3)
    args[2]._obj.scale_gate_up = None
    assert lib.moe_decode_forward_noalloc(*args) == binding.ERR_INVALID_ARG
    # unaligned x
    args = _noalloc_args(4, 7168, 896, 2048, 16)
    args[0]._obj.data += 2
    assert lib.moe_decode_forward_noalloc(*args) == binding.ERR_INVALID_ARG
