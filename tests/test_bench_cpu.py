"""Host-side checks of the benchmark script and of the ABI calls that need no
device (CPU only)."""
import ctypes
import json
import os
import subprocess
import sys

import mixture_experts_layer_decode_amd as M
from mixture_experts_layer_decode_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2


def test_measured_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    assert bench.measured_traffic() in (None,) or bench.measured_traffic() > 0
    # a copy of the tree whose gate/up kernel differs reports no traffic
    fake = tmp_path / "repo"
    (fake / "profiles").mkdir(parents=True)
    csrc = fake / "mixture_experts_layer_decode_amd" / "csrc"
    csrc.mkdir(parents=True)
    src = os.path.join(ROOT, "mixture_experts_layer_decode_amd", "csrc")
    (fake / "profiles" / "hbm_traffic_full_b1.md").write_text(
        open(os.path.join(ROOT, "profiles", "hbm_traffic_full_b1.md")).read())
    (csrc / "expert_gemv.hip").write_text(open(os.path.join(src, "expert_gemv.hip")).read() + "\n")
    (csrc / "moe_device.h").write_text(open(os.path.join(src, "moe_device.h")).read())
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(fake / "bench.py"))
    assert bench.measured_traffic() is None


def test_context_calls_without_a_context():
    lib = M.load_library()
    n = ctypes.c_int64()
    assert lib.moe_context_set_prefetch(None, None, None, 0) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_get_timing(None, None, ctypes.byref(n), 0) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_last_plan(None, None) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_set_stream(None, None) == binding.ERR_NO_CONTEXT
    assert "ctx is NULL" in M.last_error()


def test_set_path_rejects_out_of_range_values_before_touching_a_device():
    lib = M.load_library()
    # no context: the context check comes first
    assert lib.moe_context_set_path(None, 3, 0, 0) == binding.ERR_NO_CONTEXT
