"""Host-side checks of the benchmark script and of the ABI calls that need no
device (CPU only)."""
import ctypes
import json
import os
import subprocess
import sys

import pytest

import mixture_experts_layer_decode_amd as M
from mixture_experts_layer_decode_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2


def _tree_with_gate_up_source(tmp_path, name, extra):
    """A copy of the files the traffic guard reads, with `extra` appended to
    the gate/up kernel's source."""
    fake = tmp_path / name
    (fake / "profiles").mkdir(parents=True)
    csrc = fake / "mixture_experts_layer_decode_amd" / "csrc"
    csrc.mkdir(parents=True)
    src = os.path.join(ROOT, "mixture_experts_layer_decode_amd", "csrc")
    (fake / "profiles" / "hbm_traffic_full_b1.md").write_text(
        open(os.path.join(ROOT, "profiles", "hbm_traffic_full_b1.md")).read())
    (csrc / "expert_gemv.hip").write_text(open(os.path.join(src, "expert_gemv.hip")).read() + extra)
    (csrc / "moe_device.h").write_text(open(os.path.join(src, "moe_device.h")).read())
    return fake


def test_measured_traffic_follows_the_kernel_code(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    have = bench.measured_traffic()
    assert have is None or have > 0
    # comments and blank lines do not change the code the counters were taken on
    same = _tree_with_gate_up_source(tmp_path, "same", "\n// a note\n/* another\n note */\n\n")
    assert bench.gate_up_code_digest(str(same)) == bench.gate_up_code_digest(ROOT)
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(same / "bench.py"))
    assert bench.measured_traffic() == have
    # a copy whose gate/up code differs reports no traffic
    other = _tree_with_gate_up_source(tmp_path, "other", "\nstatic const int k_other = 1;\n")
    assert bench.gate_up_code_digest(str(other)) != bench.gate_up_code_digest(ROOT)
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(other / "bench.py"))
    assert bench.measured_traffic() is None


def test_context_calls_without_a_context():
    lib = M.load_library()
    n = ctypes.c_int64()
    assert lib.moe_context_set_prefetch(None, None, None, 0) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_set_prefetch_mode(None, 0, 0) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_set_fused_select(None, 1) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_set_fused_next_router(None, 1) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_get_timing(None, None, ctypes.byref(n), 0) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_last_plan(None, None) == binding.ERR_NO_CONTEXT
    assert lib.moe_context_set_stream(None, None) == binding.ERR_NO_CONTEXT
    assert "ctx is NULL" in M.last_error()


def test_set_path_rejects_out_of_range_values_before_touching_a_device():
    lib = M.load_library()
    # no context: the context check comes first
    assert lib.moe_context_set_path(None, 3, 0, 0) == binding.ERR_NO_CONTEXT


def test_binding_checks_the_tensors_the_library_sees_only_as_pointers():
    import torch
    E, H, I, B, k = 4, 512, 256, 2, 2
    x = torch.zeros(B, H, dtype=torch.bfloat16)
    gu = torch.zeros(E, 2 * I, H, dtype=torch.bfloat16)
    dn = torch.zeros(E, H, I, dtype=torch.bfloat16)
    ok = dict(bias=torch.zeros(E), idx_out=torch.zeros(B, k, dtype=torch.int32),
              weight_out=torch.zeros(B, k))
    binding.check_forward_tensors(x, gu, dn, k, **ok)
    bad = [
        dict(idx_out=torch.zeros(B, k - 1, dtype=torch.int32)),   # too small: kernel writes B*k
        dict(idx_out=torch.zeros(B, k, dtype=torch.int64)),
        dict(weight_out=torch.zeros(B * k + 1)),
        dict(bias=torch.zeros(E - 1)),
        dict(s_gu=torch.zeros(E, I), s_d=torch.zeros(E, H)),
        dict(s_gu=torch.zeros(E, 2 * I), s_d=torch.zeros(E, I)),
        dict(idx_out=torch.zeros(k, B, dtype=torch.int32).t()),   # not contiguous
    ]
    for kw in bad:
        args = dict(ok)
        args.update(kw)
        with pytest.raises(ValueError):
            binding.check_forward_tensors(x, gu, dn, k, **args)
    with pytest.raises(ValueError):
        binding.check_forward_tensors(x, gu, torch.zeros(E, H, I + 256, dtype=torch.bfloat16), k)
    with pytest.raises(ValueError):
        binding.check_forward_tensors(x, gu, dn.float(), k)


def test_input_step_makes_every_forward_take_one_batch(monkeypatch):
    # --input-step: the timed forwards all take one input batch (for counter
    # runs whose dispatches should select the same experts); by default they
    # cycle through N_INPUTS different batches
    import torch

    sys.path.insert(0, ROOT)
    import bench
    import workloads as W

    w = W.WORKLOADS["tiny_b1"]
    run = object.__new__(bench.Runner)
    run.W, run.torch, run.dev, run.w, run.layers = W, torch, "cpu", w, [None]
    monkeypatch.setattr(bench, "INPUT_STEP", None)
    xs, idxs, outs = run.inputs(2, w)
    assert len(xs) == bench.N_INPUTS and not torch.equal(xs[0], xs[1])
    monkeypatch.setattr(bench, "INPUT_STEP", 3)
    xs, idxs, outs = run.inputs(2, w)
    want = W.make_x(w, 0, step=3, device="cpu", B=2)
    assert len(xs) == bench.N_INPUTS and all(torch.equal(x, want) for x in xs)
