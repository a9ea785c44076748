"""The layer from plain C: tests/c_abi_forward.c calls libmoe_decode.so
through include/moe_decode.h with HIP device memory (no Python, no PyTorch
on the path) at batch 1 and 4 and checks it against the C oracle; built by
__graft_entry__.build()."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "c_abi_forward")


def test_the_layer_from_plain_c_matches_the_oracle():
    assert os.path.exists(EXE), "tests/_build/c_abi_forward is not built (run __graft_entry__.build())"
    print("[case] c_abi_forward: batch 1 and 4 of a 32-expert bf16 layer", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.strip().splitlines()[-1] == "c abi ok"
