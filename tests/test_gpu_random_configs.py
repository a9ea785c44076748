"""GPU parity on seeded random configurations: every supported weight type,
hidden and intermediate widths on each type's row quantum, expert counts off
every tile size, k up to min(E, 32), batches 1 to 64, both routers, all three
paths (with split-K and a row threshold on the MFMA side), softmax or sigmoid,
with or without a Zipf bias, independent or correlated rows, the folded
combine on or off.  Each case is checked against the oracle on its first,
middle and last rows.  The configurations come from a fixed seed, so a failure
names a case that can be run again.

MOE_RANDOM_CONFIGS="n,seed,e_max" draws another set (default "32,2026,128"),
e.g. "2000,11,128" or "1000,13,2048" for a longer sweep."""
import os

import numpy as np
import pytest

import mixture_experts_layer_decode_amd as M
import workloads as W
from parity_helpers import full_check, make_context

pytestmark = pytest.mark.gpu

QUANTUM = {"bf16": 512, "fp8": 1024, "f32": 256}  # elements of one 16-byte vector per lane
PATHS = {"auto": M.PATH_AUTO, "gemv": M.PATH_GEMV, "mfma": M.PATH_MFMA}
ROUTERS = {"auto": M.ROUTER_AUTO, "gemv": M.ROUTER_GEMV, "mfma": M.ROUTER_MFMA}


def _configs(n=32, seed=2026, e_max=128):
    rng = np.random.RandomState(seed)
    out = []
    for i in range(n):
        wdt = ["bf16", "bf16", "fp8", "f32"][rng.randint(4)]
        q = QUANTUM[wdt]
        hq, iq = max(512, q), max(256, q)
        # widths up to 2048 keep |out| below 8, where one bf16 rounding of the
        # output stays inside the 2e-2 bound
        H = hq * rng.randint(1, 2048 // hq + 1)
        I = iq * rng.randint(1, 2048 // iq + 1)
        E = int(rng.randint(1, e_max + 1))
        k = int(rng.randint(1, min(E, 32) + 1))
        B = int([1, 2, 3, 5, 8, 9, 16, 31, 64][rng.randint(9)])
        path = ["auto", "gemv", "mfma"][rng.randint(3)]
        if wdt == "f32" and path == "mfma":
            path = "gemv"  # fp32 weights have no MFMA kernel
        cfg = dict(
            name=f"c{i:02d}", wdt=wdt, act="f32" if wdt == "f32" else "bf16", H=int(H), I=int(I),
            E=E, k=k, B=B, score=["sigmoid", "softmax"][rng.randint(2)],
            bias=[None, "zipf"][rng.randint(2)], x_kind=["normal", "correlated"][rng.randint(2)],
            path=path, router=["auto", "gemv", "mfma"][rng.randint(3)],
            split_k=int([1, 1, 2, 3][rng.randint(4)]) if path == "mfma" else 0,
            min_rows=int([0, 2, 3][rng.randint(3)]) if path == "auto" else 0,
            fused=bool(rng.randint(2)))
        out.append(cfg)
    return out


CONFIGS = _configs(*[int(v) for v in os.environ.get("MOE_RANDOM_CONFIGS", "32,2026,128").split(",")])


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c["name"] for c in CONFIGS])
def test_random_configuration_matches_the_oracle(cfg):
    print(f"[case] {cfg}", flush=True)
    w = W.scaled(W.WORKLOADS["full_b64"], name=cfg["name"], B=cfg["B"], H=cfg["H"], E=cfg["E"],
                 k=cfg["k"], I=cfg["I"], act=cfg["act"], wdt=cfg["wdt"], score=cfg["score"],
                 bias=cfg["bias"], x_kind=cfg["x_kind"])
    seed = 900 + int(cfg["name"][1:])  # the case's inputs follow from its name
    L = W.make_layer(w, seed, device="cuda")
    x = W.make_x(w, seed, device="cuda")
    ctx = make_context(w)
    ctx.set_path(PATHS[cfg["path"]], cfg["min_rows"], cfg["split_k"])
    ctx.set_router(ROUTERS[cfg["router"]])
    ctx.set_fused_combine(cfg["fused"])
    B = cfg["B"]
    full_check(ctx, w, L, x, rows=sorted({0, B // 2, B - 1}))
    plan = ctx.last_plan()
    assert plan["gemv"] + plan["mfma"] == plan["distinct"]
    if cfg["path"] == "mfma":
        assert plan["gemv"] == 0
    if cfg["path"] == "gemv" or cfg["wdt"] == "f32":
        assert plan["mfma"] == 0
