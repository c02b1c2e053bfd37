"""The expert layer at the limits the ABI states (H or I = 65536, K = 64 slots per token,
E_total = 1024 experts), on the small-block, 64-row and 128-row (LDS-staged, tiled
weights) kernels, against the oracle.  Shapes are otherwise small so the oracle finishes
in seconds."""
import numpy as np
import pytest

from gpu_common import run_layer, say, synth
from test_gpu_forward import W4A16, W4A4, FP8B, full_check, small

pytestmark = pytest.mark.gpu

CASES = [
    # name, workload ctor, block_m[, tiled]
    ("H65536-w4a16-bm16", lambda: small(W4A16, T=5, H=65536, I=64, E=3, k=2, seed=61), 16),
    ("H65536-w4a16-bm64", lambda: small(W4A16, T=5, H=65536, I=64, E=3, k=2, seed=61), 64),
    ("H65536-w4a4-bm16", lambda: small(W4A4, T=4, H=65536, I=64, E=3, k=2, seed=62), 16),
    ("I65536-w4a16-bm16", lambda: small(W4A16, T=5, H=64, I=65536, E=3, k=2, seed=63), 16),
    ("I65536-fp8b-bm64", lambda: small(FP8B, T=4, H=128, I=65536, E=3, k=2, seed=64), 64),
    ("K64-E1024-bm16", lambda: small(W4A16, T=6, H=128, I=64, E=992, k=32, n_shared=32, seed=65), 16),
    ("K64-E1024-bm64", lambda: small(W4A16, T=6, H=128, I=64, E=992, k=32, n_shared=32, seed=65), 64),
    ("H65536-w4a16-bm128-tiled", lambda: small(W4A16, T=5, H=65536, I=64, E=3, k=2, seed=61), 128, True),
    ("H65536-w4a4-bm128-tiled", lambda: small(W4A4, T=4, H=65536, I=64, E=3, k=2, seed=62), 128, True),
    ("I65536-fp8b-bm128-tiled", lambda: small(FP8B, T=4, H=128, I=65536, E=3, k=2, seed=64), 128, True),
    ("K64-E1024-bm128-tiled", lambda: small(W4A16, T=6, H=128, I=64, E=992, k=32, n_shared=32, seed=65), 128, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_abi_limits(case):
    name, make, bm = case[:3]
    tiled = len(case) > 3 and case[3]
    w = make()
    say(f"limits {name}: T={w.T} H={w.H} I={w.I} E={w.E}+{w.n_shared} k={w.topk} K={w.K} bm={bm}")
    assert w.K <= 64 and w.E_total <= 1024 and max(w.H, w.I) <= 65536
    data = synth.make_all(w)
    res = run_layer(w, data, block_m=bm, tiled=tiled)
    assert res["bm"] == bm
    if w.n_shared:
        assert np.all(res["ids"][:, w.topk:] == w.E + np.arange(w.n_shared))
    full_check(w, data, res, what=f"limits/{name}")
