"""Host-side logic of bench.py: the algorithmic bytes and flops every roofline fraction is
taken against, checked against figures worked out by hand from the weight formats, and
the single-GPU contract (no GPU needed)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from quantized_mixture_experts_softmax_amd import synth  # noqa: E402


def all_hit(T, topk, E, n_shared=0):
    """Slot ids that use every routed expert (and every shared one)."""
    ids = (np.arange(T)[:, None] * topk + np.arange(topk)[None, :]) % E
    if n_shared:
        ids = np.concatenate([ids, E + np.tile(np.arange(n_shared), (T, 1))], axis=1)
    return ids.astype(np.int32)


def test_decode_bytes_and_flops():
    # MXFP4: per weight row of K values, K/2 code bytes and K/32 E8M0 bytes.  w13 of one
    # expert: 2 * 2880 rows * (1440 + 90) B = 8,812,800 B; w2: 2880 * 1530 = 4,406,400 B.
    w = synth.WORKLOADS["decode"]
    a = bench.algorithmic(w, all_hit(64, 4, 32))
    assert a["n_hit"] == 32 and a["slots"] == 256
    # 32 experts of both projections, x and out (64 x 2880 bf16 each)
    assert a["step_bytes"] == 32 * (8_812_800 + 4_406_400) + 2 * 64 * 2880 * 2 == 423_751_680
    # stage 1 reads w13, x and writes h (256 slots x 2880 bf16)
    assert a["gemm1_bytes"] == 32 * 8_812_800 + 64 * 2880 * 2 + 256 * 2880 * 2 == 283_852_800
    assert a["gemm1_flops"] == 2 * 256 * 2880 * 5760
    assert a["step_flops"] == 6 * 256 * 2880 * 2880


def test_fp8_block_bytes_and_flops():
    # FP8 e4m3 codes (1 B) plus one fp32 scale per 128 x 128 block: w13 of one expert is
    # 4096 x 7168 codes + 32 x 56 scales; w2 7168 x 2048 codes + 56 x 16 scales; 256 routed
    # experts and the shared one, all hit
    w = synth.WORKLOADS["fp8-block"]
    a = bench.algorithmic(w, all_hit(4096, 8, 256, n_shared=1))
    per = (4096 * 7168 + 4 * 32 * 56) + (7168 * 2048 + 4 * 56 * 16)
    assert per == 44_050_944
    assert a["n_hit"] == 257 and a["slots"] == 4096 * 9
    assert a["step_bytes"] == 257 * per + 2 * 4096 * 7168 * 2 == 11_438_533_120
    assert a["step_flops"] == 6 * 4096 * 9 * 7168 * 2048


def test_fp8_channel_bytes_and_flops():
    # FP8 codes plus one fp32 scale per output row: w13 28672 x 4096 codes + 28672 scales,
    # w2 4096 x 14336 codes + 4096 scales
    w = synth.WORKLOADS["fp8-channel"]
    per = (28672 * 4096 + 4 * 28672) + (4096 * 14336 + 4 * 4096)
    a = bench.algorithmic(w, all_hit(4096, 2, 8))
    assert a["step_bytes"] == 8 * per + 2 * 4096 * 4096 * 2 == 1_477_443_584
    # one token: only its two experts' weights count
    w1 = w.with_T(1)
    a1 = bench.algorithmic(w1, np.array([[3, 5]], np.int32))
    assert a1["n_hit"] == 2 and a1["step_bytes"] == 2 * per + 2 * 4096 * 2


def test_ids_outside_the_experts_do_not_count():
    # an expert-parallel share marks other devices' slots with -1: no weights, no rows
    w = synth.WORKLOADS["decode"]
    ids = all_hit(64, 4, 32)
    ids[:, 2:] = -1
    a = bench.algorithmic(w, ids)
    assert a["slots"] == 128 and a["gemm1_flops"] == 2 * 128 * 2880 * 5760


def test_step_roofline_picks_the_binding_roof():
    w = synth.WORKLOADS["decode"]
    a = bench.algorithmic(w, all_hit(64, 4, 32))
    ms = 0.1
    r = bench.step_roofline(w, a, ms)
    t_hbm = a["step_bytes"] / (bench.HBM_PEAK_GBS * 1e9)
    assert r["bound"] == "hbm" and abs(r["frac"] - t_hbm / (ms * 1e-3)) < 1e-4
    # prefill w4a16: bf16 MFMA time exceeds the HBM time
    wp = synth.WORKLOADS["prefill"]
    ap = bench.algorithmic(wp, all_hit(8192, 4, 128))
    rp = bench.step_roofline(wp, ap, 2.0)
    assert rp["bound"] == "mfma-bf16" and rp["mfma_frac"] > rp["hbm_frac"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)
