"""GPU parity of the unquantised bf16 expert layer (bf16 weights and activations over the
canonical layout; the persistent 16-row kernel and the 64/128-row kernel) against the oracle, under the output
bound of the quantised paths: max|gpu - oracle| <= 2e-2 * rms and per-token relative
L2 <= 1e-2 on the fp32 result, the bf16 output its round-to-nearest-even bit for bit.
"""
import numpy as np
import pytest

from gpu_common import B, run_layer, say, synth
from test_gpu_forward import full_check, small

pytestmark = pytest.mark.gpu

BF = (synth.W_BF16, synth.A_BF16)


def _no_scales_oai(w, data, interleaved, bias, kind=1):
    """SwiGLU-OAI / SiLU spec with optional interleaved w1 rows and biases (bf16 weights
    carry no scales to permute)."""
    act = dict(kind=kind, alpha=1.702, beta=1.0, limit=7.0, interleaved=interleaved)
    b1, b2 = synth.make_biases(w) if bias else (None, None)
    if interleaved:
        data = dict(data, w1=synth.interleave_rows(data["w1"], w.I))
        b1 = synth.interleave_rows(b1, w.I) if b1 is not None else None
    act.update(w1_bias=b1, w2_bias=b2)
    return act, data


CASES = [
    # name, workload, block_m
    ("ragged-bm16", lambda: small(BF, T=40, H=320, I=288, E=6, k=2, seed=51), 16),
    ("shared-sigmoid-bm16", lambda: small(BF, T=50, H=352, I=416, E=5, k=3, n_shared=1,
                                          score=synth.SCORE_SIGMOID, seed=52), 16),
    ("single-token-bm16", lambda: small(BF, T=1, H=256, I=160, E=4, k=2, seed=53), 16),
    ("max-K-bm16", lambda: small(BF, T=20, H=2944, I=2944, E=3, k=2, seed=58), 16),
    ("ragged-bm64", lambda: small(BF, T=40, H=320, I=288, E=6, k=2, seed=51), 64),
    ("ragged-bm128", lambda: small(BF, T=40, H=320, I=288, E=6, k=2, seed=51), 128),
    ("shared-sigmoid-bm64", lambda: small(BF, T=50, H=352, I=416, E=5, k=3, n_shared=1,
                                          score=synth.SCORE_SIGMOID, seed=52), 64),
    ("single-token-bm64", lambda: small(BF, T=1, H=256, I=160, E=4, k=2, seed=53), 64),
    ("many-blocks-bm128", lambda: small(BF, T=300, H=256, I=192, E=8, k=4, seed=54), 128),
]


@pytest.mark.parametrize("name,make,bm", CASES, ids=[c[0] for c in CASES])
def test_bf16_small(name, make, bm):
    # H=320 / I=288: several 128-K chunks with a 64-element tail, ragged 32-column strips, pad rows
    w = make()
    say(f"bf16 forward {name}: T={w.T} H={w.H} I={w.I} E={w.E}+{w.n_shared} k={w.topk} bm={bm}")
    data = synth.make_all(w)
    res = run_layer(w, data, block_m=bm)
    assert res["bm"] == bm
    full_check(w, data, res, what=f"bf16/{name}")


@pytest.mark.parametrize("bm,itl,bias,kind", [(16, True, True, 1), (16, False, True, 0), (64, True, True, 1),
                                              (128, True, True, 1), (64, False, True, 0), (128, False, False, 1)])
def test_bf16_act_bias(bm, itl, bias, kind):
    w = small(BF, T=45, H=320, I=288, E=8, k=2, seed=55)
    data = synth.make_all(w)
    act, data = _no_scales_oai(w, data, itl, bias, kind)
    what = f"bf16/bm{bm}/{'itl' if itl else 'sep'}/{'bias' if bias else 'nobias'}/{'oai' if kind else 'silu'}"
    say(f"forward {what}")
    res = run_layer(w, data, block_m=bm, act=act)
    full_check(w, data, res, what=what, act=act)


@pytest.mark.parametrize("bm", [16, 64])
def test_bf16_router_weight_on_input(bm):
    w = small(BF, T=40, H=320, I=288, E=6, k=1, score=synth.SCORE_SIGMOID, seed=56)
    data = synth.make_all(w)
    act = dict(kind=0, weight_on_input=True)
    res = run_layer(w, data, block_m=bm, act=act)
    full_check(w, data, res, what=f"bf16/tkw1/bm{bm}", act=act)


@pytest.mark.parametrize("H,want", [(256, 16), (3072, 64)])
def test_bf16_default_block_m(H, want):
    """Small batches take 16-row blocks while the activation tile fits the persistent
    kernel (H, I <= 2944) and 64-row blocks past that."""
    w = small(BF, T=8, H=H, I=256, E=16, k=2, seed=57)
    data = synth.make_all(w)
    res = run_layer(w, data)
    assert res["bm"] == want
    full_check(w, data, res, what=f"bf16/default-bm/H{H}")


def test_bf16_decode_full_size():
    """The decode-shaped layer (T=64, H=I=2880, 32 experts, top-4) with bf16 weights in
    the benchmark's launch configuration; all 64 tokens checked."""
    w = synth.WORKLOADS["bf16-decode"]
    say(f"full-size {w.name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.topk}")
    data = synth.make_all(w)
    res = run_layer(w, data)
    full_check(w, data, res, what=w.name)
