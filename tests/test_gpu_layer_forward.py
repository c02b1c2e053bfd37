"""moe_layer_forward (router + align-sort + expert layer in one call; small batches are
routed and sorted inside the stage-1 kernel) against the separate calls
(moe_route_align, then moe_experts_forward) on the same inputs: the routing tables,
the stage-1 h and the output are equal bit for bit (both paths run the same GEMM
kernels on the same sorted rows), and the result meets the oracle bound.
"""
import numpy as np
import pytest
import torch

from gpu_common import B, bf16_dev, bf16_host, dev_weights, run_layer, say, synth, to_dev
from test_gpu_forward import FP8C, W4A16, W4A4, full_check, oai_case, small

pytestmark = pytest.mark.gpu

SORT_KEYS = ("expert_counts", "expert_offsets", "sorted_slots", "block_expert", "num_padded")


def both_paths(w, data, tiled=False, act=None, block_m=16):
    """Runs the fused entry point and the separate calls; returns both results."""
    wd = dev_weights(data)
    fused = run_layer(w, data, block_m=block_m, wd=wd, tiled=tiled, act=act)
    f_layer = fused["layer"]
    sep_layer = B.MoELayer(wd["w1"], wd["w1_scale"], wd["w2"], wd["w2_scale"], H=w.H, I=w.I, E=w.E, topk=w.topk,
                           wfmt=w.wfmt, afmt=w.afmt, score=f_layer.score, n_shared=w.n_shared,
                           shared_weight=w.shared_weight, block_m=block_m, tiled=tiled, act=f_layer.act,
                           fuse_route=False)
    sep = run_layer_with(sep_layer, w, data)
    return fused, sep


def run_layer_with(layer, w, data):
    """Runs `layer` on the data; host copies of the routing tables, h and the output."""
    x = bf16_dev(data["x"])
    out = layer(x, to_dev(data["logits"]))
    torch.cuda.synchronize()
    b = layer._bufs[(x.shape[0], str(x.device))]
    res = dict(out=bf16_host(out), ids=b["ids"].cpu().numpy(), weights=b["w"].cpu().numpy(),
               sort={k: v.cpu().numpy() for k, v in b["sort"].items()})
    if b["workspace"] is not None:
        args = B.forward_args(x, layer.w1, layer.w1_scale, layer.w2, layer.w2_scale, b["ids"], b["w"], b["sort"],
                              w.wfmt, w.afmt, b["bm"], w.E_total, w.I, out, b["workspace"],
                              *(b["a1"] if b["a1"] else (None, None)), weight_layout=layer.weight_layout)
        L = B.moe_workspace_layout(args)
        cap = B.moe_sort_capacity(x.shape[0], w.K, w.E_total, b["bm"])
        ws = b["workspace"]
        res["h_sorted"] = ws[L["h_off"]:L["h_off"] + L["h_bytes"]].cpu().numpy().view(np.uint16).reshape(cap, w.I)
    return res


def assert_same(fused, sep, what):
    assert np.array_equal(fused["ids"], sep["ids"]), f"{what}: topk_ids"
    assert np.array_equal(fused["weights"].view(np.uint32), sep["weights"].view(np.uint32)), f"{what}: weights"
    for k in SORT_KEYS:
        assert np.array_equal(fused["sort"][k], sep["sort"][k]), f"{what}: {k}"
    npad = int(sep["sort"]["num_padded"][0])
    if "h_sorted" in sep:
        assert np.array_equal(fused["h_sorted"][:npad], sep["h_sorted"][:npad]), f"{what}: stage-1 h"
    assert np.array_equal(fused["out"], sep["out"]), f"{what}: output"
    say(f"{what}: fused and separate routing agree bit for bit ({npad} padded rows)")


CASES = [
    # name, workload ctor, tiled, oracle check
    ("tiny-ragged", lambda: small(W4A16, T=37, H=256, I=256, E=8, k=2, seed=21), False, True),
    ("single-token", lambda: small(W4A16, T=1, H=256, I=288, E=8, k=2, seed=22), True, True),
    ("shared-sigmoid", lambda: small(W4A16, T=50, H=320, I=288, E=12, k=3, n_shared=2,
                                     score=synth.SCORE_SIGMOID, seed=23), False, True),
    ("w4a4", lambda: small(W4A4, T=40, H=320, I=288, E=6, k=2, seed=24), True, True),
    ("fp8-channel", lambda: small(FP8C, T=16, H=512, I=384, E=8, k=2, seed=25), True, True),
    ("e64-max-batch", lambda: small(W4A16, T=128, H=256, I=256, E=64, k=32, seed=26), False, False),
    ("t-max", lambda: small(W4A16, T=1024, H=256, I=128, E=8, k=4, seed=27), True, False),
    ("bf16-weights", lambda: small((synth.W_BF16, synth.A_BF16), T=45, H=320, I=288, E=8, k=2, seed=33), False, True),
]


@pytest.mark.parametrize("name,make,tiled,with_oracle", CASES, ids=[c[0] for c in CASES])
def test_layer_forward_equals_separate_calls(name, make, tiled, with_oracle):
    w = make()
    say(f"layer_forward {name}: T={w.T} H={w.H} I={w.I} E={w.E}+{w.n_shared} k={w.topk} tiled={tiled}")
    data = synth.make_all(w)
    fused, sep = both_paths(w, data, tiled=tiled)
    assert_same(fused, sep, name)
    if with_oracle:
        full_check(w, data, fused, what=f"{name} fused")


def test_layer_forward_decode_full_size():
    """The decode workload (T=64, H=I=2880, 32 experts, top-4, MXFP4 w4a16, tiled
    weights) in the benchmark's launch configuration: the routed stage 1 equals the
    separate calls bit for bit and meets the oracle bound on all 64 tokens."""
    w = synth.WORKLOADS["decode"]
    data = synth.make_all(w)
    fused, sep = both_paths(w, data, tiled=True)
    assert_same(fused, sep, "decode")
    full_check(w, data, fused, what="decode fused")


@pytest.fixture(scope="module")
def decode_data():
    w = synth.WORKLOADS["decode"]
    return w, synth.make_all(w)


@pytest.mark.parametrize("T", [1, 2, 7, 33, 63])
def test_layer_forward_decode_token_sweep(decode_data, T):
    """The decode layer's weights at fewer tokens (prefixes of the 64-token draw): with 1..63
    tokens over 32 experts some experts get no rows and the workgroups' shares of the
    (unit, K chunk) steps change; the routed stage 1 still equals the separate calls bit
    for bit and meets the oracle bound on every token."""
    w0, d0 = decode_data
    w = w0.with_T(T)
    data = dict(d0, x=np.ascontiguousarray(d0["x"][:T]), logits=np.ascontiguousarray(d0["logits"][:T]))
    say(f"layer_forward decode T={T}")
    fused, sep = both_paths(w, data, tiled=True)
    assert_same(fused, sep, f"decode T={T}")
    full_check(w, data, fused, what=f"decode T={T} fused")


def test_layer_forward_tied_logits():
    """Router logits with many equal values (signed zeros included) on the decode-sized
    expert count: the in-kernel routing breaks ties as the separate router does."""
    w = small(W4A16, T=64, H=256, I=256, E=32, k=4, seed=32)
    data = synth.make_all(w)
    lg = (np.round(data["logits"] * 2) / 2).astype(np.float32)
    lg[::4, :8] = -0.0
    fused, sep = both_paths(w, dict(data, logits=lg), tiled=True)
    assert_same(fused, sep, "ties")
    full_check(w, dict(data, logits=lg), fused, what="ties fused")


def test_layer_forward_oai_bias():
    w = small(W4A16, T=45, H=320, I=288, E=8, k=2, seed=28)
    data = synth.make_all(w)
    act, data = oai_case(w, data, True, True)
    fused, sep = both_paths(w, data, tiled=True, act=act)
    assert_same(fused, sep, "oai")
    full_check(w, data, fused, what="oai fused", act=act)


@pytest.mark.parametrize("bm", [32, 64])
def test_layer_forward_unfused_block_m(bm):
    """Blocks of more than 16 rows take the separate launches inside moe_layer_forward."""
    w = small(W4A16, T=40, H=320, I=288, E=6, k=2, seed=29)
    data = synth.make_all(w)
    fused, sep = both_paths(w, data, block_m=bm)
    assert_same(fused, sep, f"bm{bm}")


def test_layer_forward_large_E_unfused():
    """E > 64 routed experts: moe_layer_forward falls back to the separate launches."""
    w = small(W4A16, T=20, H=256, I=256, E=96, k=4, n_shared=1, seed=30)
    data = synth.make_all(w)
    fused, sep = both_paths(w, data)
    assert_same(fused, sep, "E96")


def test_layer_forward_reuse_smaller_batch():
    """Two calls in a row on one layer, the second with fewer tokens (stale tables from
    the first call must not leak into the second)."""
    w = small(W4A16, T=64, H=256, I=256, E=16, k=4, seed=31)
    data = synth.make_all(w)
    r1 = run_layer(w, data, block_m=16)
    w2 = w.scaled(T=9)
    d2 = dict(data, x=np.ascontiguousarray(data["x"][:9]), logits=np.ascontiguousarray(data["logits"][:9]))
    layer = r1["layer"]
    wd = dev_weights(data)
    sep_layer = B.MoELayer(wd["w1"], wd["w1_scale"], wd["w2"], wd["w2_scale"], H=w.H, I=w.I, E=w.E, topk=w.topk,
                           wfmt=w.wfmt, afmt=w.afmt, block_m=16, fuse_route=False)
    fused2 = run_layer_with(layer, w2, d2)
    sep2 = run_layer_with(sep_layer, w2, d2)
    assert_same(fused2, sep2, "second call T=9")


def test_outputs_are_not_aliased():
    """Two calls with the same token count return distinct tensors: the second call does
    not overwrite the first call's result."""
    w = synth.WORKLOADS["tiny"]
    data = synth.make_all(w)
    wd = dev_weights(data)
    layer = B.MoELayer(wd["w1"], wd["w1_scale"], wd["w2"], wd["w2_scale"], H=w.H, I=w.I, E=w.E, topk=w.topk,
                       wfmt=w.wfmt, afmt=w.afmt)
    x1 = bf16_dev(data["x"])
    x2 = bf16_dev(np.ascontiguousarray(data["x"][::-1]))
    l1 = to_dev(data["logits"])
    l2 = to_dev(np.ascontiguousarray(data["logits"][::-1]))
    y1 = layer(x1, l1)
    first = bf16_host(y1).copy()
    y2 = layer(x2, l2)
    torch.cuda.synchronize()
    assert y1.data_ptr() != y2.data_ptr()
    assert np.array_equal(bf16_host(y1), first)
    # per-row arithmetic does not depend on the other rows: reversed tokens, reversed rows
    assert np.array_equal(bf16_host(y2), first[::-1])
