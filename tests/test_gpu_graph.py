"""Every ABI call only enqueues work on the caller's stream, so a whole layer call can be
captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.  Each replay runs with
eager calls on other inputs in between (they overwrite the layer's tables, workspace and
output) and must reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

from gpu_common import B, bf16_dev, bf16_host, dev_weights, say, synth, to_dev
from test_gpu_forward import W4A4, FP8T, small

pytestmark = pytest.mark.gpu

CASES = [
    # name, workload ctor, block_m, tiled
    ("decode-fused-route", lambda: synth.WORKLOADS["decode"], None, True),
    ("w4a4-bm64", lambda: small(W4A4, T=40, H=320, I=288, E=6, k=2, seed=71), 64, True),
    ("fp8-tensor-bm64", lambda: small(FP8T, T=33, H=320, I=416, E=4, k=2, seed=72), 64, False),
]


@pytest.mark.parametrize("name,make,bm,tiled", CASES, ids=[c[0] for c in CASES])
def test_layer_graph_replay(name, make, bm, tiled):
    w = make()
    data = synth.make_all(w)
    wd = dev_weights(data)
    layer = B.MoELayer(wd["w1"], wd["w1_scale"], wd["w2"], wd["w2_scale"], H=w.H, I=w.I, E=w.E, topk=w.topk,
                       wfmt=w.wfmt, afmt=w.afmt, n_shared=w.n_shared, shared_weight=w.shared_weight,
                       block_m=bm, tiled=tiled)
    x, lg = bf16_dev(data["x"]), to_dev(data["logits"])
    rng = np.random.default_rng(7)
    x2 = bf16_dev(synth.f32_to_bf16_bits(rng.standard_normal((w.T, w.H)).astype(np.float32)))
    lg2 = to_dev(rng.standard_normal((w.T, w.E)).astype(np.float32))

    want = bf16_host(layer(x, lg))  # eager; also allocates the layer's buffers
    other = bf16_host(layer(x2, lg2))
    torch.cuda.synchronize()
    assert not np.array_equal(want, other)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer(x, lg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer(x, lg)
    for i in range(3):
        layer(x2, lg2)  # eager work on other inputs between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = bf16_host(out)
        assert np.array_equal(got, want), f"{name}: replay {i} differs from the eager result"
    say(f"graph {name}: 3 replays equal the eager result bit for bit")
