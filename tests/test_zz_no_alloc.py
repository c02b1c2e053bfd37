"""moe_experts_forward_noalloc (the entry point for callers that cannot allocate) against
moe_experts_forward with a caller workspace: the same inputs give the same output bit for
bit, on two calls in a row with the second batch smaller than the first, for bf16 (w4a16)
and quantised (w4a4, a1 quantised inside the call) activations."""
import numpy as np
import pytest
import torch

from gpu_common import B, bf16_dev, bf16_host, dev_weights, say, synth, to_dev

pytestmark = pytest.mark.gpu


def _route(logits, w, bm):
    ids, wts, srt = B.moe_route_align(logits, w.topk, bm, "softmax" if w.score == synth.SCORE_SOFTMAX else "sigmoid",
                                      True, w.n_shared, w.shared_weight)
    return ids, wts, srt


CASES = [
    ("decode-w4a16", synth.WORKLOADS["decode"], 16, True, (64, 17)),
    ("small-w4a4-bm64", synth.Workload("na4", 48, 320, 288, 6, 2, synth.W_MXFP4, synth.A_MXFP4_G32, seed=91), 64,
     False, (48, 9)),
    ("small-fp8b-bm32", synth.Workload("na8", 40, 352, 288, 5, 3, synth.W_FP8_BLOCK128, synth.A_FP8_G128,
                                       score=synth.SCORE_SIGMOID, n_shared=1, seed=92), 32, True, (40, 7)),
]


@pytest.mark.parametrize("name,w,bm,tiled,Ts", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry(name, w, bm, tiled, Ts):
    data = synth.make_all(w)
    wd = dev_weights(data)
    layout = B.LAYOUT_TILED if tiled else B.LAYOUT_CANONICAL
    if tiled:
        w1 = B.moe_tile_weights(wd["w1"], wd["w1_scale"], w.wfmt, w.H)
        w2 = B.moe_tile_weights(wd["w2"], wd["w2_scale"], w.wfmt, w.I)
        w1s, w2s = (None, None) if w.wfmt == synth.W_MXFP4 else (wd["w1_scale"], wd["w2_scale"])
    else:
        w1, w1s, w2, w2s = wd["w1"], wd["w1_scale"], wd["w2"], wd["w2_scale"]
    for T in Ts:  # the second call is smaller than the first
        say(f"noalloc {name}: T={T} bm={bm} tiled={tiled}")
        x = bf16_dev(data["x"][:T])
        logits = to_dev(np.ascontiguousarray(data["logits"][:T]))
        ids, wts, srt = _route(logits, w, bm)
        ref, ws = B.moe_experts_forward(x, w1, w1s, w2, w2s, ids, wts, srt, w.wfmt, w.afmt, bm, w.E_total, w.I,
                                        weight_layout=layout)
        need = ws.numel()
        assert need <= B.NOALLOC_SCRATCH_BYTES
        got = B.moe_experts_forward_noalloc(x, w1, w1s, w2, w2s, ids, wts, srt, w.wfmt, w.afmt, bm, w.E_total, w.I,
                                            weight_layout=layout)
        torch.cuda.synchronize()
        r, g = bf16_host(ref), bf16_host(got)
        assert r.shape == (T, w.H) and np.isfinite(synth.bf16_bits_to_f32(g)).all()
        diff = int(np.count_nonzero(r != g))
        say(f"noalloc {name}: T={T}: {diff} of {r.size} outputs differ (workspace {need} bytes)")
        assert diff == 0, f"{name} T={T}: noalloc output differs from moe_experts_forward"
