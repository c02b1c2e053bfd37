"""Pins of the oracle's expert-parallel share (expert map and valid-token count; no GPU):
the map is numpy indexing, and the shares of a partition of the experts add up to the
whole layer."""
import numpy as np
import pytest

from quantized_mixture_experts_softmax_amd import synth


def test_map_experts_is_indexing(orc):
    rng = np.random.default_rng(3)
    ids = rng.integers(-1, 40, (50, 4)).astype(np.int32)  # includes -1 and ids past E
    emap = np.full(32, -1, np.int32)
    emap[8:16] = np.arange(8)
    got = orc.map_experts(ids, emap, 32, num_local_tokens=41)
    valid = (ids >= 0) & (ids < 32) & (np.arange(50)[:, None] < 41)
    want = np.where(valid, emap[np.clip(ids, 0, 31)], -1)
    assert np.array_equal(got, want)
    assert np.array_equal(orc.map_experts(ids, None, 32), np.where((ids >= 0) & (ids < 32), ids, -1))


@pytest.mark.parametrize("wfmt,afmt", [(synth.W_MXFP4, synth.A_BF16), (synth.W_FP8_BLOCK128, synth.A_FP8_G128),
                                       (synth.W_FP8_CHANNEL, synth.A_FP8_TOKEN)])
def test_shares_add_up_to_the_layer(orc, wfmt, afmt):
    """Experts split over 3 devices (uneven, shared expert replicated in one share): the
    partial outputs, each computed from that device's local weights and local ids, sum to
    the full output."""
    w = synth.Workload("t", 9, 128, 128, 7, 3, wfmt, afmt, n_shared=1, seed=31)
    d = synth.make_all(w)
    ids, wt = orc.route_topk(d["logits"], w.topk, n_shared=1, shared_weight=1.0)
    full = orc.forward(orc.Layer(w.H, w.I, w.E_total, w.K, wfmt, afmt, d["w1"], d["w1_scale"], d["w2"],
                                 d["w2_scale"]), d["x"], ids, wt)
    shares = [[0, 1, 2], [3, 4], [5, 6, 7]]  # expert 7 is the shared one
    total = np.zeros_like(full)
    for mine in shares:
        emap = np.full(w.E_total, -1, np.int32)
        emap[mine] = np.arange(len(mine))
        loc = orc.map_experts(ids, emap, w.E_total)
        pick = lambda a: np.ascontiguousarray(a[mine])
        ws1 = pick(d["w1_scale"])
        ws2 = pick(d["w2_scale"])
        L = orc.Layer(w.H, w.I, len(mine), w.K, wfmt, afmt, pick(d["w1"]), ws1, pick(d["w2"]), ws2)
        total += orc.forward(L, d["x"], loc, wt)
    np.testing.assert_allclose(total, full, rtol=1e-12, atol=1e-12 * np.abs(full).max())


def test_rows_past_num_local_tokens_are_zero(orc):
    w = synth.Workload("t", 6, 64, 64, 4, 2, synth.W_MXFP4, synth.A_BF16, seed=5)
    d = synth.make_all(w)
    ids, wt = orc.route_topk(d["logits"], 2)
    loc = orc.map_experts(ids, None, 4, num_local_tokens=4)
    L = orc.Layer(w.H, w.I, 4, 2, w.wfmt, w.afmt, d["w1"], d["w1_scale"], d["w2"], d["w2_scale"])
    out = orc.forward(L, d["x"], loc, wt)
    assert np.all(out[4:] == 0.0)
    assert np.array_equal(out[:4], orc.forward(L, d["x"], ids, wt)[:4])
