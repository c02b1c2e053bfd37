"""Pins of the oracle's grouped top-k router (score-correction bias, expert groups,
routed scaling factor; no GPU)."""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_grouped_router_golden(orc):
    with open(os.path.join(GOLDEN, "grouped_router_examples.txt")) as f:
        lines = [l.strip() for l in f if l.strip() and not l.startswith("#")]
    assert len(lines) >= 4
    for line in lines:
        head, lg, bias, ids, ws = [p.split() for p in line.split("|")]
        score = orc.SCORE_SOFTMAX if head[0] == "softmax" else orc.SCORE_SIGMOID
        k, G, TG, scaling, renorm = int(head[1]), int(head[2]), int(head[3]), float(head[4]), bool(int(head[5]))
        logits = np.array([[float(v) for v in lg]], np.float32)
        b = None if bias == ["-"] else np.array([float(v) for v in bias], np.float32)
        got_ids, got_w = orc.route_grouped_topk(logits, k, G, TG, b, score, renorm, scaling)
        assert got_ids[0].tolist() == [int(i) for i in ids], line
        np.testing.assert_allclose(got_w[0], [float(w) for w in ws], rtol=2e-7, err_msg=line)


@pytest.mark.parametrize("score", [0, 1])
@pytest.mark.parametrize("renorm", [True, False])
def test_grouped_router_one_group_is_plain_topk(orc, score, renorm):
    """One group, no bias, scaling 1: the plain top-k router (itself pinned by brute force)."""
    logits = np.random.default_rng(11).standard_normal((300, 64)).astype(np.float32)
    logits[:30] = np.round(logits[:30] * 2) / 2  # exact ties
    ids, w = orc.route_grouped_topk(logits, 6, 1, 1, None, score, renorm, 1.0)
    ids0, w0 = orc.route_topk(logits, 6, score, renorm)
    assert np.array_equal(ids, ids0)
    np.testing.assert_allclose(w, w0, rtol=3e-7)


def _reference(logits, bias, k, G, TG, score, renorm, scaling):
    """The same reading written with numpy sorts: group scores from np.sort, group and
    expert choice from np.lexsort on (-value, id)."""
    T, E = logits.shape
    gs = E / G
    l64 = logits.astype(np.float64)
    if score == 1:
        s = 1 / (1 + np.exp(-l64))
    else:
        z = np.exp(l64 - l64.max(axis=1, keepdims=True))
        s = z / z.sum(axis=1, keepdims=True)
    key = s + bias.astype(np.float64)[None, :] if bias is not None else l64
    ids = np.zeros((T, k), np.int64)
    w = np.zeros((T, k), np.float64)
    for t in range(T):
        kg = key[t].reshape(G, int(gs))
        srt = -np.sort(-kg, axis=1)
        gsc = srt[:, :2].sum(axis=1) if (bias is not None and gs > 1) else srt[:, 0]
        gorder = np.lexsort((np.arange(G), -gsc))[:TG]
        allowed = np.isin(np.arange(E) // int(gs), gorder)
        cand = np.flatnonzero(allowed)
        order = cand[np.lexsort((cand, -key[t, cand]))][:k]
        ids[t] = order
        sel = s[t, order]
        w[t] = (sel / sel.sum() if renorm else sel) * scaling
    return ids, w


@pytest.mark.parametrize("E,k,G,TG,score,use_bias,renorm,scaling", [
    (256, 8, 8, 4, 1, True, True, 2.5),     # DeepSeek-V3 shape
    (64, 6, 8, 3, 0, False, True, 1.0),     # V2-style: softmax, no bias
    (32, 4, 4, 2, 1, True, False, 1.5),
    (16, 3, 16, 3, 0, True, True, 1.0),     # one expert per group
    (48, 5, 6, 6, 1, False, True, 1.0),     # every group kept
])
def test_grouped_router_vs_numpy_sorts(orc, E, k, G, TG, score, use_bias, renorm, scaling):
    rng = np.random.default_rng(E + k + G)
    logits = rng.standard_normal((200, E)).astype(np.float32)
    logits[:20] = np.round(logits[:20] * 2) / 2  # exact logit ties
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32) if use_bias else None
    if bias is not None:
        bias[: E // 2] = np.round(bias[: E // 2] * 4) / 4
    ids, w = orc.route_grouped_topk(logits, k, G, TG, bias, score, renorm, scaling)
    rid, rw = _reference(logits, bias, k, G, TG, score, renorm, scaling)
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(w, rw, rtol=3e-7)
    gs = E // G
    for t in range(logits.shape[0]):
        assert len(set((ids[t] // gs).tolist())) <= TG  # slots come from at most topk_group groups
    if renorm:
        np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), scaling, rtol=1e-6)


def test_grouped_router_bias_moves_ids_not_weights(orc):
    """Weights are the unbiased scores of whatever is chosen; a uniform shift of all
    biases (a power of two, exact here) chooses the same experts."""
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((100, 32)).astype(np.float32)
    bias = (rng.standard_normal(32) * 0.05).astype(np.float32)
    ids, w = orc.route_grouped_topk(logits, 4, 4, 2, bias, 1, False, 1.0)
    s = 1 / (1 + np.exp(-logits.astype(np.float64)))
    np.testing.assert_allclose(w, np.take_along_axis(s, ids, axis=1), rtol=3e-7)
    ids2, _ = orc.route_grouped_topk(logits, 4, 4, 2, bias + np.float32(0.5), 1, False, 1.0)
    assert np.array_equal(ids, ids2)


def test_grouped_router_shared_slots_and_rejects(orc):
    logits = np.random.default_rng(6).standard_normal((10, 16)).astype(np.float32)
    ids, w = orc.route_grouped_topk(logits, 2, 4, 2, None, 1, True, 1.0, n_shared=1, shared_weight=1.0)
    assert np.all(ids[:, 2] == 16) and np.all(w[:, 2] == 1.0)
    with pytest.raises(ValueError):
        orc.route_grouped_topk(logits, 2, 5, 2)      # 16 experts do not split into 5 groups
    with pytest.raises(ValueError):
        orc.route_grouped_topk(logits, 9, 4, 2)      # 9 slots > 2 groups x 4 experts
