"""Pins of the oracle's per-tensor FP8 formats (one weight scale per expert and
projection, one dynamic activation scale per tensor; no GPU)."""
import numpy as np
import pytest
import torch

from quantized_mixture_experts_softmax_amd import synth


def test_tensor_quant_is_row_rule_on_flattened_tensor(orc):
    rng = np.random.default_rng(8)
    x = synth.f32_to_bf16_bits((rng.standard_normal((37, 160)) * np.linspace(0.1, 5, 160)).astype(np.float32))
    c, s = orc.quant_act(x, orc.A_FP8_TENSOR)
    c1, s1 = orc.quant_act(np.ascontiguousarray(x.reshape(1, -1)), orc.A_FP8_TOKEN)
    assert np.array_equal(c.reshape(-1), c1.reshape(-1)) and s[0] == s1[0]
    z, sz = orc.quant_act(np.zeros((3, 64), np.uint16), orc.A_FP8_TENSOR)
    assert sz[0] == 1.0 and not z.any()


def layer(orc, w, d, wfmt=None, afmt=None, w1s=None, w2s=None):
    return orc.Layer(w.H, w.I, w.E_total, w.K, wfmt if wfmt is not None else w.wfmt,
                     afmt if afmt is not None else w.afmt, d["w1"], d["w1_scale"] if w1s is None else w1s,
                     d["w2"], d["w2_scale"] if w2s is None else w2s)


def test_tensor_weights_are_broadcast_channel_weights(orc):
    w = synth.Workload("t", 5, 128, 96, 4, 2, synth.W_FP8_TENSOR, synth.A_FP8_TOKEN, seed=12)
    d = synth.make_all(w)
    ids, wt = orc.route_topk(d["logits"], 2)
    per_t = orc.forward(layer(orc, w, d), d["x"], ids, wt)
    b1 = np.ascontiguousarray(np.repeat(d["w1_scale"][:, None], 2 * w.I, axis=1))
    b2 = np.ascontiguousarray(np.repeat(d["w2_scale"][:, None], w.H, axis=1))
    per_c = orc.forward(layer(orc, w, d, wfmt=synth.W_FP8_CHANNEL, w1s=b1, w2s=b2), d["x"], ids, wt)
    assert np.array_equal(per_t, per_c)


def test_one_token_one_slot_tensor_is_token(orc):
    w = synth.Workload("t", 1, 128, 96, 4, 1, synth.W_FP8_TENSOR, synth.A_FP8_TENSOR, seed=13)
    d = synth.make_all(w)
    ids, wt = orc.route_topk(d["logits"], 1)
    a = orc.forward(layer(orc, w, d), d["x"], ids, wt)
    b = orc.forward(layer(orc, w, d, afmt=synth.A_FP8_TOKEN), d["x"], ids, wt)
    assert np.array_equal(a, b)


E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def qdq_tensor(v64):
    """Per-tensor FP8 with torch's e4m3 cast: s = amax / 448 in fp32, codes = RNE(v / s)."""
    v32 = v64.astype(np.float32)
    amax = np.float32(np.abs(v32).max())
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    q = torch.from_numpy(v32 / s).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return q * np.float64(s)


def test_tensor_layer_brute_force(orc):
    w = synth.Workload("t", 6, 128, 96, 4, 2, synth.W_FP8_TENSOR, synth.A_FP8_TENSOR, seed=14)
    d = synth.make_all(w)
    ids, wt = orc.route_topk(d["logits"], 2)
    got = orc.forward(layer(orc, w, d), d["x"], ids, wt)
    W1 = E4M3[d["w1"]] * d["w1_scale"].astype(np.float64)[:, None, None]
    W2 = E4M3[d["w2"]] * d["w2_scale"].astype(np.float64)[:, None, None]
    X = synth.bf16_bits_to_f32(d["x"]).astype(np.float64)
    A = qdq_tensor(X)
    hs = np.zeros((w.T, w.K, w.I))
    for t in range(w.T):
        for j in range(w.K):
            e = ids[t, j]
            g, u = W1[e, :w.I] @ A[t], W1[e, w.I:] @ A[t]
            hs[t, j] = torch.from_numpy(g / (1 + np.exp(-g)) * u).to(torch.bfloat16).to(torch.float64).numpy()
    H2 = qdq_tensor(hs.reshape(-1, w.I)).reshape(w.T, w.K, w.I)
    ref = np.zeros((w.T, w.H))
    for t in range(w.T):
        for j in range(w.K):
            ref[t] += float(wt[t, j]) * (W2[ids[t, j]] @ H2[t, j])
    assert np.max(np.abs(got - ref)) <= 1e-3 * np.sqrt(np.mean(ref ** 2))
    with pytest.raises(ValueError):
        orc.forward(layer(orc, w, d), d["x"], ids, wt, tokens=[0, 1])  # per-tensor needs the whole batch
