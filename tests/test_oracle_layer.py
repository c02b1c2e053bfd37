"""Pins of the oracle's expert layer (stage 1, stage 2, forward) against numpy
reimplementations that decode weights from the literal tables, closed forms and
invariances (no GPU)."""
import math

import numpy as np
import pytest
import torch

from quantized_mixture_experts_softmax_amd import synth

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def decode_weights(wfmt, w, s, N, K):
    """[E, N, K] fp64 from the literal e2m1 table / torch's e4m3 decode."""
    E = w.shape[0]
    if wfmt == synth.W_BF16:  # the bf16 number: its 16 bits are the top half of an fp32
        return (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if wfmt == synth.W_MXFP4:
        nib = np.stack([w & 15, w >> 4], axis=-1).reshape(E, N, K)
        scale = np.ldexp(1.0, s.astype(np.int64) - 127)
        return E2M1[nib] * np.repeat(scale, 32, axis=-1)
    vals = E4M3[w]
    if wfmt == synth.W_FP8_BLOCK128:
        sb = np.repeat(np.repeat(s.astype(np.float64), 128, axis=1)[:, :N], 128, axis=2)[:, :, :K]
        return vals * sb
    return vals * s.astype(np.float64)[:, :, None]


def bf16_round(a64):
    return torch.from_numpy(np.asarray(a64, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def quant_dequant(x64, afmt):
    """Reference activation quantisers: torch's e4m3 cast, brute-force e2m1."""
    if afmt == synth.A_BF16:
        return x64
    x32 = x64.astype(np.float32)
    out = np.empty_like(x64)
    if afmt in (synth.A_FP8_G128, synth.A_FP8_TOKEN):
        g = 128 if afmt == synth.A_FP8_G128 else x32.shape[-1]
        for c0 in range(0, x32.shape[-1], g):
            grp = x32[..., c0:c0 + g]
            amax = np.abs(grp).max(axis=-1, keepdims=True)
            s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
            q = np.clip((grp / s).astype(np.float32), -448, 448)
            codes = torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
            out[..., c0:c0 + g] = codes * s.astype(np.float64)
        return out
    grid = E2M1[:8]
    for c0 in range(0, x32.shape[-1], 32):
        grp = x64[..., c0:c0 + 32]
        amax = np.abs(grp).max(axis=-1)
        for idx in np.ndindex(amax.shape):
            es = -127 if amax[idx] == 0 else max(-127, math.frexp(amax[idx])[1] - 3)
            for i in range(32):
                v = grp[idx + (i,)] * 2.0 ** -es
                d = np.abs(grid - abs(v))
                best = [c for c in range(8) if d[c] == d.min()]
                if len(best) > 1:
                    best = [c for c in best if c % 2 == 0]
                out[idx + (c0 + i,)] = math.copysign(grid[best[0]], v) * 2.0 ** es
    return out


def numpy_forward(wl, data, ids, w):
    """Brute-force per token / per slot, fp64."""
    H, I = wl.H, wl.I
    W1 = decode_weights(wl.wfmt, data["w1"], data["w1_scale"], 2 * I, H)
    W2 = decode_weights(wl.wfmt, data["w2"], data["w2_scale"], H, I)
    x = synth.bf16_bits_to_f32(data["x"]).astype(np.float64)
    T, K = ids.shape
    out = np.zeros((T, H))
    for t in range(T):
        a = quant_dequant(x[t], wl.afmt)
        for j in range(K):
            e = ids[t, j]
            g = W1[e, :I] @ a
            u = W1[e, I:] @ a
            h = bf16_round(g / (1 + np.exp(-g)) * u)
            hq = quant_dequant(h, wl.afmt)
            out[t] += float(w[t, j]) * (W2[e] @ hq)
    return out


def layer_of(orc, wl, data):
    return orc.Layer(wl.H, wl.I, wl.E_total, wl.K, wl.wfmt, wl.afmt,
                     data["w1"], data["w1_scale"], data["w2"], data["w2_scale"])


def tiny(wfmt, afmt, T=4, H=64, I=32, E=4, k=2, n_shared=0, seed=7):
    return synth.Workload("t", T, H, I, E, k, wfmt, afmt, n_shared=n_shared, seed=seed)


FORMATS = [(synth.W_MXFP4, synth.A_BF16), (synth.W_MXFP4, synth.A_MXFP4_G32),
           (synth.W_FP8_BLOCK128, synth.A_FP8_G128), (synth.W_FP8_CHANNEL, synth.A_FP8_TOKEN),
           (synth.W_FP8_BLOCK128, synth.A_BF16), (synth.W_FP8_CHANNEL, synth.A_BF16), (synth.W_BF16, synth.A_BF16)]


@pytest.mark.parametrize("wfmt,afmt", FORMATS)
def test_forward_brute_force_fp64(orc, wfmt, afmt):
    wl = tiny(wfmt, afmt, H=160 if wfmt == synth.W_FP8_BLOCK128 else 64, I=160 if wfmt == synth.W_FP8_BLOCK128 else 32)
    data = synth.make_all(wl)
    ids, w = orc.route_topk(data["logits"], wl.topk)
    got = orc.forward(layer_of(orc, wl, data), data["x"], ids, w)
    ref = numpy_forward(wl, data, ids, w)
    rms = np.sqrt(np.mean(ref ** 2))
    # the two sides may round h to bf16 differently only in double-rounding corner cases
    assert np.max(np.abs(got - ref)) <= 1e-3 * rms


@pytest.mark.parametrize("wfmt", [synth.W_MXFP4, synth.W_FP8_BLOCK128, synth.W_FP8_CHANNEL, synth.W_BF16])
def test_top1_weight1_is_dense_gated_mlp(orc, wfmt):
    """With one routed slot of weight 1 the layer is W2 . (silu(Wg x) * (Wu x))."""
    wl = tiny(wfmt, synth.A_BF16, T=6, H=256, I=128, E=3, k=1)
    data = synth.make_all(wl)
    ids = np.array([[2], [0], [1], [2], [2], [0]], np.int32)
    w = np.ones((6, 1), np.float32)
    got = orc.forward(layer_of(orc, wl, data), data["x"], ids, w)
    W1 = decode_weights(wfmt, data["w1"], data["w1_scale"], 2 * wl.I, wl.H)
    W2 = decode_weights(wfmt, data["w2"], data["w2_scale"], wl.H, wl.I)
    X = synth.bf16_bits_to_f32(data["x"]).astype(np.float64)
    for t in range(6):
        e = ids[t, 0]
        gate = np.matmul(W1[e, :wl.I], X[t])
        up = np.matmul(W1[e, wl.I:], X[t])
        h = bf16_round(gate / (1.0 + np.exp(-gate)) * up)
        ref = np.matmul(W2[e], h)
        assert np.max(np.abs(got[t] - ref)) <= 1e-3 * np.sqrt(np.mean(ref ** 2))
    # gate/up order matters: swapping the halves of w1 changes the answer
    sw = dict(data)
    sw["w1"] = np.ascontiguousarray(np.concatenate([data["w1"][:, wl.I:], data["w1"][:, :wl.I]], axis=1))
    sw["w1_scale"] = np.ascontiguousarray(np.concatenate([data["w1_scale"][:, wl.I:], data["w1_scale"][:, :wl.I]], axis=1)) \
        if wfmt not in (synth.W_FP8_BLOCK128, synth.W_BF16) else data["w1_scale"]
    other = orc.forward(layer_of(orc, wl, sw), data["x"], ids, w)
    assert not np.allclose(other, got)


def test_closed_form_all_equal(orc):
    """Every w1 code 1.0 at scale 1, every w2 code 1.0 at scale 2^-1: gate = up =
    S = sum(x), h = bf16(silu(S) S), out_m = 0.5 * I * h for each token (k=1)."""
    H, I, E = 64, 32, 2
    x = synth.f32_to_bf16_bits(np.array([[0.5] * 32 + [-0.25] * 32, [0.125] * 64], np.float32))
    w1 = np.full((E, 2 * I, H // 2), 0x22, np.uint8)
    w1s = np.full((E, 2 * I, H // 32), 127, np.uint8)
    w2 = np.full((E, H, I // 2), 0x22, np.uint8)
    w2s = np.full((E, H, I // 32), 126, np.uint8)
    L = orc.Layer(H, I, E, 1, orc.W_MXFP4, orc.A_BF16, w1, w1s, w2, w2s)
    out = orc.forward(L, x, np.array([[1], [0]], np.int32), np.ones((2, 1), np.float32))
    for t, S in enumerate([8.0, 8.0]):
        h = float(bf16_round(np.array([S / (1 + math.exp(-S)) * S]))[0])
        assert np.all(out[t] == 0.5 * I * h)


def test_token_permutation_invariance(orc):
    wl = tiny(synth.W_MXFP4, synth.A_BF16, T=12, H=64, I=64, E=5, k=2)
    data = synth.make_all(wl)
    ids, w = orc.route_topk(data["logits"], 2)
    L = layer_of(orc, wl, data)
    out = orc.forward(L, data["x"], ids, w)
    p = np.random.default_rng(1).permutation(12)
    out_p = orc.forward(L, np.ascontiguousarray(data["x"][p]), np.ascontiguousarray(ids[p]), np.ascontiguousarray(w[p]))
    assert np.array_equal(out_p, out[p])


def test_expert_relabelling_invariance(orc):
    wl = tiny(synth.W_FP8_BLOCK128, synth.A_FP8_G128, T=6, H=128, I=128, E=4, k=2)
    data = synth.make_all(wl)
    ids, w = orc.route_topk(data["logits"], 2)
    out = orc.forward(layer_of(orc, wl, data), data["x"], ids, w)
    perm = np.array([2, 0, 3, 1])          # new id of old expert e is perm[e]
    inv = np.argsort(perm)
    d2 = {k: (np.ascontiguousarray(v[inv]) if k.startswith("w") else v) for k, v in data.items()}
    out2 = orc.forward(layer_of(orc, wl, d2), data["x"], np.ascontiguousarray(perm[ids]).astype(np.int32), w)
    assert np.array_equal(out, out2)


def test_w2_scale_plus_one_doubles_output(orc):
    wl = tiny(synth.W_MXFP4, synth.A_BF16, T=5, H=64, I=64, E=3, k=2)
    data = synth.make_all(wl)
    ids, w = orc.route_topk(data["logits"], 2)
    out = orc.forward(layer_of(orc, wl, data), data["x"], ids, w)
    d2 = dict(data)
    d2["w2_scale"] = (data["w2_scale"] + 1).astype(np.uint8)
    out2 = orc.forward(layer_of(orc, wl, d2), data["x"], ids, w)
    assert np.array_equal(out2, 2 * out)


def test_zero_weight_slot_contributes_nothing(orc):
    wl = tiny(synth.W_MXFP4, synth.A_BF16, T=5, H=64, I=64, E=3, k=2)
    data = synth.make_all(wl)
    ids, w = orc.route_topk(data["logits"], 2)
    w0 = w.copy()
    w0[:, 1] = 0
    L = layer_of(orc, wl, data)
    out = orc.forward(L, data["x"], ids, w0)
    L1 = orc.Layer(wl.H, wl.I, wl.E_total, 1, wl.wfmt, wl.afmt, data["w1"], data["w1_scale"], data["w2"], data["w2_scale"])
    out1 = orc.forward(L1, data["x"], np.ascontiguousarray(ids[:, :1]), np.ascontiguousarray(w0[:, :1]))
    assert np.array_equal(out, out1)


def test_stage_split_matches_forward_and_token_subset(orc):
    wl = tiny(synth.W_FP8_CHANNEL, synth.A_FP8_TOKEN, T=7, H=96, I=64, E=3, k=2)
    data = synth.make_all(wl)
    ids, w = orc.route_topk(data["logits"], 2)
    L = layer_of(orc, wl, data)
    out = orc.forward(L, data["x"], ids, w)
    sub = np.array([5, 1, 6], np.int32)
    h = orc.stage1(L, data["x"], ids, sub)
    out_sub = orc.stage2(L, h, ids, w, sub)
    assert np.array_equal(out_sub, out[sub])


def test_shared_expert_slot(orc):
    """A shared expert in slot k with weight 1 adds that expert's dense MLP output."""
    wl = tiny(synth.W_MXFP4, synth.A_BF16, T=4, H=64, I=32, E=4, k=2, n_shared=1)
    data = synth.make_all(wl)
    ids, w = orc.route_topk(data["logits"], 2, n_shared=1, shared_weight=1.0)
    assert np.all(ids[:, 2] == 4)
    L = layer_of(orc, wl, data)
    out = orc.forward(L, data["x"], ids, w)
    L2 = orc.Layer(wl.H, wl.I, wl.E_total, 2, wl.wfmt, wl.afmt, data["w1"], data["w1_scale"], data["w2"], data["w2_scale"])
    routed = orc.forward(L2, data["x"], np.ascontiguousarray(ids[:, :2]), np.ascontiguousarray(w[:, :2]))
    L1 = orc.Layer(wl.H, wl.I, wl.E_total, 1, wl.wfmt, wl.afmt, data["w1"], data["w1_scale"], data["w2"], data["w2_scale"])
    shared = orc.forward(L1, data["x"], np.full((4, 1), 4, np.int32), np.ones((4, 1), np.float32))
    assert np.array_equal(out, routed + shared)


@pytest.mark.parametrize("wfmt,afmt", [(synth.W_MXFP4, synth.A_BF16), (synth.W_FP8_CHANNEL, synth.A_FP8_TOKEN)])
def test_router_weight_on_input(orc, wfmt, afmt):
    """Router weight on the input (top-1): weight 1 is the ordinary layer bit for bit;
    weight w is W2 . act(w Wg a, w Wu a), unweighted -- written with numpy matmul on
    weights decoded from the literal tables -- and differs from w times the ordinary
    layer (the activation is not linear)."""
    wl = tiny(wfmt, afmt, T=6, H=256, I=128, E=3, k=1)
    data = synth.make_all(wl)
    ids = np.array([[2], [0], [1], [2], [2], [0]], np.int32)
    ones = np.ones((6, 1), np.float32)
    plain = layer_of(orc, wl, data)
    tk = orc.Layer(wl.H, wl.I, wl.E_total, 1, wfmt, afmt, data["w1"], data["w1_scale"], data["w2"], data["w2_scale"],
                   weight_on_input=True)
    assert np.array_equal(orc.forward(tk, data["x"], ids, ones), orc.forward(plain, data["x"], ids, ones))
    wt = np.array([[0.25], [0.8], [1.5], [0.5], [0.125], [1.0]], np.float32)
    got = orc.forward(tk, data["x"], ids, wt)
    W1 = decode_weights(wfmt, data["w1"], data["w1_scale"], 2 * wl.I, wl.H)
    W2 = decode_weights(wfmt, data["w2"], data["w2_scale"], wl.H, wl.I)
    X = synth.bf16_bits_to_f32(data["x"]).astype(np.float64)
    for t in range(6):
        e, w = ids[t, 0], float(wt[t, 0])
        a = quant_dequant(X[t], afmt)
        gate = w * np.matmul(W1[e, :wl.I], a)
        up = w * np.matmul(W1[e, wl.I:], a)
        h = quant_dequant(bf16_round(gate / (1.0 + np.exp(-gate)) * up), afmt)
        ref = np.matmul(W2[e], h)
        assert np.max(np.abs(got[t] - ref)) <= 1e-3 * np.sqrt(np.mean(ref ** 2))
    weighted_out = orc.forward(plain, data["x"], ids, wt)
    assert not np.allclose(got, weighted_out, rtol=1e-3)


def test_bf16_weights_scale_linearly(orc):
    """Unquantised weights: doubling every w2 value (adding one to each bf16 exponent)
    doubles the output exactly, and negating w1's up half negates it (silu(g) * (-u))."""
    wl = tiny(synth.W_BF16, synth.A_BF16, T=5, H=64, I=32, E=3, k=2)
    data = synth.make_all(wl)
    ids, w = orc.route_topk(data["logits"], wl.topk)
    L = layer_of(orc, wl, data)
    base = orc.forward(L, data["x"], ids, w)
    w2 = data["w2"].copy()
    nz = (w2 & 0x7F80) != 0
    w2[nz] = w2[nz] + np.uint16(0x80)  # exponent + 1 (no value here is near overflow)
    dbl = orc.forward(orc.Layer(wl.H, wl.I, wl.E_total, wl.K, wl.wfmt, wl.afmt, data["w1"], None, w2, None),
                      data["x"], ids, w)
    assert np.array_equal(dbl, 2.0 * base)
    w1 = data["w1"].copy()
    w1[:, wl.I:] ^= np.uint16(0x8000)
    neg = orc.forward(orc.Layer(wl.H, wl.I, wl.E_total, wl.K, wl.wfmt, wl.afmt, w1, None, data["w2"], None),
                      data["x"], ids, w)
    assert np.array_equal(neg, -base)
