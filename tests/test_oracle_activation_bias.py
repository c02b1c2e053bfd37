"""Pins of the oracle's SwiGLU-OAI activation, projection biases and interleaved
gate/up rows (no GPU): reduction to the SiLU layer, row-permutation equivalence,
bias additivity, and the clamp's invariances."""
import numpy as np
import pytest

from quantized_mixture_experts_softmax_amd import synth


def small(wfmt=synth.W_MXFP4, afmt=synth.A_BF16, T=6, H=64, I=64, E=3, k=2, seed=21):
    w = synth.Workload("t", T, H, I, E, k, wfmt, afmt, seed=seed)
    return w, synth.make_all(w)


def layer(orc, w, d, **kw):
    return orc.Layer(w.H, w.I, w.E_total, w.K, w.wfmt, w.afmt, d["w1"], d["w1_scale"], d["w2"], d["w2_scale"], **kw)


FMTS = [(synth.W_MXFP4, synth.A_BF16), (synth.W_MXFP4, synth.A_MXFP4_G32),
        (synth.W_FP8_BLOCK128, synth.A_FP8_G128), (synth.W_FP8_CHANNEL, synth.A_FP8_TOKEN)]


@pytest.mark.parametrize("wfmt,afmt", FMTS)
def test_swiglu_oai_alpha1_beta0_nolimit_is_silu(orc, wfmt, afmt):
    w, d = small(wfmt, afmt, H=128, I=128)
    ids, wt = orc.route_topk(d["logits"], w.K)
    silu = orc.forward(layer(orc, w, d), d["x"], ids, wt)
    oai = orc.forward(layer(orc, w, d, act=orc.ACT_SWIGLU_OAI, alpha=1.0, beta=0.0, limit=0.0), d["x"], ids, wt)
    assert np.array_equal(silu, oai)


# FP8 128x128 block scales cover 128 consecutive rows, which interleaving would mix;
# interleaved rows are used with MXFP4 (per-row scales) and per-channel FP8.
FMTS_ITL = [f for f in FMTS if f[0] != synth.W_FP8_BLOCK128]


@pytest.mark.parametrize("wfmt,afmt", FMTS_ITL)
@pytest.mark.parametrize("act", [0, 1])
def test_interleaved_rows_equal_separated(orc, wfmt, afmt, act):
    """Interleaving w13's gate and up rows (codes, scales and biases alike) and saying
    so gives the same layer bit for bit."""
    w, d = small(wfmt, afmt, H=128, I=256)
    ids, wt = orc.route_topk(d["logits"], w.K)
    b1, b2 = synth.make_biases(w)
    sep = layer(orc, w, d, act=act, w1_bias=b1, w2_bias=b2)
    w1i = synth.interleave_rows(d["w1"], w.I)
    w1si = synth.interleave_rows(d["w1_scale"], w.I)
    itl = orc.Layer(w.H, w.I, w.E_total, w.K, w.wfmt, w.afmt, w1i, w1si, d["w2"], d["w2_scale"], act=act,
                    gate_up_interleaved=True, w1_bias=synth.interleave_rows(b1, w.I), w2_bias=b2)
    assert np.array_equal(orc.forward(sep, d["x"], ids, wt), orc.forward(itl, d["x"], ids, wt))
    if act == 0:  # and the wrong row order does not
        wrong = orc.Layer(w.H, w.I, w.E_total, w.K, w.wfmt, w.afmt, w1i, w1si, d["w2"], d["w2_scale"], act=act)
        assert not np.allclose(orc.forward(wrong, d["x"], ids, wt), orc.forward(sep, d["x"], ids, wt))


def test_w2_bias_adds_weighted_bias(orc):
    w, d = small()
    ids, wt = orc.route_topk(d["logits"], w.K)
    b1, b2 = synth.make_biases(w)
    base = orc.forward(layer(orc, w, d, w1_bias=b1), d["x"], ids, wt)
    withb = orc.forward(layer(orc, w, d, w1_bias=b1, w2_bias=b2), d["x"], ids, wt)
    b2f = synth.bf16_bits_to_f32(b2).astype(np.float64)
    want = np.einsum("tk,tkh->th", wt.astype(np.float64), b2f[ids])
    np.testing.assert_allclose(withb - base, want, rtol=1e-9, atol=1e-9 * np.abs(base).max())


def zero_w1_layer(orc, w, d, b1, **kw):
    """w1 codes all zero: gate and up are exactly their biases for every token."""
    z = np.zeros_like(d["w1"])
    return orc.Layer(w.H, w.I, w.E_total, w.K, w.wfmt, w.afmt, z, d["w1_scale"], d["w2"], d["w2_scale"],
                     act=orc.ACT_SWIGLU_OAI, w1_bias=b1, **kw)


def h_for(orc, w, d, gate, up, **kw):
    b1 = np.zeros((w.E_total, 2 * w.I), np.float32)
    b1[:, : w.I] = gate
    b1[:, w.I:] = up
    L = zero_w1_layer(orc, w, d, synth.f32_to_bf16_bits(b1), **kw)
    ids = np.zeros((w.T, w.K), np.int32)
    ids[:, 1:] = -1  # one slot
    h = orc.stage1(L, d["x"], ids)
    return synth.bf16_bits_to_f32(h.reshape(w.T, w.K, w.I)[:, 0])


def test_swiglu_oai_clamp_invariances(orc):
    w, d = small()
    at = lambda g, u, **kw: h_for(orc, w, d, g, u, **kw)
    # the gate is clamped from above only, the up value on both sides, at the limit 7
    assert np.array_equal(at(7.0, 2.0), at(8.0, 2.0)) and np.array_equal(at(7.0, 2.0), at(96.0, 2.0))
    assert not np.array_equal(at(-7.0, 2.0), at(-8.0, 2.0))
    assert np.array_equal(at(3.0, 7.0), at(3.0, 9.0)) and np.array_equal(at(3.0, -7.0), at(3.0, -40.0))
    assert not np.array_equal(at(3.0, 6.0), at(3.0, 6.5))
    # no clamping with limit 0
    assert not np.array_equal(at(7.0, 2.0, limit=0.0), at(8.0, 2.0, limit=0.0))
    # zeros: up = -beta, or gate = 0
    assert np.all(at(2.5, -1.0) == 0.0) and np.all(at(0.0, 3.0) == 0.0)
    # positive below the limit, and a larger gate gives more (gate * sigmoid(alpha*gate) is increasing there)
    a, b = at(1.0, 1.0), at(2.0, 1.0)
    assert np.all(a > 0) and np.all(b > a)
