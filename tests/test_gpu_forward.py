"""GPU parity of the full expert layer (route -> sort -> quantise -> stage 1 ->
stage 2 -> combine) against the oracle.

Output bound: max|gpu - oracle| <= 2e-2 * rms(oracle) and per-token relative L2 <=
1e-2, on the GPU's fp32 result before its final rounding to bf16 (rebuilt exactly
from the per-slot fp32 rows in the workspace); the bf16 output is separately checked
to be that result rounded to nearest even, bit for bit.  The bound is not applied to
the bf16 values themselves because half a bf16 ulp of the largest outputs (up to ~9x
rms on these workloads) already exceeds 2e-2 * rms.  Stage-1 h is checked element-wise
to one bf16 ulp: both sides round an accumulated value to bf16 and the GPU's fp32 MFMA
sum runs in another order than the oracle's fp64 sum.

Quantised activations: that one-ulp freedom in h can move an a2 value across a
rounding boundary of its code, and a code step is a large change (1/8 of a value for
e4m3, up to 1/2 for e2m1).  The gate is staged: stage-1 h within one ulp of the
oracle's, the GPU's a2 codes bit-exactly equal to the oracle quantiser applied to the
GPU's own h, and the output bound against the oracle's stage 2 fed the GPU's h.  The
end-to-end result (oracle h, oracle a2) is reported with the count of differing a2 codes
(asserted below 0.2%), and its difference from the oracle is asserted to be at most the
difference between the oracle's outputs from its own h and from the GPU's h, plus the
output bound (per element and per row).  Measured on the
full-size fp8-block workload (N(0, 1/K) weights quantised per 128x128 block), the FP8
MFMA's 128-product sums leave 2.1% of h values one ulp from the oracle's fp64 result
(bf16 MFMA paths: 0.1-0.2%), 0.17% of a2 codes then differ, and one such step in the
shared expert's slot (weight 1) moves an output by up to ~4% of rms, so no implementation
whose h differs from the oracle's in the last bit can hold 2e-2 * rms end to end there.
"""
import numpy as np
import pytest
import torch

from gpu_common import (B, DEV, MAX_ABS_REL_RMS, ROW_REL_L2, bf16_dev, check_output, check_rounding, combine_f32,
                        dev_weights, h_by_slot, layer_for, orc, run_layer, say, synth, targeted_tokens,
                        tiled_reference, to_dev)

pytestmark = pytest.mark.gpu

W4A16 = (synth.W_MXFP4, synth.A_BF16)
W4A4 = (synth.W_MXFP4, synth.A_MXFP4_G32)
FP8B = (synth.W_FP8_BLOCK128, synth.A_FP8_G128)
FP8C = (synth.W_FP8_CHANNEL, synth.A_FP8_TOKEN)


def small(fmt, T=40, H=320, I=288, E=6, k=2, n_shared=0, score=synth.SCORE_SOFTMAX, seed=11):
    return synth.Workload(f"small-{fmt[0]}-{fmt[1]}", T, H, I, E, k, fmt[0], fmt[1], score=score,
                          n_shared=n_shared, seed=seed)


def check_a2(res, w, what):
    """GPU a2 codes and scales equal the oracle quantiser applied to the GPU's own h."""
    npad = int(res["sort"]["num_padded"][0])
    h = np.ascontiguousarray(res["h_sorted"][:npad])
    rc, rs = orc.quant_act(h, w.afmt)
    cs, ss, sdt = B.quant_shapes(w.afmt, res["cap"], w.I)
    gc = res["a2_codes"].reshape(cs)[:npad]
    gs = res["a2_scales"].view(np.uint8 if sdt == torch.uint8 else np.float32).reshape(ss)[:npad]
    assert np.array_equal(gc, rc), f"{what}: a2 codes differ at {np.argwhere(gc != rc)[:5]}"
    assert np.array_equal(gs.view(np.uint8), rs.view(np.uint8)), f"{what}: a2 scales differ"
    say(f"{what}: a2 codes/scales bit-exact on {npad} sorted rows")


def check_h_rows(h_gpu, ref_h, what):
    """Stage-1 h: both sides round an accumulated value to bf16, so they may differ by
    one bf16 ulp (<= 2^-7 relative) plus the fp32 accumulation error of the GPU sum."""
    got = synth.bf16_bits_to_f32(h_gpu).astype(np.float64)
    ref = synth.bf16_bits_to_f32(ref_h).astype(np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bound = 2.0 ** -7 * np.maximum(np.abs(ref), np.abs(got)) + 1e-3 * rms
    bad = np.abs(got - ref) > bound
    rows = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
    ulp_flips = int(np.count_nonzero(h_gpu != ref_h))
    say(f"{what}: stage-1 h differs in {ulp_flips}/{h_gpu.size} values, worst row rel L2={rows.max():.3e}")
    assert not bad.any(), f"{what}: stage-1 h outside one bf16 ulp at {np.argwhere(bad)[:5]}"
    assert rows.max() <= 1e-2


def full_check(w, data, res, tokens=None, what="", act=None):
    """Parity of one GPU run against the oracle on the listed tokens.
    bf16 activations: the end-to-end output meets the output bound.
    Quantised activations: a2 codes are bit-exact given the GPU's h, the output meets
    the bound against the oracle's stage 2 fed the GPU's h, and the end-to-end result
    (where a2 codes may differ because h was rounded differently) differs from the
    oracle's by no more than the oracle's own outputs from the two h differ, plus the
    bound; the number of a2 codes that differ must stay a small fraction.
    Returns the plain end-to-end figures (max |d| / rms, worst row relative L2)."""
    L = layer_for(w, data, act)
    ids, wts = res["ids"], res["weights"]
    ref_ids, ref_w = orc.route_topk(data["logits"], w.topk, w.score, True, w.n_shared, w.shared_weight)
    assert np.array_equal(ids, ref_ids), f"{what}: topk_ids"
    np.testing.assert_allclose(wts, ref_w, rtol=2e-6)
    tk = np.arange(w.T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    ref_h = orc.stage1(L, data["x"], ids, tk, topk_weights=wts)
    h_gpu = np.ascontiguousarray(h_by_slot(res, w.T, w.K, w.I).reshape(w.T, w.K, w.I)[tk].reshape(-1, w.I))
    check_h_rows(h_gpu, ref_h, what)
    ref = orc.stage2(L, ref_h, ids, wts, tk, T=w.T)  # == orc.forward on these tokens
    on_input = bool((act or {}).get("weight_on_input"))
    acc = combine_f32(dict(res, weights=np.ones_like(wts)) if on_input else res, tk, w.K, w.H, w.E_total)
    check_rounding(res["out"][tk], acc, what)
    if w.afmt == synth.A_BF16:
        return check_output(acc, ref, f"{what} end-to-end")
    check_a2(res, w, what)
    out2 = orc.stage2(L, h_gpu, ids, wts, tk, T=w.T)
    check_output(acc, out2, f"{what} stage 2 on GPU h")
    # a2 codes of the oracle's own h vs the GPU's h on the same slots
    valid = ids[tk].reshape(-1) < w.E_total
    c_ref, _ = orc.quant_act(ref_h[valid], w.afmt)
    c_gpu, _ = orc.quant_act(h_gpu[valid], w.afmt)
    flips = int(np.count_nonzero(c_ref != c_gpu))
    assert flips <= max(4, c_ref.size // 500), f"{what}: {flips} a2 code bytes differ"
    # each differing a2 code moves its row by one code step (module notes).  End to end, the
    # GPU may differ from the oracle by what those steps move, which the oracle computes
    # itself (its stage 2 fed the GPU's h), plus the output bound
    return check_end_to_end(acc, ref, out2, f"{what} end-to-end ({flips} of {c_ref.size} a2 code bytes differ)")


def check_end_to_end(got, ref, ref_gpu_h, what):
    """|got - ref| <= |ref_gpu_h - ref| + 2e-2 * rms(ref) per element, and per row
    |got - ref| <= |ref_gpu_h - ref| + 1e-2 |ref| in L2: the end-to-end difference is the
    one the oracle itself shows between its own h and the GPU's h, within the output
    bound.  Reports the plain end-to-end figures too."""
    got = got.astype(np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    d, dq = np.abs(got - ref), np.abs(ref_gpu_h - ref)
    rn = np.linalg.norm(ref, axis=1)
    en, eq = np.linalg.norm(got - ref, axis=1), np.linalg.norm(ref_gpu_h - ref, axis=1)
    rows = en / np.maximum(rn, 1e-300)
    say(f"{what}: max|d|/rms={d.max() / rms:.3e} worst row rel L2={rows.max():.3e} "
        f"(the oracle's own, from the GPU's h: {dq.max() / rms:.3e}, {(eq / np.maximum(rn, 1e-300)).max():.3e})")
    excess = d - dq - MAX_ABS_REL_RMS * rms
    assert excess.max() <= 0, f"{what}: end-to-end error exceeds the a2-step difference + bound at {np.argwhere(excess > 0)[:5]}"
    rex = en - eq - ROW_REL_L2 * rn
    assert rex.max() <= 0, f"{what}: row L2 exceeds the a2-step difference + bound in rows {np.argwhere(rex > 0)[:5]}"
    return d.max() / rms, rows.max()


SMALL = []
for fmt in (W4A16, W4A4, FP8B, FP8C):
    for bm in (16, 32, 64, 128):
        for tiled in (False, True):
            SMALL.append((fmt, bm, tiled))


@pytest.mark.parametrize("fmt,bm,tiled", SMALL,
                         ids=[f"w{f[0]}a{f[1]}-bm{bm}-{'tiled' if t else 'canon'}" for f, bm, t in SMALL])
def test_small_all_formats(fmt, bm, tiled):
    # several K chunks with a ragged tail (H=320, I=288), ragged column strips, pad rows
    if fmt == FP8B:
        w = small(fmt, T=40, H=352, I=288, E=5, k=3, n_shared=1, score=synth.SCORE_SIGMOID)
    elif fmt == FP8C:
        w = small(fmt, T=33, H=320, I=416, E=4, k=2)
    else:
        w = small(fmt)
    say(f"small forward {w.name} bm={bm} tiled={tiled} T={w.T} H={w.H} I={w.I} E={w.E_total} K={w.K}")
    data = synth.make_all(w)
    res = run_layer(w, data, block_m=bm, tiled=tiled)
    full_check(w, data, res, what=f"{w.name}/bm{bm}/{'tiled' if tiled else 'canon'}")


@pytest.mark.parametrize("fmt", [W4A16, W4A4, FP8B, FP8C], ids=["w4a16", "w4a4", "fp8b", "fp8c"])
def test_lds_ring_wraps(fmt):
    # 128-row blocks on tiled weights: more K chunks than the LDS ring holds (H=1440 is
    # 11.25 chunks, I=1056 8.25), so every ring buffer is reused, with ragged K tails, two
    # row blocks per expert (the second partly padding) and ragged column strips
    w = small(fmt, T=300, H=1440, I=1056, E=4, k=2, seed=71)
    say(f"ring wrap {w.name} bm=128 tiled T={w.T} H={w.H} I={w.I} E={w.E_total} K={w.K}")
    data = synth.make_all(w)
    res = run_layer(w, data, block_m=128, tiled=True)
    full_check(w, data, res, what=f"{w.name}/ring-wrap")


RING64 = [(W4A16, False, False), (W4A4, True, False), (FP8B, True, False), (FP8C, True, False),
          (FP8C, False, False), ((synth.W_FP8_TENSOR, synth.A_FP8_TENSOR), True, False),
          ((synth.W_BF16, synth.A_BF16), False, False), (W4A16, True, True), (FP8C, True, True)]


@pytest.mark.parametrize("fmt,tiled,oai", RING64,
                         ids=[f"w{f[0]}a{f[1]}-{'tiled' if t else 'canon'}{'-bias-oai' if o else ''}"
                              for f, t, o in RING64])
def test_bm64_long_k(fmt, tiled, oai):
    """64-row blocks over a longer stage-2 K: I = 1056 is 9 K chunks with a ragged last
    one, more than the kernel's register ring period (6 chunks at two chunks ahead), so
    the ring wraps in stage 2 as well as stage 1, on every format and layout, with biases
    and SwiGLU-OAI on interleaved rows."""
    w = small(fmt, T=40, H=320, I=1056, E=4, k=2, seed=83)
    data = synth.make_all(w)
    act = None
    if oai:
        act, data = oai_case(w, data, True, True, kind=1)
    what = f"{w.name}/bm64-long-k/{'tiled' if tiled else 'canon'}{'/bias-oai' if oai else ''}"
    say(f"forward {what} T={w.T} H={w.H} I={w.I}")
    res = run_layer(w, data, block_m=64, tiled=tiled, act=act)
    full_check(w, data, res, what=what, act=act)


@pytest.mark.parametrize("wfmt,N,K", [(synth.W_MXFP4, 64, 320), (synth.W_MXFP4, 576, 2880),
                                      (synth.W_FP8_BLOCK128, 96, 352), (synth.W_FP8_CHANNEL, 32, 4096)])
def test_tile_weights_layout(wfmt, N, K):
    """The kernel layout is an exact permutation of the canonical codes (and scales)."""
    rng = np.random.default_rng(N + K)
    E = 3
    if wfmt == synth.W_MXFP4:
        w = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
        ws = rng.integers(100, 140, (E, N, K // 32), dtype=np.uint8)
    else:
        w = rng.integers(0, 256, (E, N, K), dtype=np.uint8)
        ws = None
    got = B.moe_tile_weights(to_dev(w), to_dev(ws) if ws is not None else None, wfmt, K)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), tiled_reference(wfmt, w, ws, K))


def oai_case(w, data, interleaved, bias, kind=1):
    """Host act spec and matching data: SwiGLU-OAI (alpha 1.702, beta 1, limit 7) or SiLU,
    optionally interleaved gate/up rows (codes and scales permuted) and biases."""
    act = dict(kind=kind, alpha=1.702, beta=1.0, limit=7.0, interleaved=interleaved)
    b1, b2 = synth.make_biases(w) if bias else (None, None)
    if interleaved:
        s1 = data["w1_scale"]  # per-tensor scales ([E]) have no rows to permute
        data = dict(data, w1=synth.interleave_rows(data["w1"], w.I),
                    w1_scale=synth.interleave_rows(s1, w.I) if s1 is not None and s1.ndim > 1 else s1)
        b1 = synth.interleave_rows(b1, w.I) if b1 is not None else None
    act.update(w1_bias=b1, w2_bias=b2)
    return act, data


OAI = []
for fmt in (W4A16, W4A4, FP8C):
    for bm in (16, 32, 64, 128):
        OAI.append((fmt, bm, True, True, 1))
for bm in (16, 32, 64, 128):
    OAI.append((FP8B, bm, False, True, 1))
OAI += [(W4A16, 16, False, True, 0), (W4A16, 64, False, True, 0), (W4A16, 16, True, False, 1),
        (W4A16, 64, False, False, 1)]


@pytest.mark.parametrize("fmt,bm,itl,bias,kind", OAI,
                         ids=[f"w{f[0]}a{f[1]}-bm{bm}-{'itl' if i else 'sep'}-{'bias' if b else 'nobias'}-"
                              f"{'oai' if k else 'silu'}" for f, bm, i, b, k in OAI])
def test_swiglu_oai_bias_interleave(fmt, bm, itl, bias, kind):
    """SwiGLU-OAI / SiLU with projection biases and interleaved or separated gate/up rows,
    every kernel (16/32-row and 64/128-row blocks), against the oracle."""
    if fmt == FP8B:
        w = small(fmt, T=40, H=352, I=288, E=5, k=3, n_shared=1, score=synth.SCORE_SIGMOID)
    elif fmt == FP8C:
        w = small(fmt, T=33, H=320, I=416, E=4, k=2)
    else:
        w = small(fmt)
    data = synth.make_all(w)
    act, data = oai_case(w, data, itl, bias, kind)
    what = f"{w.name}/bm{bm}/{'itl' if itl else 'sep'}/{'bias' if bias else 'nobias'}/{'oai' if kind else 'silu'}"
    say(f"act forward {what}")
    res = run_layer(w, data, block_m=bm, tiled=True, act=act)
    full_check(w, data, res, what=what, act=act)


TKW1 = [(fmt, bm) for fmt in (W4A16, W4A4, FP8B, FP8C) for bm in (16, 32, 64)]


@pytest.mark.parametrize("fmt,bm", TKW1, ids=[f"w{f[0]}a{f[1]}-bm{bm}" for f, bm in TKW1])
def test_router_weight_on_input(fmt, bm):
    """Top-1 routing with the router weight on the input (the tkw1 form): the weight
    scales both stage-1 projections and the combine is unweighted."""
    if fmt == FP8B:
        w = small(fmt, T=40, H=352, I=288, E=5, k=1, score=synth.SCORE_SIGMOID)
    elif fmt == FP8C:
        w = small(fmt, T=33, H=320, I=416, E=4, k=1)
    else:
        w = small(fmt, k=1)
    data = synth.make_all(w)
    act = dict(kind=0, weight_on_input=True)
    what = f"{w.name}/bm{bm}/tkw1"
    say(f"forward {what}")
    res = run_layer(w, data, block_m=bm, tiled=True, act=act)
    # with one routed slot the softmax weight is exactly 1: use sigmoid-style weights instead
    assert res["weights"].shape[1] == 1
    full_check(w, data, res, what=what, act=act)


def test_router_weight_on_input_non_unit_weights():
    """The same with weights != 1 (sigmoid scores without renormalisation)."""
    w = synth.Workload("tk", 48, 320, 288, 6, 1, synth.W_MXFP4, synth.A_BF16, score=synth.SCORE_SIGMOID, seed=41)
    data = synth.make_all(w)
    wd = dev_weights(data)
    x = bf16_dev(data["x"])
    ids, wts = B.moe_route_topk(to_dev(data["logits"]), 1, "sigmoid", False)
    srt = B.moe_align_sort(ids, w.E_total, 16)
    act = dict(kind=0, weight_on_input=True)
    out, ws = B.moe_experts_forward(x, wd["w1"], wd["w1_scale"], wd["w2"], wd["w2_scale"], ids, wts, srt, w.wfmt,
                                    w.afmt, 16, w.E_total, w.I, act=act)
    torch.cuda.synchronize()
    ids_h, wts_h = ids.cpu().numpy(), wts.cpu().numpy()
    assert np.all(wts_h < 1.0)
    L = layer_for(w, data, act)
    ref = orc.forward(L, data["x"], ids_h, wts_h)
    args = B.forward_args(x, wd["w1"], wd["w1_scale"], wd["w2"], wd["w2_scale"], ids, wts, srt, w.wfmt, w.afmt, 16,
                          w.E_total, w.I, out, ws, act=act)
    lay = B.moe_workspace_layout(args)
    res = dict(ids=ids_h, weights=np.ones_like(wts_h),
               ybuf_dev=ws[lay["ybuf_off"]:lay["ybuf_off"] + lay["ybuf_bytes"]].view(torch.float32).view(-1, w.H))
    acc = combine_f32(res, np.arange(w.T, dtype=np.int32), 1, w.H, w.E_total)
    check_rounding(out.view(torch.int16).cpu().numpy().view(np.uint16), acc, "tkw1 sigmoid weights")
    check_output(acc, ref, "tkw1 sigmoid weights")


def test_swiglu_oai_decode_full_size():
    """The decode-shaped layer (H=I=2880, 32 experts, top-4) as a gpt-oss-style layer:
    SwiGLU-OAI, interleaved w13 rows, both biases, tiled weights, the benchmark's launch
    configuration; all 64 tokens checked."""
    w = synth.WORKLOADS["decode"]
    data = synth.make_all(w)
    act, data = oai_case(w, data, True, True)
    res = run_layer(w, data, tiled=True, act=act)
    full_check(w, data, res, what="decode/oai", act=act)


def test_determinism_and_token_permutation():
    w = small(W4A16, T=48, E=5, k=2)
    data = synth.make_all(w)
    r1 = run_layer(w, data, block_m=16)
    r2 = run_layer(w, data, block_m=16)
    assert np.array_equal(r1["out"], r2["out"])
    p = np.random.default_rng(0).permutation(w.T)
    dp = dict(data, x=np.ascontiguousarray(data["x"][p]), logits=np.ascontiguousarray(data["logits"][p]))
    r3 = run_layer(w, dp, block_m=16)
    assert np.array_equal(r3["out"], r1["out"][p])


def test_empty_tokens():
    w = small(W4A16, T=0)
    data = synth.make_all(w)
    res = run_layer(w, data, block_m=16)
    assert res["out"].shape == (0, w.H)


def test_single_token_all_slots_one_expert():
    w = small(W4A16, T=1, E=4, k=2)
    data = synth.make_all(w)
    res = run_layer(w, data, block_m=16)
    full_check(w, data, res, what="single-token")


# ---------------------------------------------------------------- full-size workloads
@pytest.mark.parametrize("name,tiled", [("tiny", False), ("decode", False), ("decode", True), ("prefill", False),
                                        ("prefill", True)])
def test_full_size_mxfp4_w4a16(name, tiled):
    w = synth.WORKLOADS[name]
    say(f"full-size {name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.topk} tiled={tiled}")
    data = synth.make_all(w)
    res = run_layer(w, data, tiled=tiled)  # library-picked block_m, as the benchmark runs it
    tk = None if w.T <= 64 else targeted_tokens(res, w.T, w.K, n_min=32, seed=5)
    full_check(w, data, res, tokens=tk, what=f"{name}/{'tiled' if tiled else 'canon'}")


def test_full_size_prefill_w4a4():
    w = synth.WORKLOADS["prefill-w4a4"]
    say(f"full-size {w.name}: T={w.T}")
    data = synth.make_all(w)
    res = run_layer(w, data, tiled=True)  # the benchmark's launch configuration (tiled, picked block_m)
    # a1 codes are an integer product of the GPU quantiser: bit-exact on every token
    rc, rs = orc.quant_act(data["x"], w.afmt)
    assert np.array_equal(res["a1_codes"], rc) and np.array_equal(res["a1_scales"], rs)
    full_check(w, data, res, tokens=targeted_tokens(res, w.T, w.K, n_min=32, seed=6), what=w.name)


def test_full_size_fp8_block_shared():
    w = synth.WORKLOADS["fp8-block"]
    say(f"full-size {w.name}: T={w.T} H={w.H} I={w.I} E={w.E}+{w.n_shared}")
    data = synth.make_all(w)
    res = run_layer(w, data, tiled=True)  # the benchmark's launch configuration (tiled, picked block_m)
    say(f"{w.name}: block_m {res['bm']}")
    rc, rs = orc.quant_act(data["x"], w.afmt)
    assert np.array_equal(res["a1_codes"], rc) and np.array_equal(res["a1_scales"], rs)
    assert np.all(res["ids"][:, w.topk] == w.E) and np.all(res["weights"][:, w.topk] == 1.0)
    tk = targeted_tokens(res, w.T, w.K, n_min=16, seed=7)
    say(f"{w.name}: {len(tk)} targeted tokens (last row block of each of {w.E_total} experts, hot and cold experts)")
    full_check(w, data, res, tokens=tk, what=w.name)


@pytest.fixture(scope="module")
def fp8_channel_data():
    w = synth.WORKLOADS["fp8-channel"]
    return w, synth.make_all(w)


@pytest.mark.parametrize("T", [1, 16, 256, 4096])
def test_full_size_fp8_channel_sweep(fp8_channel_data, T):
    w0, d0 = fp8_channel_data
    w = w0.with_T(T)
    say(f"full-size {w.name}: T={T}")
    data = dict(d0, x=np.ascontiguousarray(d0["x"][:T]), logits=np.ascontiguousarray(d0["logits"][:T]))
    res = run_layer(w, data, tiled=True)  # the benchmark's launch configuration (tiled, picked block_m)
    rc, rs = orc.quant_act(data["x"], w.afmt)
    assert np.array_equal(res["a1_codes"], rc) and np.array_equal(res["a1_scales"], rs)
    e_max, e_row = full_check(w, data, res, tokens=targeted_tokens(res, T, w.K, n_min=16, seed=8),
                              what=f"{w.name}/T{T}")
    # per-token a2 over I = 14336 values and two softmax-weighted slots: one a2 code step
    # moves an output row by about 1/8 of one of 14336 terms, so the output bound holds end
    # to end here as well, and is asserted as it stands
    assert e_max <= MAX_ABS_REL_RMS, f"{w.name}/T{T}: end-to-end max|d| = {e_max:.3e} rms"
    assert e_row <= ROW_REL_L2, f"{w.name}/T{T}: end-to-end row L2 = {e_row:.3e}"


FP8T = (synth.W_FP8_TENSOR, synth.A_FP8_TENSOR)
FP8T_CASES = [(bm, tiled) for bm in (16, 32, 64, 128) for tiled in (False, True)]


@pytest.mark.parametrize("bm,tiled", FP8T_CASES, ids=[f"bm{bm}-{'tiled' if t else 'canon'}" for bm, t in FP8T_CASES])
def test_fp8_per_tensor(bm, tiled):
    """Per-tensor FP8 (one weight scale per expert and projection, one dynamic activation
    scale per tensor) on every kernel; the whole batch is checked (the scales depend on it)."""
    w = small(FP8T, T=33, H=320, I=416, E=4, k=2)
    data = synth.make_all(w)
    say(f"forward fp8-tensor bm={bm} tiled={tiled}")
    res = run_layer(w, data, block_m=bm, tiled=tiled)
    assert res["a1_scales"].view(np.float32).size == 1
    full_check(w, data, res, what=f"fp8-tensor/bm{bm}/{'tiled' if tiled else 'canon'}")


@pytest.mark.parametrize("bm", [16, 32, 64])
def test_fp8_per_tensor_with_biases(bm):
    """Per-tensor FP8 with both projection biases and interleaved gate/up rows: pad rows of
    h are written as 0, so the per-tensor a2 scale covers the routed rows only, as the
    oracle's does (a pad row with act(bias) would raise the amax)."""
    w = small(FP8T, T=33, H=320, I=416, E=4, k=2, seed=73)
    data = synth.make_all(w)
    act, data = oai_case(w, data, True, True, kind=1)
    what = f"fp8-tensor/bm{bm}/itl/bias/oai"
    say(f"forward {what}")
    res = run_layer(w, data, block_m=bm, tiled=True, act=act)
    npad = int(res["sort"]["num_padded"][0])
    pad = res["sort"]["sorted_slots"][:npad] >= w.T * w.K
    assert pad.any() and not res["h_sorted"][:npad][pad].any(), "pad rows of h must be 0"
    full_check(w, data, res, what=what, act=act)


UNIFORM = [(FP8B, 16), (FP8B, 64), (FP8C, 32), (FP8C, 64)]


@pytest.mark.parametrize("fmt,bm", UNIFORM, ids=[f"w{f[0]}a{f[1]}-bm{bm}" for f, bm in UNIFORM])
def test_small_fp8_uniform_codes(fmt, bm):
    """FP8 weights drawn as uniform codes over [0.125, 1.875] with random fp32 scales (the
    other weight generator), on the small shapes."""
    if fmt == FP8B:
        w = small(fmt, T=40, H=352, I=288, E=5, k=3, n_shared=1, score=synth.SCORE_SIGMOID, seed=13)
    else:
        w = small(fmt, T=33, H=320, I=416, E=4, k=2, seed=14)
    w = w.scaled(fp8_weights="uniform")
    data = synth.make_all(w)
    res = run_layer(w, data, block_m=bm, tiled=True)
    full_check(w, data, res, what=f"{w.name}/bm{bm}/uniform-codes")
