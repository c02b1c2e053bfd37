"""GPU parity of the router, the align-sort and the activation quantisers against
the oracle: bit-exact ids, counts, offsets, sorted slots, block owners, codes and
scales; router weights within fp32 rounding of the oracle's fp64 values."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, B, bf16_dev, orc, say, synth, to_dev

pytestmark = pytest.mark.gpu

ROUTER_CASES = [
    # name, T, E, topk, score, renorm, n_shared, logits
    ("tiny", 64, 8, 2, "softmax", True, 0, "normal"),
    ("decode", 64, 32, 4, "softmax", True, 0, "normal15"),
    ("prefill-zipf", 8192, 128, 4, "softmax", True, 0, "zipf"),
    ("fp8-block", 4096, 256, 8, "sigmoid", True, 1, "normal"),
    ("fp8-channel", 4096, 8, 2, "softmax", True, 0, "normal"),
    ("ties", 300, 64, 6, "softmax", True, 0, "ties"),
    ("no-renorm", 100, 96, 3, "softmax", False, 2, "normal"),
    ("sigmoid-no-renorm", 100, 20, 5, "sigmoid", False, 0, "normal"),
    ("max-E", 37, 1024, 32, "softmax", True, 32, "normal"),
    ("top1", 50, 16, 1, "softmax", True, 0, "normal"),
    ("single-token", 1, 8, 2, "softmax", True, 0, "normal"),
]


def make_logits(T, E, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "zipf":
        w = synth.WORKLOADS["prefill"].scaled(T=T)
        return synth.make_logits(w)
    if kind == "ties":
        return (np.round(rng.standard_normal((T, E)) * 2) / 2).astype(np.float32)
    std = 1.5 if kind == "normal15" else 1.0
    return rng.normal(0, std, (T, E)).astype(np.float32)


@pytest.mark.parametrize("case", ROUTER_CASES, ids=[c[0] for c in ROUTER_CASES])
def test_route_topk(case):
    name, T, E, k, score, renorm, ns, kind = case
    say(f"route {name}: T={T} E={E} k={k} {score} renorm={renorm} shared={ns}")
    logits = make_logits(T, E, kind, 100 + T + E)
    ids, w = B.moe_route_topk(to_dev(logits), k, score, renorm, ns, 0.5 if ns else 1.0)
    torch.cuda.synchronize()
    ref_ids, ref_w = orc.route_topk(logits, k, orc.SCORE_SOFTMAX if score == "softmax" else orc.SCORE_SIGMOID,
                                    renorm, ns, 0.5 if ns else 1.0)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-30)


def test_route_empty():
    ids, w = B.moe_route_topk(torch.empty((0, 8), dtype=torch.float32, device=DEV), 2)
    torch.cuda.synchronize()
    assert ids.shape == (0, 2)


ROUTE_ALIGN_CASES = [
    # T, E, topk, score, renorm, n_shared, bm   (fused when E <= 64, T*(topk+n_shared) <= 4096, T*E <= 8192)
    (64, 32, 4, "softmax", True, 0, 16), (1, 8, 2, "softmax", True, 0, 16), (0, 32, 4, "softmax", True, 0, 16),
    (32, 256, 8, "sigmoid", True, 1, 16), (8, 992, 32, "softmax", False, 32, 16), (1024, 8, 2, "softmax", True, 0, 32),
    (455, 256, 8, "sigmoid", True, 1, 32), (1024, 128, 4, "softmax", True, 0, 64), (37, 992, 32, "softmax", True, 32, 128),
    (100, 96, 3, "softmax", False, 2, 16), (1025, 128, 4, "softmax", True, 0, 64), (8192, 128, 4, "softmax", True, 0, 128),
]


@pytest.mark.parametrize("case", ROUTE_ALIGN_CASES)
def test_route_align(case):
    """The fused call equals route + sort run separately, bit for bit, and the oracle."""
    T, E, k, score, renorm, ns, bm = case
    say(f"route_align T={T} E={E} k={k} {score} renorm={renorm} shared={ns} bm={bm} fused={E <= 64 and T * (k + ns) <= 4096 and T * E <= 8192}")
    logits = make_logits(T, E, "normal", 500 + T + E)
    sw = 0.5 if ns else 1.0
    lg = to_dev(logits)
    ids, w, srt = B.moe_route_align(lg, k, bm, score, renorm, ns, sw)
    ids2, w2 = B.moe_route_topk(lg, k, score, renorm, ns, sw)
    srt2 = B.moe_align_sort(ids2, E + ns, bm)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w.view(torch.int32), w2.view(torch.int32))
    for key in ("expert_counts", "expert_offsets", "sorted_slots", "block_expert", "num_padded"):
        assert torch.equal(srt[key], srt2[key]), key
    ref_ids, _ = orc.route_topk(logits, k, orc.SCORE_SOFTMAX if score == "softmax" else orc.SCORE_SIGMOID, renorm,
                                ns, sw)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ref = orc.align_sort(ref_ids, E + ns, bm)
    for key in ("expert_counts", "expert_offsets", "sorted_slots"):
        assert np.array_equal(srt[key].cpu().numpy(), ref[key]), key
    assert int(srt["num_padded"].cpu()[0]) == ref["num_padded"]


@pytest.mark.parametrize("T,E,k,score,ns", [(64, 32, 4, "softmax", 0), (200, 40, 6, "sigmoid", 1),
                                            (128, 64, 32, "softmax", 0), (37, 8, 3, "softmax", 2)])
def test_route_align_ties(T, E, k, score, ns):
    """Logits on a coarse grid (many equal values per token, signed zeros included): the
    ids follow the value-then-lower-id rule, on the fused and the separate paths."""
    say(f"route_align ties T={T} E={E} k={k} {score} shared={ns}")
    logits = make_logits(T, E, "ties", 900 + T + E)
    logits[::3, : E // 2] = -0.0
    logits[1::3, E // 2:] = 0.0
    sw = 0.5 if ns else 1.0
    lg = to_dev(logits)
    ids, w, srt = B.moe_route_align(lg, k, 16, score, True, ns, sw)
    ids2, w2 = B.moe_route_topk(lg, k, score, True, ns, sw)
    srt2 = B.moe_align_sort(ids2, E + ns, 16)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w.view(torch.int32), w2.view(torch.int32))
    for key in ("expert_counts", "expert_offsets", "sorted_slots", "block_expert", "num_padded"):
        assert torch.equal(srt[key], srt2[key]), key
    sc = orc.SCORE_SOFTMAX if score == "softmax" else orc.SCORE_SIGMOID
    ref_ids, ref_w = orc.route_topk(logits, k, sc, True, ns, sw)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-30)


SORT_CASES = [(64, 2, 8, 16), (64, 4, 32, 16), (64, 4, 32, 32), (8192, 4, 128, 128), (8192, 4, 128, 64),
              (4096, 9, 257, 128), (1, 2, 8, 16), (16, 2, 8, 16), (256, 2, 8, 64), (4096, 2, 8, 128),
              (1000, 5, 1024, 16), (0, 4, 32, 16), (20000, 3, 7, 32)]


@pytest.mark.parametrize("T,K,E,bm", SORT_CASES)
def test_align_sort(T, K, E, bm):
    say(f"align_sort T={T} K={K} E={E} bm={bm}")
    rng = np.random.default_rng(T * 7 + K + E + bm)
    if T >= 8192:  # Zipf-skewed ids from the router
        logits = synth.make_logits(synth.WORKLOADS["prefill"].scaled(T=T, E=E))
        ids, _ = orc.route_topk(logits, K)
    else:
        ids = rng.integers(0, E, (T, K)).astype(np.int32)
    got = B.moe_align_sort(to_dev(ids), E, bm)
    torch.cuda.synchronize()
    ref = orc.align_sort(ids, E, bm)
    for key in ("expert_counts", "expert_offsets", "sorted_slots"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key
    nb = len(ref["block_expert"])
    assert np.array_equal(got["block_expert"].cpu().numpy()[:nb], ref["block_expert"])
    assert int(got["num_padded"].cpu()[0]) == ref["num_padded"]


@pytest.mark.parametrize("T,K,E,bm,offset", [(16384, 4, 128, 64, 0), (20000, 4, 61, 32, 1), (20000, 4, 61, 32, 0),
                                              (3000, 3, 9, 16, 3)])
def test_align_sort_id_layouts(T, K, E, bm, offset):
    """ids as a view into a larger buffer (starting 4 or 12 bytes past an aligned
    address) and at 16 workgroup chunks exactly, with ids outside [0, E) mixed in."""
    say(f"align_sort layouts T={T} K={K} E={E} bm={bm} offset={offset}")
    rng = np.random.default_rng(T + K + E + bm + offset)
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    ids[rng.random((T, K)) < 0.01] = -1
    ids[rng.random((T, K)) < 0.01] = E + 3
    buf = torch.empty(offset + T * K, dtype=torch.int32, device=DEV)
    buf[offset:] = to_dev(ids).reshape(-1)
    view = buf[offset:].view(T, K)
    assert (view.data_ptr() % 16) == 4 * offset % 16
    got = B.moe_align_sort(view, E, bm)
    torch.cuda.synchronize()
    ref = orc.align_sort(ids, E, bm)
    for key in ("expert_counts", "expert_offsets", "sorted_slots"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key
    nb = len(ref["block_expert"])
    assert np.array_equal(got["block_expert"].cpu().numpy()[:nb], ref["block_expert"])
    assert int(got["num_padded"].cpu()[0]) == ref["num_padded"]


def test_align_sort_invalid_ids_dropped():
    ids = np.array([[0, 5], [9, -1], [2, 2], [5, 5]], np.int32)
    got = B.moe_align_sort(to_dev(ids), 6, 16)
    torch.cuda.synchronize()
    ref = orc.align_sort(ids, 6, 16)
    for key in ("expert_counts", "expert_offsets", "sorted_slots"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key


QUANT_CASES = [("fp8-g128", B.A_FP8_G128, 40, 7168), ("fp8-g128-ragged", B.A_FP8_G128, 33, 160),
               ("fp8-token", B.A_FP8_TOKEN, 40, 4096), ("fp8-token-wide", B.A_FP8_TOKEN, 3, 14336),
               ("mxfp4", B.A_MXFP4_G32, 40, 2880), ("mxfp4-small", B.A_MXFP4_G32, 1, 32),
               ("fp8-tensor", B.A_FP8_TENSOR, 40, 4096), ("fp8-tensor-big", B.A_FP8_TENSOR, 4096, 7168),
               ("fp8-tensor-one", B.A_FP8_TENSOR, 1, 32),
               # eight columns per lane: a row narrower than one pass of the workgroup, an
               # odd number of 32-groups, and a last 128-group half full
               ("fp8-token-narrow", B.A_FP8_TOKEN, 5, 96), ("mxfp4-odd-groups", B.A_MXFP4_G32, 9, 96),
               ("fp8-g128-half-group", B.A_FP8_G128, 7, 2880), ("fp8-tensor-narrow", B.A_FP8_TENSOR, 3, 96),
               # per-token FP8: the widest row of the 256-thread kernel, the narrowest and
               # the widest of the 1024-thread one
               ("fp8-token-2048", B.A_FP8_TOKEN, 4, 2048), ("fp8-token-2080", B.A_FP8_TOKEN, 4, 2080),
               ("fp8-token-16416", B.A_FP8_TOKEN, 2, 16416), ("fp8-token-32768", B.A_FP8_TOKEN, 2, 32768),
               ("fp8-token-max", B.A_FP8_TOKEN, 3, 65536),
               # many rows: the 256- and 512-thread shapes (few rows take 1024 threads per row)
               ("fp8-token-rows-8192", B.A_FP8_TOKEN, 600, 8192), ("fp8-token-rows-14336", B.A_FP8_TOKEN, 600, 14336), ("fp8-token-rows-32768", B.A_FP8_TOKEN, 520, 32768),
               ("fp8-token-rows-65536", B.A_FP8_TOKEN, 513, 65536),
               # the group quantisers take 4 runs of lanes per workgroup: a grid whose last
               # workgroup is partly past the end
               ("fp8-g128-runs", B.A_FP8_G128, 65, 384), ("mxfp4-runs", B.A_MXFP4_G32, 37, 224)]


@pytest.mark.parametrize("case", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_quant_act(case):
    name, fmt, rows, cols = case
    say(f"quant {name} rows={rows} cols={cols}")
    rng = np.random.default_rng(rows * cols)
    scale = np.exp(rng.uniform(-8, 8, (rows, 1)))
    xf = rng.standard_normal((rows, cols)) * scale
    xf[0, :] = 0.0                      # all-zero row
    if rows > 2:
        xf[1, ::7] = -0.0
        xf[2, :] = np.round(xf[2, :] * 4) / 4  # many exact grid points / ties
    x = synth.f32_to_bf16_bits(xf.astype(np.float32))
    codes, scales = B.moe_quant_act(bf16_dev(x), fmt)
    torch.cuda.synchronize()
    rc, rs = orc.quant_act(x, fmt)
    gc = codes.cpu().numpy()
    gs = scales.cpu().numpy()
    assert np.array_equal(gs.view(np.uint8) if gs.dtype != np.uint8 else gs, rs.view(np.uint8)), "scales"
    assert np.array_equal(gc, rc), f"codes differ at {np.argwhere(gc != rc)[:5]}"


def test_quant_act_empty():
    codes, scales = B.moe_quant_act(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), B.A_FP8_G128)
    torch.cuda.synchronize()
    assert codes.shape == (0, 64)
