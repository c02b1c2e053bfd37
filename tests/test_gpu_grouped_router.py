"""GPU parity of the grouped top-k router (score-correction bias, expert groups,
routed scaling factor) against the oracle: bit-exact ids, weights within fp32
rounding of the oracle's fp64 values; its ids feed the align-sort unchanged."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, B, orc, say, to_dev

pytestmark = pytest.mark.gpu

GROUPED_CASES = [
    # name, T, E, topk, groups, topk_group, score, bias, renorm, scaling, n_shared
    ("v3-shape", 4096, 256, 8, 8, 4, "sigmoid", True, True, 2.5, 1),
    ("v2-softmax", 1000, 64, 6, 8, 3, "softmax", False, True, 1.0, 0),
    ("ragged-no-renorm", 37, 32, 4, 4, 2, "sigmoid", True, False, 1.5, 0),
    ("max-E", 5, 1024, 8, 64, 8, "sigmoid", True, True, 1.0, 0),
    ("shared-2", 77, 512, 8, 16, 4, "sigmoid", True, True, 1.0, 2),
    ("group-of-one", 300, 16, 3, 16, 3, "softmax", True, True, 1.0, 0),
    ("all-groups-kept", 200, 48, 5, 6, 6, "sigmoid", False, True, 1.0, 0),
    ("one-group", 129, 160, 7, 1, 1, "softmax", True, True, 1.0, 0),
    ("single-token", 1, 128, 4, 4, 2, "sigmoid", True, True, 2.0, 0),
]


@pytest.mark.parametrize("case", GROUPED_CASES, ids=[c[0] for c in GROUPED_CASES])
def test_route_grouped_topk(case):
    name, T, E, k, G, TG, score, use_bias, renorm, scaling, ns = case
    say(f"grouped route {name}: T={T} E={E} k={k} groups={G} keep={TG} {score} bias={use_bias}")
    rng = np.random.default_rng(500 + T + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[: T // 10] = np.round(logits[: T // 10] * 2) / 2  # exact logit ties
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32) if use_bias else None
    ids, w = B.moe_route_grouped_topk(to_dev(logits), k, G, TG, None if bias is None else to_dev(bias), score,
                                      renorm, scaling, ns, 1.0)
    torch.cuda.synchronize()
    sc = orc.SCORE_SOFTMAX if score == "softmax" else orc.SCORE_SIGMOID
    ref_ids, ref_w = orc.route_grouped_topk(logits, k, G, TG, bias, sc, renorm, scaling, ns, 1.0)
    got = ids.cpu().numpy()
    assert np.array_equal(got, ref_ids), f"{name}: {int((got != ref_ids).any(axis=1).sum())} tokens differ"
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=2e-7, atol=1e-30)
    # the ids are valid input of the align-sort
    srt = B.moe_align_sort(ids, E + ns, 16)
    torch.cuda.synchronize()
    ref = orc.align_sort(ref_ids, E + ns, 16)
    assert np.array_equal(srt["expert_counts"].cpu().numpy(), ref["expert_counts"])


def test_route_grouped_empty():
    ids, w = B.moe_route_grouped_topk(torch.empty((0, 256), dtype=torch.float32, device=DEV), 8, 8, 4)
    torch.cuda.synchronize()
    assert ids.shape == (0, 8)
