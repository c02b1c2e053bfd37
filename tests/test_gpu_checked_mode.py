"""Checked mode (moe_set_checked_mode): with it on, the forward entry points verify the
caller's routing tables on the device before any kernel reads them.  Valid tables give the
same output bit for bit as unchecked calls; a table entry outside the bounds the kernels
index with is reported as MOE_EINVAL, naming the entry, and nothing else runs.  The
corrupted tables are only ever passed with checked mode on."""
import numpy as np
import pytest
import torch

from gpu_common import B, bf16_dev, bf16_host, dev_weights, say, synth, to_dev

pytestmark = pytest.mark.gpu

W = synth.Workload("checked", 40, 320, 288, 6, 2, synth.W_MXFP4, synth.A_MXFP4_G32, seed=95)
BM = 16


@pytest.fixture(scope="module")
def setup():
    data = synth.make_all(W)
    wd = dev_weights(data)
    x = bf16_dev(data["x"])
    ids, wts, srt = B.moe_route_align(to_dev(data["logits"]), W.topk, BM, "softmax", True, 0, 1.0)
    torch.cuda.synchronize()
    yield data, wd, x, ids, wts, srt
    B.moe_set_checked_mode(False)


def forward(setup, srt, noalloc=False):
    data, wd, x, ids, wts, _ = setup
    if noalloc:
        out = B.moe_experts_forward_noalloc(x, wd["w1"], wd["w1_scale"], wd["w2"], wd["w2_scale"], ids, wts, srt,
                                            W.wfmt, W.afmt, BM, W.E_total, W.I)
    else:
        out, _ = B.moe_experts_forward(x, wd["w1"], wd["w1_scale"], wd["w2"], wd["w2_scale"], ids, wts, srt, W.wfmt,
                                       W.afmt, BM, W.E_total, W.I)
    torch.cuda.synchronize()
    return bf16_host(out)


def test_valid_tables_pass_unchanged(setup):
    srt = setup[5]
    B.moe_set_checked_mode(False)
    ref = forward(setup, srt)
    B.moe_set_checked_mode(True)
    try:
        assert np.array_equal(forward(setup, srt), ref)
        assert np.array_equal(forward(setup, srt, noalloc=True), ref)
    finally:
        B.moe_set_checked_mode(False)
    say(f"checked mode: valid tables ({int(srt['num_padded'][0])} padded rows) give the unchecked output")


def corrupt(srt, key, index, value):
    bad = {k: v.clone() for k, v in srt.items()}
    bad[key][index] = value
    return bad


CORRUPTIONS = [
    # a sorted slot past the pad sentinel T*K (its token row and per-slot row would be out of bounds)
    ("sorted_slots", 5, W.T * W.K + 7, "sorted_slots[5]"),
    ("sorted_slots", 3, -2, "sorted_slots[3]"),
    # a block owner past the experts (its weights would be read out of bounds)
    ("block_expert", 1, W.E_total + 3, "block_expert[1]"),
    # a padded total beyond the tables' capacity, and one that is not a multiple of block_m
    ("num_padded", 0, 1 << 20, "num_padded"),
    ("num_padded", 0, BM + 1, "num_padded"),
]


@pytest.mark.parametrize("key,index,value,named", CORRUPTIONS,
                         ids=[f"{c[0]}-{c[2]}" for c in CORRUPTIONS])
@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_corrupt_tables_are_rejected(setup, key, index, value, named, noalloc):
    bad = corrupt(setup[5], key, index, value)
    B.moe_set_checked_mode(True)
    try:
        with pytest.raises(B.MoeError) as ex:
            forward(setup, bad, noalloc=noalloc)
    finally:
        B.moe_set_checked_mode(False)
    assert ex.value.status == B.MOE_EINVAL and named in str(ex.value), str(ex.value)
    say(f"checked mode rejects {key}[{index}] = {value}: {ex.value}")
