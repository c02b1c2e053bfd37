"""GPU parity of the expert-parallel share: the global -> local id map is bit-exact,
and each device's share of the layer (local weights, local ids) matches the oracle's
share; rows past the valid-token count come out zero."""
import numpy as np
import pytest
import torch

from gpu_common import (B, DEV, bf16_dev, bf16_host, check_output, check_rounding, combine_f32, h_by_slot, orc, say,
                        synth, to_dev)
from test_gpu_forward import check_end_to_end

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,K,E,n_valid", [(64, 4, 32, None), (1000, 9, 257, 700), (1, 2, 8, 1), (0, 4, 32, None),
                                           (333, 8, 1024, 0)])
def test_map_experts(T, K, E, n_valid):
    rng = np.random.default_rng(T + K + E)
    ids = rng.integers(-2, E + 3, (T, K)).astype(np.int32)
    emap = np.full(E, -1, np.int32)
    mine = rng.choice(E, max(1, E // 3), replace=False)
    emap[mine] = rng.permutation(len(mine)).astype(np.int32)
    nv = None if n_valid is None else to_dev(np.array([n_valid], np.int32))
    got = B.moe_map_experts(to_dev(ids), to_dev(emap), E, nv)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), orc.map_experts(ids, emap, E, n_valid))
    got2 = B.moe_map_experts(to_dev(ids), None, E)
    torch.cuda.synchronize()
    assert np.array_equal(got2.cpu().numpy(), orc.map_experts(ids, None, E))


def run_share(w, data, ids_dev, wts_dev, mine, bm, tiled, n_valid=None):
    """This device's share: local weights of the experts in `mine`, local ids, forward."""
    E_loc = len(mine)
    emap = np.full(w.E_total, -1, np.int32)
    emap[mine] = np.arange(E_loc, dtype=np.int32)
    pick = lambda a: None if a is None else np.ascontiguousarray(a[mine])
    wl = {k: pick(data[k]) for k in ("w1", "w1_scale", "w2", "w2_scale")}
    dev = lambda a: None if a is None else (bf16_dev(a) if a.dtype == np.uint16 else to_dev(a))
    nv = None if n_valid is None else to_dev(np.array([n_valid], np.int32))
    loc = B.moe_map_experts(ids_dev, to_dev(emap), w.E_total, nv)
    srt = B.moe_align_sort(loc, E_loc, bm)
    w1, w1s, w2, w2s = (dev(wl[k]) for k in ("w1", "w1_scale", "w2", "w2_scale"))
    layout = B.LAYOUT_CANONICAL
    if tiled:
        w1, w2 = B.moe_tile_weights(w1, w1s, w.wfmt, w.H), B.moe_tile_weights(w2, w2s, w.wfmt, w.I)
        layout = B.LAYOUT_TILED
        if w.wfmt == synth.W_MXFP4:
            w1s = w2s = None
    x = bf16_dev(data["x"])
    a1c = a1s = None
    if w.afmt != synth.A_BF16:
        a1c, a1s = B.moe_quant_act(x, w.afmt)
    out, ws = B.moe_experts_forward(x, w1, w1s, w2, w2s, loc, wts_dev, srt, w.wfmt, w.afmt, bm, E_loc, w.I,
                                    a1_codes=a1c, a1_scales=a1s, weight_layout=layout)
    torch.cuda.synchronize()
    args = B.forward_args(x, w1, w1s, w2, w2s, loc, wts_dev, srt, w.wfmt, w.afmt, bm, E_loc, w.I, out, ws, a1c, a1s,
                          weight_layout=layout)
    L = B.moe_workspace_layout(args)
    cap = B.moe_sort_capacity(w.T, w.K, E_loc, bm)
    res = dict(out=bf16_host(out), ids=loc.cpu().numpy(), weights=wts_dev.cpu().numpy(),
               ybuf_dev=ws[L["ybuf_off"]:L["ybuf_off"] + L["ybuf_bytes"]].view(torch.float32).view(-1, w.H),
               sort={k: v.cpu().numpy() for k, v in srt.items()},
               h_sorted=ws[L["h_off"]:L["h_off"] + L["h_bytes"]].cpu().numpy().view(np.uint16).reshape(cap, w.I))
    Lo = orc.Layer(w.H, w.I, E_loc, w.K, w.wfmt, w.afmt, wl["w1"], wl["w1_scale"], wl["w2"], wl["w2_scale"])
    return res, Lo


@pytest.mark.parametrize("name,bm,tiled", [("decode", 16, True), ("tiny", 64, False), ("fp8c", 32, True),
                                           ("bf16", 16, False), ("bf16", 64, False)])
def test_ep_shares(name, bm, tiled):
    if name == "fp8c":
        w = synth.Workload("fp8c", 16, 256, 512, 8, 2, synth.W_FP8_CHANNEL, synth.A_FP8_TOKEN, seed=77)
    elif name == "bf16":
        w = synth.Workload("bf16", 48, 320, 288, 16, 3, synth.W_BF16, synth.A_BF16, seed=78)
    else:
        w = synth.WORKLOADS[name]
    data = synth.make_all(w)
    ids, wts = B.moe_route_topk(to_dev(data["logits"]), w.topk, "softmax")
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    perm = rng.permutation(w.E_total)
    shares = np.array_split(perm, 4)
    tk = np.arange(w.T, dtype=np.int32)
    for s_i, mine in enumerate(shares):
        mine = np.sort(mine)
        say(f"ep share {name} {s_i}: experts {mine.tolist()} bm={bm}")
        res, Lo = run_share(w, data, ids, wts, mine, bm, tiled)
        ref_loc = orc.map_experts(ids.cpu().numpy(), np.where(np.isin(np.arange(w.E_total), mine),
                                                              np.searchsorted(mine, np.arange(w.E_total)), -1),
                                  w.E_total)
        assert np.array_equal(res["ids"], ref_loc)
        ref = orc.forward(Lo, data["x"], ref_loc, res["weights"])
        acc = combine_f32(res, tk, w.K, w.H, len(mine))
        check_rounding(res["out"], acc, f"ep {name} share {s_i}")
        if w.afmt == synth.A_BF16:
            check_output(acc, ref, f"ep {name} share {s_i}")
        else:  # quantised activations: the staged check of full_check in test_gpu_forward
            h_gpu = h_by_slot(res, w.T, w.K, w.I)
            out2 = orc.stage2(Lo, h_gpu, ref_loc, res["weights"])
            check_output(acc, out2, f"ep {name} share {s_i} stage 2 on GPU h")
            check_end_to_end(acc, ref, out2, f"ep {name} share {s_i} end-to-end")
        no_local = (ref_loc < 0).all(axis=1)
        assert np.all(res["out"][no_local] == 0)


def test_ep_share_valid_token_count():
    w = synth.WORKLOADS["tiny"]
    data = synth.make_all(w)
    ids, wts = B.moe_route_topk(to_dev(data["logits"]), w.topk, "softmax")
    res, Lo = run_share(w, data, ids, wts, np.arange(w.E_total), 16, False, n_valid=40)
    assert np.all(res["out"][40:] == 0)
    ref = orc.forward(Lo, data["x"], res["ids"], res["weights"])
    acc = combine_f32(res, np.arange(w.T, dtype=np.int32), w.K, w.H, w.E_total)
    check_output(acc[:40], ref[:40], "ep valid-token count")
