"""Helpers of the GPU parity tests: move synthetic inputs to the device, run the
HIP path through the C-ABI binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import oracle as orc
from quantized_mixture_experts_softmax_amd import binding as B
from quantized_mixture_experts_softmax_amd import synth

DEV = "cuda:0"

# Output bound on floating point results (max abs error relative to the oracle's rms,
# and relative L2 error per token row).
MAX_ABS_REL_RMS = 2e-2
ROW_REL_L2 = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def layer_for(w: synth.Workload, data: dict, act: dict | None = None) -> orc.Layer:
    """act (host spec): dict(kind, alpha, beta, limit, interleaved, w1_bias, w2_bias), the
    biases as bf16 bit arrays or None; data's w1 rows are in the spec's order."""
    a = act or {}
    return orc.Layer(w.H, w.I, w.E_total, w.K, w.wfmt, w.afmt, data["w1"], data["w1_scale"], data["w2"],
                     data["w2_scale"], act=a.get("kind", 0), alpha=a.get("alpha", 1.702), beta=a.get("beta", 1.0),
                     limit=a.get("limit", 7.0), gate_up_interleaved=bool(a.get("interleaved", False)),
                     w1_bias=a.get("w1_bias"), w2_bias=a.get("w2_bias"),
                     weight_on_input=bool(a.get("weight_on_input", False)))


def act_dev(act: dict | None) -> dict | None:
    """The host act spec with its biases moved to the GPU as bf16 tensors."""
    if act is None:
        return None
    d = dict(act)
    for k in ("w1_bias", "w2_bias"):
        if d.get(k) is not None:
            d[k] = to_dev(d[k], torch.bfloat16)
    return d


def dev_weights(data: dict) -> dict:
    """The weights and scales on the GPU (bf16 weights as bf16 tensors; absent scales None)."""
    out = {}
    for k in ("w1", "w1_scale", "w2", "w2_scale"):
        a = data[k]
        out[k] = None if a is None else (bf16_dev(a) if a.dtype == np.uint16 else to_dev(a))
    return out


def score_name(w: synth.Workload) -> str:
    return "softmax" if w.score == synth.SCORE_SOFTMAX else "sigmoid"


def combine_f32(res: dict, tokens: np.ndarray, K: int, H: int, E_total: int) -> np.ndarray:
    """The GPU's fp32 result before its final bf16 rounding, rebuilt from the per-slot
    rows it left in the workspace the way the combine kernel sums them: in ascending
    slot order, each row times its top-k weight rounded to fp32, then added in fp32."""
    ybuf = res["ybuf_dev"]
    ids, wts = res["ids"], res["weights"].astype(np.float32)
    rows = (tokens[:, None] * K + np.arange(K)[None, :]).reshape(-1)
    y = ybuf[torch.from_numpy(rows).to(ybuf.device)].cpu().numpy().reshape(len(tokens), K, H)
    acc = np.zeros((len(tokens), H), np.float32)
    for j in range(K):
        ok = (ids[tokens, j] >= 0) & (ids[tokens, j] < E_total)
        prod = (y[:, j] * wts[tokens, j][:, None]).astype(np.float32)
        acc = np.where(ok[:, None], acc + prod, acc).astype(np.float32)
    return acc


def check_rounding(got_bf16: np.ndarray, acc_f32: np.ndarray, what: str):
    """The bf16 output is the round-to-nearest-even of the fp32 result, bit for bit."""
    want = synth.f32_to_bf16_bits(acc_f32)
    assert np.array_equal(got_bf16, want), f"{what}: bf16 output is not the rounded fp32 sum"


def check_output(got, ref: np.ndarray, what: str, max_rel=MAX_ABS_REL_RMS, row_l2=ROW_REL_L2):
    got = (synth.bf16_bits_to_f32(got) if got.dtype == np.uint16 else got).astype(np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(got - ref)
    max_rel_err = float(err.max() / rms) if rms > 0 else float(err.max())
    rn = np.sqrt(np.sum(ref ** 2, axis=1))
    en = np.sqrt(np.sum((got - ref) ** 2, axis=1))
    rows = en / np.maximum(rn, 1e-300)
    say(f"{what}: max|d|/rms={max_rel_err:.3e} worst row rel L2={rows.max():.3e} rms={rms:.4g}")
    assert max_rel_err <= max_rel, f"{what}: max|gpu-oracle| = {max_rel_err:.3e} * rms > {max_rel}"
    assert rows.max() <= row_l2, f"{what}: row relative L2 {rows.max():.3e} > {row_l2}"
    return max_rel_err, float(rows.max())


def run_layer(w: synth.Workload, data: dict, block_m: int | None = None, wd: dict | None = None, tiled=False,
              act: dict | None = None):
    """Route, sort, quantise and run the expert layer on the GPU through the ABI.
    Returns a dict of host copies of every intermediate."""
    wd = wd or dev_weights(data)
    x = bf16_dev(data["x"])
    logits = to_dev(data["logits"])
    layer = B.MoELayer(wd["w1"], wd["w1_scale"], wd["w2"], wd["w2_scale"], H=w.H, I=w.I, E=w.E, topk=w.topk,
                       wfmt=w.wfmt, afmt=w.afmt, score=score_name(w), n_shared=w.n_shared,
                       shared_weight=w.shared_weight, block_m=block_m, tiled=tiled, act=act_dev(act))
    out = layer(x, logits)
    torch.cuda.synchronize()
    b = layer._bufs[(x.shape[0], str(x.device))]
    res = dict(out=bf16_host(out), ids=b["ids"].cpu().numpy(), weights=b["w"].cpu().numpy(), bm=b["bm"],
               sort={k: v.cpu().numpy() for k, v in b["sort"].items()}, layer=layer, bufs=b)
    if b["workspace"] is not None:
        args = B.forward_args(x, layer.w1, layer.w1_scale, layer.w2, layer.w2_scale, b["ids"], b["w"], b["sort"],
                              w.wfmt, w.afmt, b["bm"], w.E_total, w.I, out, b["workspace"],
                              *(b["a1"] if b["a1"] else (None, None)), weight_layout=layer.weight_layout)
        L = B.moe_workspace_layout(args)
        ws = b["workspace"]
        cap = B.moe_sort_capacity(x.shape[0], w.K, w.E_total, b["bm"])
        res["h_sorted"] = ws[L["h_off"]:L["h_off"] + L["h_bytes"]].cpu().numpy().view(np.uint16).reshape(cap, w.I)
        if w.afmt != synth.A_BF16:
            res["a2_codes"] = ws[L["a2_codes_off"]:L["a2_codes_off"] + L["a2_codes_bytes"]].cpu().numpy()
            res["a2_scales"] = ws[L["a2_scales_off"]:L["a2_scales_off"] + L["a2_scales_bytes"]].cpu().numpy()
            res["a1_codes"] = b["a1"][0].cpu().numpy()
            res["a1_scales"] = b["a1"][1].cpu().numpy()
        res["cap"] = cap
        res["ybuf_dev"] = ws[L["ybuf_off"]:L["ybuf_off"] + L["ybuf_bytes"]].view(torch.float32).view(-1, w.H)
    return res


def targeted_tokens(res: dict, T: int, K: int, n_min: int = 16, seed: int = 0) -> np.ndarray:
    """Tokens for a sampled full-size parity check, chosen from the routing of the run:
    for every expert with slots, the token of its last sorted row (the expert's last,
    usually partial, row block); the first and last tokens of the hottest expert; every
    token of the (up to) four coldest experts; then random tokens up to n_min (at least
    as many tokens as the oracle's threads, which parallelise over tokens)."""
    ss = res["sort"]["sorted_slots"]
    counts = res["sort"]["expert_counts"]
    offs = res["sort"]["expert_offsets"]
    pick = set()
    hit = np.flatnonzero(counts > 0)
    for e in hit:
        pick.add(int(ss[offs[e] + counts[e] - 1]) // K)
    if len(hit):
        hot = hit[np.argmax(counts[hit])]
        pick.add(int(ss[offs[hot]]) // K)
        pick.add(int(ss[offs[hot] + counts[hot] - 1]) // K)
        for e in hit[np.argsort(counts[hit], kind="stable")][:4]:
            for r in range(offs[e], offs[e] + min(int(counts[e]), 8)):
                pick.add(int(ss[r]) // K)
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(T), np.fromiter(pick, np.int64, len(pick)))
    extra = max(0, min(n_min - len(pick), len(rest)))
    if extra:
        pick.update(int(t) for t in rng.choice(rest, extra, replace=False))
    return np.array(sorted(pick), np.int32)


def h_by_slot(res: dict, T: int, K: int, I: int) -> np.ndarray:
    """GPU stage-1 output rearranged from sorted rows to slot order [T*K, I]."""
    ss = res["sort"]["sorted_slots"]
    h = np.zeros((T * K, I), np.uint16)
    valid = ss < T * K
    h[ss[valid]] = res["h_sorted"][:len(ss)][valid]
    return h


def tiled_reference(wfmt: int, w: np.ndarray, ws: np.ndarray | None, K: int) -> np.ndarray:
    """The tiled weight layout written out with numpy index arithmetic: blocks
    [E][N/16][ceil(K/128)], lane l = 16g + r holds row r's K elements [128c + 32g, +32)."""
    E, N = w.shape[0], w.shape[1]
    nch = (K + 127) // 128
    if wfmt == synth.W_MXFP4:
        kb = K // 2
        wp = np.zeros((E, N, nch * 64), np.uint8)
        wp[:, :, :kb] = w
        sp = np.zeros((E, N, nch * 4), np.uint8)
        sp[:, :, :K // 32] = ws
        data = wp.reshape(E, N // 16, 16, nch, 4, 16).transpose(0, 1, 3, 4, 2, 5)  # e, n16, c, g, r, byte
        scal = sp.reshape(E, N // 16, 16, nch, 4).transpose(0, 1, 3, 4, 2)       # e, n16, c, g, r
        out = np.concatenate([data.reshape(E, N // 16, nch, 1024), scal.reshape(E, N // 16, nch, 64)], axis=3)
        return out.reshape(-1)
    wp = np.zeros((E, N, nch * 128), np.uint8)
    wp[:, :, :K] = w
    v = wp.reshape(E, N // 16, 16, nch, 4, 2, 16).transpose(0, 1, 3, 5, 4, 2, 6)  # e, n16, c, half, g, r, byte
    return v.reshape(-1)
