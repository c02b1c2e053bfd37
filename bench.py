#!/usr/bin/env python3
"""Benchmark of the fused MoE expert layer hot path on one MI355X.

One step = one pass of the whole hot path over one batch already resident in HBM:
moe_route_topk -> moe_align_sort -> (moe_quant_act for quantised activations) ->
moe_experts_forward (stage-1 GEMM + SiLU-and-mul, a2 quantisation, stage-2 GEMM
weighted by the top-k weights, ordered combine).  Every step reads a different copy of
the weights when one copy would fit twice in the 256 MB Infinity Cache, so weight
bytes come from HBM.

Default workload: the decode-shaped MXFP4 w4a16 layer (T=64, H=I=2880, E=32, top-4),
with the weights in the tiled kernel layout (moe_tile_weights, a one-time permutation
done when the weights are loaded, outside the timed region).

Prints ONE JSON line.  `roofline` is for the stage-1 GEMM (the dominant kernel): its
algorithmic bytes (or flops) per launch divided by its average duration, timed with HIP
events recorded on the launch stream around the stage-1 launch of every n-th timed step
(--event-every, default 10: each event record adds a few microseconds to its step, so
the other steps run without them).
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same workload.

`extra_configs` (after the headline, --extra all): the prefill-sized workloads timed the
same way with fewer steps -- prefill MXFP4 w4a16 and w4a4 (T=8192, E=128, top-4), FP8 block
with a shared expert (T=4096, E=256+1, top-8+1) and the FP8 per-channel sweep (T = 1, 16,
256, 4096) -- each with tokens/s, its step's fraction of the binding roofline (HBM or the
path's MFMA peak, whichever bounds its algorithmic bytes and flops) and the stage-1 kernel
time from events on one more step.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused-MoE layer tokens/s; % HBM peak (decode) / % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
MALL_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")


def _hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


def _event(hip):
    e = ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(e)) == 0
    return e.value


def _elapsed_ms(hip, a, b) -> float:
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
    return ms.value


def algorithmic(w, ids_np):
    """Algorithmic bytes and flops of one step and of its stage-1 GEMM launch.
    Weights count once per expert that at least one slot uses; rows are the routed
    slots (pad rows are overhead, not work)."""
    import numpy as np

    from quantized_mixture_experts_softmax_amd import synth

    hit = np.unique(ids_np[(ids_np >= 0) & (ids_np < w.E_total)])
    n_hit = len(hit)
    slots = int(np.count_nonzero((ids_np >= 0) & (ids_np < w.E_total)))
    if w.wfmt == synth.W_MXFP4:
        w1_per = 2 * w.I * (w.H // 2 + w.H // 32)
        w2_per = w.H * (w.I // 2 + w.I // 32)
    elif w.wfmt == synth.W_BF16:
        w1_per = 2 * w.I * w.H * 2
        w2_per = w.H * w.I * 2
    elif w.wfmt == synth.W_FP8_BLOCK128:
        w1_per = 2 * w.I * w.H + 4 * ((2 * w.I + 127) // 128) * ((w.H + 127) // 128)
        w2_per = w.H * w.I + 4 * ((w.H + 127) // 128) * ((w.I + 127) // 128)
    else:
        w1_per = 2 * w.I * w.H + 4 * 2 * w.I
        w2_per = w.H * w.I + 4 * w.H
    x_bytes = w.T * w.H * 2
    out_bytes = w.T * w.H * 2
    h_bytes = slots * w.I * 2
    step_bytes = n_hit * (w1_per + w2_per) + x_bytes + out_bytes
    gemm1_bytes = n_hit * w1_per + x_bytes + h_bytes
    gemm1_flops = 2.0 * slots * w.H * 2 * w.I
    step_flops = 6.0 * slots * w.H * w.I
    return dict(n_hit=n_hit, slots=slots, step_bytes=step_bytes, gemm1_bytes=gemm1_bytes, gemm1_flops=gemm1_flops,
                step_flops=step_flops)


def mfma_dtype(w):
    from quantized_mixture_experts_softmax_amd import synth

    if w.wfmt == synth.W_MXFP4:
        return "fp4" if w.afmt == synth.A_MXFP4_G32 else "bf16"
    if w.wfmt == synth.W_BF16:
        return "bf16"
    return "fp8"


# Sources compiled into the grouped-GEMM kernels (the route + sort fused into stage 1
# comes from sort_device.h, which includes route_device.h): a counter summary is current
# only for these bytes.
GEMM_SOURCES = ("experts_gemm.hip", "gemm_lds.hip", "gemm_common.h", "moe_device.h", "moe_internal.h", "sort_device.h",
                "route_device.h")


def gemm_source_sha() -> str:
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, "quantized_mixture_experts_softmax_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload_name: str):
    """HBM bytes per stage-1 launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(PROFILES, f"gemm1_{workload_name}_pmc.txt")
    if not os.path.exists(path):
        return None
    sha = gemm_source_sha()
    vals = {}
    for line in open(path):
        if "=" in line and line.strip().startswith("TRAFFIC_"):
            k, v = line.strip().split("=", 1)
            vals[k] = v.strip()
    if vals.get("TRAFFIC_SOURCE_SHA") != sha or "TRAFFIC_BYTES_PER_LAUNCH" not in vals:
        return None
    return float(vals["TRAFFIC_BYTES_PER_LAUNCH"])


def cpu_baseline(w, data, seconds: float, act_host: dict | None = None, emap=None):
    """The oracle, as it stands, on a bounded sample of the same workload (rank 0, N=1).
    act_host: SwiGLU-OAI settings and host bias arrays when the layer uses them; emap: the
    expert map of an expert-parallel share (data then holds the local experts only)."""
    import numpy as np

    from oracle import oracle as orc

    ids, wts = orc.route_topk(data["logits"], w.topk, w.score, True, w.n_shared, w.shared_weight)
    E_loc = w.E_total
    if emap is not None:
        ids = orc.map_experts(ids, emap, w.E_total)
        E_loc = int(emap.max()) + 1
    L = orc.Layer(w.H, w.I, E_loc, w.K, w.wfmt, w.afmt, data["w1"], data["w1_scale"], data["w2"],
                  data["w2_scale"], **(act_host or {}))
    per_call = max(1, min(w.T, 64))
    done, t0, start = 0, time.perf_counter(), 0
    while True:
        tk = (np.arange(per_call) + start) % w.T
        orc.forward(L, data["x"], ids, wts, tk.astype(np.int32))
        done += per_call
        start += per_call
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"{done} tokens of the {w.name} workload ({per_call} per call), oracle forward "
                      f"(fp64 per-token loop, OpenMP), {el:.1f} s"}


WFMT_NAMES = ["mxfp4", "fp8-block128", "fp8-channel", "fp8-tensor", "bf16"]
AFMT_NAMES = ["w4a16", "a-mxfp4", "a-fp8-g128", "a-fp8-token", "a-fp8-tensor"]


def workload_label(w) -> str:
    from quantized_mixture_experts_softmax_amd import synth

    a = "a-bf16" if w.wfmt == synth.W_BF16 else AFMT_NAMES[w.afmt]
    return f"{w.name}-{WFMT_NAMES[w.wfmt]}-{a}"


def stage1_roofline(w, alg, g1_ms: float, profile_name: str, launches: int) -> dict:
    """The stage-1 GEMM (the dominant kernel) against its binding roof: algorithmic bytes per
    launch at HBM peak or algorithmic flops at the path's MFMA peak, whichever takes longer,
    divided by the launch's event-timed duration; traffic from the committed counter summary of
    this workload when it was taken on the current kernel sources (else null)."""
    dt = mfma_dtype(w)
    t_hbm = alg["gemm1_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = alg["gemm1_flops"] / (MFMA_PEAK_TFLOPS[dt] * 1e12)
    if t_hbm >= t_mfma:
        achieved = alg["gemm1_bytes"] / (g1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = alg["gemm1_flops"] / (g1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS[dt], "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_PEAK_TFLOPS[dt], 4)}
    roof["traffic"] = traffic_from_profiles(profile_name)
    roof["alg_bytes_per_launch"] = alg["gemm1_bytes"]
    roof["alg_flops_per_launch"] = alg["gemm1_flops"]
    roof["avg_launch_us"] = round(g1_ms * 1e3, 2)
    roof["launches_timed"] = launches
    return roof


def step_roofline(w, alg, ms: float) -> dict:
    """The step's fraction of its binding roofline: algorithmic bytes at HBM peak against
    algorithmic flops at the path's MFMA peak, whichever takes longer."""
    dt = mfma_dtype(w)
    t_hbm = alg["step_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = alg["step_flops"] / (MFMA_PEAK_TFLOPS[dt] * 1e12)
    s = ms * 1e-3
    return {"bound": "hbm" if t_hbm >= t_mfma else f"mfma-{dt}", "frac": round(max(t_hbm, t_mfma) / s, 4),
            "hbm_frac": round(t_hbm / s, 4), "mfma_frac": round(t_mfma / s, 4),
            "achieved_gbs": round(alg["step_bytes"] / s / 1e9, 1), "achieved_tflops": round(alg["step_flops"] / s / 1e12, 1)}


# (workload, token count) of the extra bench entries; the fp8-channel sweep takes prefixes
# of one T = 4096 draw
EXTRA_CONFIGS = [("prefill", None), ("prefill-w4a4", None), ("fp8-block", None), ("fp8-channel", 1),
                 ("fp8-channel", 16), ("fp8-channel", 256), ("fp8-channel", 4096)]


def measure_extra(steps: int, warmup: int, hip, dev) -> dict:
    """Times each EXTRA_CONFIGS workload: tiled weights (rotated copies when one copy is
    smaller than twice the Infinity Cache), plain top-k routing through MoELayer, `warmup`
    untimed steps, `steps` timed steps between HIP events on the launch stream and wall
    clock, then one step with the per-stage events."""
    import numpy as np
    import torch

    from quantized_mixture_experts_softmax_amd import binding as B
    from quantized_mixture_experts_softmax_amd import synth

    out = {}
    cache = {}
    for name, T in EXTRA_CONFIGS:
        w0 = synth.WORKLOADS[name]
        if name not in cache:
            cache.clear()
            cache[name] = synth.make_all(w0)
        full = cache[name]
        w = w0.with_T(T) if T else w0
        data = dict(full, x=full["x"][:w.T], logits=full["logits"][:w.T])
        wbytes = sum(data[k].nbytes for k in ("w1", "w1_scale", "w2", "w2_scale") if data[k] is not None)
        copies = 1 if wbytes >= 2 * MALL_BYTES else min(64, -(-2 * MALL_BYTES // wbytes) + 1)
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        layers = [B.MoELayer(t(data["w1"]), t(data["w1_scale"]), t(data["w2"]), t(data["w2_scale"]), H=w.H, I=w.I,
                             E=w.E, topk=w.topk, wfmt=w.wfmt, afmt=w.afmt,
                             score="softmax" if w.score == synth.SCORE_SOFTMAX else "sigmoid", n_shared=w.n_shared,
                             shared_weight=w.shared_weight, tiled=True) for _ in range(copies)]
        x = torch.from_numpy(np.ascontiguousarray(data["x"]).view(np.int16)).view(torch.bfloat16).to(dev)
        logits = t(data["logits"])
        for i in range(warmup):
            layers[i % copies](x, logits)
        stream = torch.cuda.current_stream(dev).cuda_stream
        e0, e1 = _event(hip), _event(hip)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        hip.hipEventRecord(ctypes.c_void_p(e0), ctypes.c_void_p(stream))
        for i in range(steps):
            layers[i % copies](x, logits)
        hip.hipEventRecord(ctypes.c_void_p(e1), ctypes.c_void_p(stream))
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        gpu_ms = _elapsed_ms(hip, e0, e1) / steps
        # per-stage events on three more steps (each record adds a few microseconds)
        evs = [[_event(hip) for _ in range(4)] for _ in range(3)]
        for i, ev in enumerate(evs):
            B.moe_profile_events(ev)
            layers[i % copies](x, logits)
            B.moe_profile_events(None)
        torch.cuda.synchronize()
        ev = evs[-1]
        g1 = sum(_elapsed_ms(hip, e[0], e[1]) for e in evs) / len(evs)
        b = layers[0]._bufs[(w.T, str(dev))]
        alg = algorithmic(w, b["ids"].cpu().numpy())
        label = workload_label(w) + (f"-T{w.T}" if T else "")
        out[label] = {
            "T": w.T, "steps": steps, "ms_per_step": round(wall_ms, 5), "gpu_ms_per_step": round(gpu_ms, 5),
            "tokens_per_s": round(w.T / (wall_ms * 1e-3), 1), "block_m": b["bm"], "weight_copies": copies,
            "experts_hit": alg["n_hit"], "roofline": step_roofline(w, alg, wall_ms),
            "stage1_roofline": stage1_roofline(w, alg, g1, w.name + (f"-T{w.T}" if T else ""), len(evs)),
            "stage_us": {"stage1_gemm": round(g1 * 1e3, 2),
                         "a2_quant+stage2_gemm": round(_elapsed_ms(hip, ev[1], ev[2]) * 1e3, 2),
                         "combine": round(_elapsed_ms(hip, ev[2], ev[3]) * 1e3, 2)},
        }
        del layers, x, logits, b
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        print(f"bench.py: {label}: {wall_ms:.4f} ms/step, {out[label]['roofline']['frac']:.3f} of the "
              f"{out[label]['roofline']['bound']} roof", file=sys.stderr, flush=True)
    return out


def main() -> int:
    from quantized_mixture_experts_softmax_amd import synth

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--tokens", type=int, default=None, help="token count (fp8-channel sweep: 1, 16, 256, 4096)")
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--weight-copies", type=int, default=None)
    ap.add_argument("--layout", choices=["tiled", "canonical"], default=None,
                    help="weight layout: the kernel layout prepared once by moe_tile_weights, or canonical")
    ap.add_argument("--router", choices=["plain", "grouped"], default="plain",
                    help="grouped: group-limited router (8 groups, 4 kept, seeded correction bias, scaling 2.5)")
    ap.add_argument("--act", choices=["silu", "swiglu-oai"], default="silu",
                    help="swiglu-oai: SwiGLU-OAI (alpha 1.702, beta 1, limit 7) with interleaved gate/up rows and "
                         "seeded bf16 biases on both projections (the gpt-oss layer form)")
    ap.add_argument("--ep-share", type=int, default=1,
                    help="G > 1: time device 0's share of an expert-parallel layer over G devices (experts "
                         "[0, E/G) plus the replicated shared experts; all T tokens routed globally)")
    ap.add_argument("--route", choices=["fused", "separate"], default="fused",
                    help="fused: moe_layer_forward (small batches routed inside stage 1); separate: "
                         "moe_route_align, then moe_experts_forward")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=10,
                    help="record the per-stage HIP events on every n-th timed step (each record adds a few us)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--extra", choices=["all", "none"], default="all",
                    help="all: also time the prefill-sized workloads and the fp8-channel sweep (extra_configs)")
    ap.add_argument("--extra-steps", type=int, default=30)
    ap.add_argument("--extra-warmup", type=int, default=5)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU; the sharded multi-GPU (expert / tensor parallel) path is not "
              "implemented. Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from quantized_mixture_experts_softmax_amd import binding as B

    if not os.path.exists(B.LIB_PATH):
        from quantized_mixture_experts_softmax_amd import build as hip_build

        hip_build.build()
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    if args.tokens:
        w = w.with_T(args.tokens)
    data = synth.make_all(w)
    wbytes = sum(data[k].nbytes for k in ("w1", "w1_scale", "w2", "w2_scale") if data[k] is not None)
    # enough copies that one rotation is larger than twice the Infinity Cache
    copies = args.weight_copies or (1 if wbytes >= 2 * MALL_BYTES else min(64, -(-2 * MALL_BYTES // wbytes) + 1))
    def t(a):  # host array -> device tensor (bf16 bit arrays as bf16; absent scales stay None)
        if a is None:
            return None
        a = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a))
        return (a.view(torch.bfloat16) if a.dtype == torch.int16 else a).to(dev)

    if args.layout is None:
        args.layout = "canonical" if w.wfmt == synth.W_BF16 else "tiled"
    if w.wfmt == synth.W_BF16 and (args.layout == "tiled" or args.block_m == 32):
        print("bench.py: bf16 weights run on the canonical layout with 16-, 64- or 128-row blocks", file=sys.stderr)
        return 2
    grouped = None
    if args.router == "grouped":
        if w.E % 8:
            print("bench.py: --router grouped needs the expert count to split into 8 groups", file=sys.stderr)
            return 2
        grouped = dict(num_expert_group=8, topk_group=4, routed_scaling_factor=2.5,
                       correction_bias=t(synth.make_correction_bias(w)))
    act = act_host = None
    if args.act == "swiglu-oai":
        if w.wfmt == synth.W_FP8_BLOCK128:
            print("bench.py: --act swiglu-oai interleaves w13 rows, which FP8 128x128 block scales do not allow",
                  file=sys.stderr)
            return 2
        b1, b2 = synth.make_biases(w)
        data = dict(data, w1=synth.interleave_rows(data["w1"], w.I),
                    w1_scale=None if data["w1_scale"] is None else synth.interleave_rows(data["w1_scale"], w.I))
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(dev)
        act = dict(kind=B.ACT_SWIGLU_OAI, alpha=1.702, beta=1.0, limit=7.0, interleaved=True,
                   w1_bias=bf(synth.interleave_rows(b1, w.I)), w2_bias=bf(b2))
        act_host = dict(act=1, alpha=1.702, beta=1.0, limit=7.0, gate_up_interleaved=True,
                        w1_bias=synth.interleave_rows(b1, w.I), w2_bias=b2)
    emap = None
    if args.ep_share > 1:
        G = args.ep_share
        if w.E % G:
            print(f"bench.py: --ep-share {G} needs the expert count to split into {G} shares", file=sys.stderr)
            return 2
        mine = np.concatenate([np.arange(w.E // G), w.E + np.arange(w.n_shared)])
        m = np.full(w.E_total, -1, np.int32)
        m[mine] = np.arange(len(mine), dtype=np.int32)
        emap = torch.from_numpy(m).to(dev)
        data = dict(data, **{k: np.ascontiguousarray(data[k][mine]) for k in ("w1", "w1_scale", "w2", "w2_scale")
                             if data[k] is not None})
        wbytes = sum(data[k].nbytes for k in ("w1", "w1_scale", "w2", "w2_scale") if data[k] is not None)
        copies = args.weight_copies or (1 if wbytes >= 2 * MALL_BYTES else min(64, -(-2 * MALL_BYTES // wbytes) + 1))
    layers = []
    for _ in range(copies):
        layers.append(B.MoELayer(t(data["w1"]), t(data["w1_scale"]), t(data["w2"]), t(data["w2_scale"]), H=w.H,
                                 I=w.I, E=w.E, topk=w.topk, wfmt=w.wfmt, afmt=w.afmt,
                                 score="softmax" if w.score == synth.SCORE_SOFTMAX else "sigmoid",
                                 n_shared=w.n_shared, shared_weight=w.shared_weight, block_m=args.block_m,
                                 fuse_route=args.route == "fused",
                                 tiled=args.layout == "tiled", grouped=grouped, act=act, expert_map=emap))
    x = torch.from_numpy(data["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    logits = t(data["logits"])
    hip = _hip()

    for i in range(args.warmup):
        layers[i % copies](x, logits)
    torch.cuda.synchronize()
    every = max(1, args.event_every)
    sampled = [s for s in range(args.steps) if s % every == every - 1] or [args.steps - 1]
    evs = {s: [_event(hip) for _ in range(4)] for s in sampled}
    ev_start, ev_stop = _event(hip), _event(hip)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev).cuda_stream
    t0 = time.perf_counter()
    hip.hipEventRecord(ctypes.c_void_p(ev_start), ctypes.c_void_p(stream))
    for s in range(args.steps):
        if s in evs:
            B.moe_profile_events(evs[s])
        layers[s % copies](x, logits)
        if s in evs:
            B.moe_profile_events(None)
    hip.hipEventRecord(ctypes.c_void_p(ev_stop), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = list(evs.values())
    gpu_ms = _elapsed_ms(hip, ev_start, ev_stop)
    g1 = [_elapsed_ms(hip, e[0], e[1]) for e in evs]
    g2 = [_elapsed_ms(hip, e[1], e[2]) for e in evs]
    cb = [_elapsed_ms(hip, e[2], e[3]) for e in evs]

    ms_per_step = wall * 1e3 / args.steps
    b = layers[0]._bufs[(w.T, str(dev))]
    ids_np = b["ids"].cpu().numpy()
    alg = algorithmic(w, ids_np)
    g1_ms = float(np.mean(g1))
    dt = mfma_dtype(w)
    roof = stage1_roofline(w, alg, g1_ms, w.name if not args.tokens else f"{w.name}-T{w.T}", len(evs))
    roof["kernel"] = ("stage-1 grouped GEMM (gate/up + SiLU-and-mul): "
                      + ("moe_gemm_persist_kernel" if b["bm"] == 16 else
                         "moe_gemm_ksplit_kernel" if b["bm"] == 32 else
                         "moe_gemm_lds_kernel" if b["bm"] == 128 and args.layout == "tiled" else "moe_gemm_kernel"))

    result = {
        "metric": METRIC,
        "value": round(w.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded; random weight codes and scales, no checkpoint)",
        "config": {"workload": workload_label(w),
                   "T": w.T, "H": w.H, "I": w.I, "experts": w.E, "shared_experts": w.n_shared, "topk": w.topk,
                   "router": "softmax" if w.score == synth.SCORE_SOFTMAX else "sigmoid",
                   "block_m": b["bm"], "weight_copies": copies, "experts_hit": alg["n_hit"],
                   "weight_layout": args.layout,
                   "router_kind": "grouped (8 groups, 4 kept, bias, scaling 2.5)" if grouped else "plain top-k",
                   "route_path": args.route,
                   "activation": "swiglu-oai, interleaved w13, biases" if act else "silu-and-mul",
                   "ep_share": (f"device 0 of EP{args.ep_share}: {w.E // args.ep_share} routed + {w.n_shared} "
                                f"shared experts; value = T / this device's step time") if emap is not None else None},
        "roofline": roof,
        "step_breakdown_us": {"gpu_step": round(gpu_ms * 1e3 / args.steps, 2),
                              "stage1_gemm": round(g1_ms * 1e3, 2), "a2_quant+stage2_gemm": round(float(np.mean(g2)) * 1e3, 2),
                              "combine": round(float(np.mean(cb)) * 1e3, 2)},
        "step_roofline": {"alg_bytes": alg["step_bytes"], "alg_flops": alg["step_flops"],
                          "hbm_frac": round(alg["step_bytes"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "mfma_frac": round(alg["step_flops"] / (ms_per_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[dt], 4)},
    }
    if args.calib_copy_mb:
        n = args.calib_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = n
    if args.extra == "all":
        del layers
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["extra_configs"] = measure_extra(args.extra_steps, args.extra_warmup, hip, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, data, args.cpu_seconds, act_host,
                                              None if emap is None else emap.cpu().numpy())
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
