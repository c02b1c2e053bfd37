"""Python binding of libmoe (include/moe.h): argument marshalling only.

Every computation runs in the HIP library; this module allocates outputs and the
workspace with torch on the tensors' device and passes raw device pointers and the
current HIP stream.  If libmoe.so is missing or cannot be loaded, every entry point
raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, 1, 2, 3, 4
SCORE = {"softmax": 0, "sigmoid": 1}
W_MXFP4, W_FP8_BLOCK128, W_FP8_CHANNEL, W_FP8_TENSOR, W_BF16 = 0, 1, 2, 3, 4
# bf16 weights on 16-row blocks: the persistent kernel's activation tile (16 x K bf16) must fit
# its LDS, i.e. at most 23 chunks of 128 (moe_experts_forward refuses larger H or I there)
BF16_SMALL_BLOCK_MAX_K = 2944
A_BF16, A_MXFP4_G32, A_FP8_G128, A_FP8_TOKEN, A_FP8_TENSOR = 0, 1, 2, 3, 4
ACT_SILU, ACT_SWIGLU_OAI = 0, 1

EXPORTED = [
    "moe_route_topk", "moe_route_grouped_topk", "moe_map_experts", "moe_sort_capacity", "moe_align_sort", "moe_route_align", "moe_quant_act",
    "moe_experts_workspace_bytes", "moe_workspace_layout", "moe_experts_forward", "moe_layer_forward",
    "moe_supports", "moe_pick_block_m", "moe_profile_events", "moe_last_error",
    "moe_tiled_weight_bytes", "moe_tile_weights", "moe_experts_forward_noalloc", "moe_set_checked_mode",
]
# library-owned workspace of moe_experts_forward_noalloc (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20
LAYOUT_CANONICAL, LAYOUT_TILED = 0, 1


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libmoe status {status}: {msg}")
        self.status = status


class ForwardArgs(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int), ("E_total", ctypes.c_int),
        ("K", ctypes.c_int), ("block_m", ctypes.c_int),
        ("wfmt", ctypes.c_int), ("afmt", ctypes.c_int), ("act", ctypes.c_int),
        ("hidden_states", ctypes.c_void_p),
        ("a1_codes", ctypes.c_void_p), ("a1_scales", ctypes.c_void_p),
        ("w1", ctypes.c_void_p), ("w1_scale", ctypes.c_void_p),
        ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
        ("topk_ids", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p),
        ("sorted_slots", ctypes.c_void_p), ("block_expert", ctypes.c_void_p), ("num_padded", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("weight_layout", ctypes.c_int),
        ("act_alpha", ctypes.c_float), ("act_beta", ctypes.c_float), ("act_limit", ctypes.c_float),
        ("gate_up_interleaved", ctypes.c_int),
        ("w1_bias", ctypes.c_void_p), ("w2_bias", ctypes.c_void_p),
        ("apply_router_weight_on_input", ctypes.c_int),
    ]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "h_off", "h_bytes", "a1_codes_off", "a1_codes_bytes", "a1_scales_off", "a1_scales_bytes",
        "a2_codes_off", "a2_codes_bytes", "a2_scales_off", "a2_scales_bytes", "ybuf_off", "ybuf_bytes", "total")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so; raises if it is not built.  There is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmoe.so not found at {LIB_PATH}; run "
                               "`python -m quantized_mixture_experts_softmax_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_int
        L.moe_route_topk.restype = S
        L.moe_route_topk.argtypes = [P, I, I, I, I, I, I, ctypes.c_float, P, P, P]
        L.moe_map_experts.restype = S
        L.moe_map_experts.argtypes = [P, P, P, I, I, I, P, P]
        L.moe_route_grouped_topk.restype = S
        L.moe_route_grouped_topk.argtypes = [P, P, I, I, I, I, I, I, I, ctypes.c_float, I, ctypes.c_float, P, P, P]
        L.moe_sort_capacity.restype = ctypes.c_size_t
        L.moe_sort_capacity.argtypes = [I, I, I, I]
        L.moe_align_sort.restype = S
        L.moe_align_sort.argtypes = [P, I, I, I, I, P, P, P, P, P, P]
        L.moe_route_align.restype = S
        L.moe_route_align.argtypes = [P, I, I, I, I, I, I, ctypes.c_float, I, P, P, P, P, P, P, P, P]
        L.moe_quant_act.restype = S
        L.moe_quant_act.argtypes = [P, I, I, I, P, P, P]
        L.moe_experts_workspace_bytes.restype = ctypes.c_size_t
        L.moe_experts_workspace_bytes.argtypes = [ctypes.POINTER(ForwardArgs)]
        L.moe_workspace_layout.restype = S
        L.moe_workspace_layout.argtypes = [ctypes.POINTER(ForwardArgs), ctypes.POINTER(WorkspaceLayout)]
        L.moe_experts_forward.restype = S
        L.moe_experts_forward.argtypes = [ctypes.POINTER(ForwardArgs), P]
        L.moe_experts_forward_noalloc.restype = S
        L.moe_experts_forward_noalloc.argtypes = [ctypes.POINTER(ForwardArgs), P]
        L.moe_layer_forward.restype = S
        L.moe_layer_forward.argtypes = [ctypes.POINTER(ForwardArgs), P, I, I, I, ctypes.c_float, P, P, P]
        L.moe_supports.restype = S
        L.moe_supports.argtypes = [I, I, I, I, I]
        L.moe_pick_block_m.restype = I
        L.moe_pick_block_m.argtypes = [I, I, I, I, I]
        L.moe_profile_events.restype = S
        L.moe_profile_events.argtypes = [P, I]
        L.moe_set_checked_mode.restype = S
        L.moe_set_checked_mode.argtypes = [I]
        L.moe_tiled_weight_bytes.restype = ctypes.c_size_t
        L.moe_tiled_weight_bytes.argtypes = [I, I, I, I]
        L.moe_tile_weights.restype = S
        L.moe_tile_weights.argtypes = [I, I, I, I, P, P, P, P]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        _lib = L
    return _lib


def _check(st: int) -> None:
    if st != MOE_OK:
        raise MoeError(st, lib().moe_last_error().decode())


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("libmoe tensors must be contiguous")
    return t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _dev(t: torch.Tensor) -> torch.device:
    if t.device.type != "cuda":
        raise ValueError("libmoe tensors must live on the GPU")
    return t.device


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_set_checked_mode(on: bool) -> None:
    """Forward calls verify caller-built routing tables on the device first (see moe.h)."""
    _check(lib().moe_set_checked_mode(1 if on else 0))


def moe_profile_events(events: list | None) -> None:
    """Enable (4 raw hipEvent_t handles) or disable (None) the stage-boundary events."""
    if not events:
        _check(lib().moe_profile_events(None, 0))
        return
    arr = (ctypes.c_void_p * 4)(*events)
    _check(lib().moe_profile_events(arr, 4))


def moe_tile_weights(w: torch.Tensor, w_scale: torch.Tensor | None, wfmt: int, K: int, stream=None) -> torch.Tensor:
    """Tiled (kernel-layout) copy of one [E, N, K] weight tensor; see include/moe.h."""
    dev = _dev(w)
    E, N = w.shape[0], w.shape[1]
    n = lib().moe_tiled_weight_bytes(wfmt, E, N, K)
    if n == 0:
        raise ValueError("moe_tiled_weight_bytes: unsupported shape")
    out = torch.empty(n, dtype=torch.uint8, device=dev)
    _check(lib().moe_tile_weights(wfmt, E, N, K, _ptr(w), _ptr(w_scale) if wfmt == W_MXFP4 else None, _ptr(out),
                                  _stream(stream, dev)))
    return out


def moe_supports(wfmt: int, afmt: int, H: int, I: int, act: int = ACT_SILU) -> bool:
    return lib().moe_supports(wfmt, afmt, act, H, I) == MOE_OK


def moe_pick_block_m(T: int, K: int, E_total: int, wfmt: int = W_MXFP4, layout: int = LAYOUT_CANONICAL) -> int:
    return lib().moe_pick_block_m(T, K, E_total, wfmt, layout)


def moe_sort_capacity(T: int, K: int, E_total: int, block_m: int) -> int:
    return lib().moe_sort_capacity(T, K, E_total, block_m)


def moe_route_topk(router_logits: torch.Tensor, topk: int, score: str = "softmax", renormalize: bool = True,
                   n_shared: int = 0, shared_weight: float = 1.0, topk_ids=None, topk_weights=None, stream=None):
    dev = _dev(router_logits)
    assert router_logits.dtype == torch.float32 and router_logits.dim() == 2
    T, E = router_logits.shape
    KP = topk + n_shared
    if topk_ids is None:
        topk_ids = torch.empty((T, KP), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, KP), dtype=torch.float32, device=dev)
    _check(lib().moe_route_topk(_ptr(router_logits), T, E, topk, SCORE[score], int(renormalize), n_shared,
                                shared_weight, _ptr(topk_ids), _ptr(topk_weights), _stream(stream, dev)))
    return topk_ids, topk_weights


def moe_route_grouped_topk(router_logits: torch.Tensor, topk: int, num_expert_group: int, topk_group: int,
                           correction_bias: torch.Tensor | None = None, score: str = "sigmoid",
                           renormalize: bool = True, routed_scaling_factor: float = 1.0, n_shared: int = 0,
                           shared_weight: float = 1.0, topk_ids=None, topk_weights=None, stream=None):
    dev = _dev(router_logits)
    assert router_logits.dtype == torch.float32 and router_logits.dim() == 2
    T, E = router_logits.shape
    if correction_bias is not None:
        assert correction_bias.dtype == torch.float32 and correction_bias.numel() == E
        _dev(correction_bias)
    KP = topk + n_shared
    if topk_ids is None:
        topk_ids = torch.empty((T, KP), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, KP), dtype=torch.float32, device=dev)
    _check(lib().moe_route_grouped_topk(_ptr(router_logits), _ptr(correction_bias), T, E, topk, num_expert_group,
                                        topk_group, SCORE[score], int(renormalize), routed_scaling_factor, n_shared,
                                        shared_weight, _ptr(topk_ids), _ptr(topk_weights), _stream(stream, dev)))
    return topk_ids, topk_weights


def moe_map_experts(topk_ids: torch.Tensor, expert_map: torch.Tensor | None, E_global: int,
                    num_local_tokens: torch.Tensor | None = None, out=None, stream=None) -> torch.Tensor:
    """Local ids of this device's expert-parallel share (-1: not here)."""
    dev = _dev(topk_ids)
    assert topk_ids.dtype == torch.int32 and topk_ids.dim() == 2
    for t in (expert_map, num_local_tokens):
        if t is not None:
            assert t.dtype == torch.int32
            _dev(t)
    T, K = topk_ids.shape
    if out is None:
        out = torch.empty((T, K), dtype=torch.int32, device=dev)
    _check(lib().moe_map_experts(_ptr(topk_ids), _ptr(expert_map), _ptr(num_local_tokens), T, K, E_global,
                                 _ptr(out), _stream(stream, dev)))
    return out


def moe_align_sort(topk_ids: torch.Tensor, E_total: int, block_m: int, out: dict | None = None, stream=None) -> dict:
    dev = _dev(topk_ids)
    assert topk_ids.dtype == torch.int32 and topk_ids.dim() == 2
    T, K = topk_ids.shape
    cap = moe_sort_capacity(T, K, E_total, block_m)
    if out is None:
        out = dict(
            expert_counts=torch.empty(E_total, dtype=torch.int32, device=dev),
            expert_offsets=torch.empty(E_total + 1, dtype=torch.int32, device=dev),
            sorted_slots=torch.empty(cap, dtype=torch.int32, device=dev),
            block_expert=torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev),
            num_padded=torch.empty(1, dtype=torch.int32, device=dev),
        )
    _check(lib().moe_align_sort(_ptr(topk_ids), T, K, E_total, block_m, _ptr(out["expert_counts"]),
                                _ptr(out["expert_offsets"]), _ptr(out["sorted_slots"]), _ptr(out["block_expert"]),
                                _ptr(out["num_padded"]), _stream(stream, dev)))
    return out


def moe_route_align(router_logits: torch.Tensor, topk: int, block_m: int, score: str = "softmax",
                    renormalize: bool = True, n_shared: int = 0, shared_weight: float = 1.0, topk_ids=None,
                    topk_weights=None, out: dict | None = None, stream=None):
    """moe_route_topk then moe_align_sort in one call (one launch for small batches);
    returns (topk_ids, topk_weights, sort dict as moe_align_sort)."""
    dev = _dev(router_logits)
    assert router_logits.dtype == torch.float32 and router_logits.dim() == 2
    T, E = router_logits.shape
    K, E_total = topk + n_shared, E + n_shared
    if topk_ids is None:
        topk_ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, K), dtype=torch.float32, device=dev)
    if out is None:
        cap = moe_sort_capacity(T, K, E_total, block_m)
        out = dict(
            expert_counts=torch.empty(E_total, dtype=torch.int32, device=dev),
            expert_offsets=torch.empty(E_total + 1, dtype=torch.int32, device=dev),
            sorted_slots=torch.empty(cap, dtype=torch.int32, device=dev),
            block_expert=torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev),
            num_padded=torch.empty(1, dtype=torch.int32, device=dev),
        )
    _check(lib().moe_route_align(_ptr(router_logits), T, E, topk, SCORE[score], int(renormalize), n_shared,
                                 shared_weight, block_m, _ptr(topk_ids), _ptr(topk_weights),
                                 _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]), _ptr(out["sorted_slots"]),
                                 _ptr(out["block_expert"]), _ptr(out["num_padded"]), _stream(stream, dev)))
    return topk_ids, topk_weights, out


def quant_shapes(fmt: int, rows: int, cols: int):
    if fmt == A_MXFP4_G32:
        return (rows, cols // 2), (rows, cols // 32), torch.uint8
    if fmt == A_FP8_G128:
        return (rows, cols), (rows, (cols + 127) // 128), torch.float32
    if fmt == A_FP8_TOKEN:
        return (rows, cols), (rows,), torch.float32
    if fmt == A_FP8_TENSOR:
        return (rows, cols), (1,), torch.float32
    raise ValueError("bf16 activations have no quantiser")


def moe_quant_act(x: torch.Tensor, fmt: int, codes=None, scales=None, stream=None):
    dev = _dev(x)
    assert x.dtype == torch.bfloat16 and x.dim() == 2
    rows, cols = x.shape
    cs, ss, sdt = quant_shapes(fmt, rows, cols)
    if codes is None:
        codes = torch.empty(cs, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(ss, dtype=sdt, device=dev)
    _check(lib().moe_quant_act(_ptr(x), rows, cols, fmt, _ptr(codes), _ptr(scales), _stream(stream, dev)))
    return codes, scales


def forward_args(hidden_states, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sort: dict, wfmt: int,
                 afmt: int, block_m: int, E_total: int, I: int, out=None, workspace=None, a1_codes=None,
                 a1_scales=None, weight_layout: int = LAYOUT_CANONICAL, act: dict | None = None) -> ForwardArgs:
    """act: None (SiLU-and-mul) or dict(kind=ACT_SILU | ACT_SWIGLU_OAI, alpha, beta, limit,
    interleaved, w1_bias, w2_bias, weight_on_input) -- biases are bf16 tensors [E, 2I] /
    [E, H] or None; weight_on_input puts the top-1 weight on the stage-1 projections."""
    T, H = hidden_states.shape
    K = topk_ids.shape[1]
    a = ForwardArgs()
    a.T, a.H, a.I, a.E_total, a.K, a.block_m = T, H, I, E_total, K, block_m
    act = act or {}
    a.wfmt, a.afmt, a.act = wfmt, afmt, act.get("kind", ACT_SILU)
    a.act_alpha, a.act_beta, a.act_limit = act.get("alpha", 1.702), act.get("beta", 1.0), act.get("limit", 7.0)
    a.gate_up_interleaved = int(bool(act.get("interleaved", False)))
    a.apply_router_weight_on_input = int(bool(act.get("weight_on_input", False)))
    for name, n in (("w1_bias", 2 * I), ("w2_bias", H)):
        b = act.get(name)
        if b is not None:
            assert b.dtype == torch.bfloat16 and b.shape == (E_total, n), (name, b.shape)
            _dev(b)
        setattr(a, name, _ptr(b))
    a.hidden_states = _ptr(hidden_states)
    a.a1_codes, a.a1_scales = _ptr(a1_codes), _ptr(a1_scales)
    a.w1, a.w1_scale, a.w2, a.w2_scale = _ptr(w1), _ptr(w1_scale), _ptr(w2), _ptr(w2_scale)
    a.topk_ids, a.topk_weights = _ptr(topk_ids), _ptr(topk_weights)
    a.sorted_slots, a.block_expert, a.num_padded = (_ptr(sort["sorted_slots"]), _ptr(sort["block_expert"]),
                                                    _ptr(sort["num_padded"]))
    a.out = _ptr(out)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a.weight_layout = weight_layout
    return a


def moe_experts_workspace_bytes(args: ForwardArgs) -> int:
    n = lib().moe_experts_workspace_bytes(ctypes.byref(args))
    if n == 0:
        _check(lib().moe_workspace_layout(ctypes.byref(args), ctypes.byref(WorkspaceLayout())))
    return n


def moe_workspace_layout(args: ForwardArgs) -> dict:
    L = WorkspaceLayout()
    _check(lib().moe_workspace_layout(ctypes.byref(args), ctypes.byref(L)))
    return {n: getattr(L, n) for n, _ in WorkspaceLayout._fields_}


def moe_experts_forward(hidden_states, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sort: dict, wfmt: int,
                        afmt: int, block_m: int, E_total: int, I: int, out=None, workspace=None, a1_codes=None,
                        a1_scales=None, stream=None, weight_layout: int = LAYOUT_CANONICAL, act: dict | None = None):
    """Returns (out, workspace).  The workspace may be passed back in on later calls.
    act: see forward_args."""
    dev = _dev(hidden_states)
    assert hidden_states.dtype == torch.bfloat16
    T, H = hidden_states.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    args = forward_args(hidden_states, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sort, wfmt, afmt,
                        block_m, E_total, I, out, workspace, a1_codes, a1_scales, weight_layout, act)
    need = moe_experts_workspace_bytes(args)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel()
    _check(lib().moe_experts_forward(ctypes.byref(args), _stream(stream, dev)))
    return out, workspace


def moe_experts_forward_noalloc(hidden_states, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sort: dict,
                                wfmt: int, afmt: int, block_m: int, E_total: int, I: int, out=None, a1_codes=None,
                                a1_scales=None, stream=None, weight_layout: int = LAYOUT_CANONICAL,
                                act: dict | None = None):
    """moe_experts_forward with the workspace in the library's own scratch (no workspace
    argument; see include/moe.h).  Returns out."""
    dev = _dev(hidden_states)
    assert hidden_states.dtype == torch.bfloat16
    T, H = hidden_states.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    args = forward_args(hidden_states, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sort, wfmt, afmt,
                        block_m, E_total, I, out, None, a1_codes, a1_scales, weight_layout, act)
    _check(lib().moe_experts_forward_noalloc(ctypes.byref(args), _stream(stream, dev)))
    return out


def moe_layer_forward(hidden_states, router_logits, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sort: dict,
                      wfmt: int, afmt: int, block_m: int, E_total: int, I: int, score: str = "softmax",
                      renormalize: bool = True, n_shared: int = 0, shared_weight: float = 1.0, out=None,
                      workspace=None, a1_codes=None, a1_scales=None, stream=None,
                      weight_layout: int = LAYOUT_CANONICAL, act: dict | None = None):
    """Route + align-sort into topk_ids, topk_weights and sort (the moe_align_sort dict),
    then the expert layer, in one call; small batches are routed inside stage 1.
    Returns (out, workspace)."""
    dev = _dev(hidden_states)
    assert hidden_states.dtype == torch.bfloat16
    assert router_logits.dtype == torch.float32 and router_logits.dim() == 2
    T, H = hidden_states.shape
    assert router_logits.shape == (T, E_total - n_shared)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    args = forward_args(hidden_states, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sort, wfmt, afmt,
                        block_m, E_total, I, out, workspace, a1_codes, a1_scales, weight_layout, act)
    need = moe_experts_workspace_bytes(args)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel()
    _check(lib().moe_layer_forward(ctypes.byref(args), _ptr(router_logits), SCORE[score], int(renormalize), n_shared,
                                   shared_weight, _ptr(sort["expert_counts"]), _ptr(sort["expert_offsets"]),
                                   _stream(stream, dev)))
    return out, workspace


class MoELayer:
    """Device-resident weights of one quantised MoE expert layer and the full hot
    path: route + align-sort, optional a1 quantisation, experts forward (one
    moe_layer_forward call, or moe_route_align + moe_experts_forward with
    fuse_route=False).

    Every call returns a new output tensor.  The routing tables, a1 codes and the
    workspace are allocated on first use for a token count and reused by later calls with
    that count, so two calls on different streams must not overlap (the second would
    overwrite the first's intermediates); a call on a stream other than the current one
    records that stream on the reused buffers, so the caching allocator does not hand
    their memory out while its kernels may still run."""

    def __init__(self, w1, w1_scale, w2, w2_scale, *, H: int, I: int, E: int, topk: int, wfmt: int, afmt: int,
                 score: str = "softmax", n_shared: int = 0, shared_weight: float = 1.0, block_m: int | None = None,
                 tiled: bool = False, grouped: dict | None = None, act: dict | None = None,
                 expert_map: torch.Tensor | None = None, fuse_route: bool = True):
        """tiled=True re-lays the weights once into the kernel layout (moe_tile_weights).
        grouped = dict(num_expert_group, topk_group, correction_bias (tensor or None),
        routed_scaling_factor) routes with moe_route_grouped_topk (then moe_align_sort).
        act: activation, row order and biases, as for forward_args (None: SiLU-and-mul).
        expert_map (int32 [E + n_shared] global -> local id or -1): this device's share of an
        expert-parallel layer; the weights hold the local experts only, the router runs over
        the global experts and moe_map_experts turns its ids into local ones.
        fuse_route: plain top-k routing goes through moe_layer_forward (routing inside
        stage 1 where the batch allows); False keeps the separate calls."""
        self.E_local = w1.shape[0]
        if wfmt == W_BF16:
            if tiled:
                raise ValueError("MoELayer: unquantised bf16 weights take the canonical layout only (tiled=False)")
            if block_m == 32 or (block_m == 16 and max(H, I) > BF16_SMALL_BLOCK_MAX_K):
                raise ValueError(f"MoELayer: unquantised bf16 weights take block_m 16 (H, I <= "
                                 f"{BF16_SMALL_BLOCK_MAX_K}), 64 or 128 (got {block_m})")
        self.weight_layout = LAYOUT_TILED if tiled else LAYOUT_CANONICAL
        if tiled:
            w1 = moe_tile_weights(w1, w1_scale, wfmt, H)
            w2 = moe_tile_weights(w2, w2_scale, wfmt, I)
            if wfmt == W_MXFP4:
                w1_scale = w2_scale = None
        self.w1, self.w1_scale, self.w2, self.w2_scale = w1, w1_scale, w2, w2_scale
        self.H, self.I, self.E, self.topk = H, I, E, topk
        self.wfmt, self.afmt, self.score = wfmt, afmt, score
        self.n_shared, self.shared_weight = n_shared, shared_weight
        self.E_total = E + n_shared
        self.K = topk + n_shared
        self.block_m = block_m
        self.grouped = grouped
        self.act = act
        self.expert_map = expert_map
        self.fuse_route = fuse_route
        if expert_map is None:
            assert self.E_local == self.E_total, "weights hold E + n_shared experts (or pass expert_map)"
        self._bufs: dict = {}

    def _buffers(self, T: int, dev):
        key = (T, str(dev))
        if key not in self._bufs:
            bm = self.block_m or moe_pick_block_m(T, self.K, self.E_total, self.wfmt, self.weight_layout)
            if self.wfmt == W_BF16 and (bm == 32 or (bm == 16 and max(self.H, self.I) > BF16_SMALL_BLOCK_MAX_K)):
                bm = 64  # bf16 weights: no 32-row kernel; 16-row blocks only with the activation tile in LDS
            cap = moe_sort_capacity(T, self.K, self.E_local, bm)
            b = dict(
                bm=bm,
                ids=torch.empty((T, self.K), dtype=torch.int32, device=dev),
                ids_global=torch.empty((T, self.K), dtype=torch.int32, device=dev),
                w=torch.empty((T, self.K), dtype=torch.float32, device=dev),
                sort=dict(
                    expert_counts=torch.empty(self.E_local, dtype=torch.int32, device=dev),
                    expert_offsets=torch.empty(self.E_local + 1, dtype=torch.int32, device=dev),
                    sorted_slots=torch.empty(cap, dtype=torch.int32, device=dev),
                    block_expert=torch.empty(max(cap // bm, 1), dtype=torch.int32, device=dev),
                    num_padded=torch.empty(1, dtype=torch.int32, device=dev)),
                workspace=None, a1=None,
            )
            if self.afmt != A_BF16:
                cs, ss, sdt = quant_shapes(self.afmt, T, self.H)
                b["a1"] = (torch.empty(cs, dtype=torch.uint8, device=dev), torch.empty(ss, dtype=sdt, device=dev))
            self._bufs = {key: b}
        return self._bufs[key]

    def _record(self, b: dict, stream, dev) -> None:
        """Marks every reused buffer as in use on `stream` when it is not the current one."""
        if stream is None or stream == torch.cuda.current_stream(dev):
            return
        ts = [b["ids"], b["ids_global"], b["w"], *b["sort"].values(), *(b["a1"] or ())]
        if b["workspace"] is not None:
            ts.append(b["workspace"])
        for t in ts:
            t.record_stream(stream)

    def __call__(self, x: torch.Tensor, router_logits: torch.Tensor, stream=None) -> torch.Tensor:
        T = x.shape[0]
        b = self._buffers(T, x.device)
        out = torch.empty((T, self.H), dtype=torch.bfloat16, device=x.device)
        if stream is not None and stream != torch.cuda.current_stream(x.device):
            out.record_stream(stream)
        try:
            return self._forward(x, router_logits, b, out, stream)
        finally:
            self._record(b, stream, x.device)

    def _forward(self, x, router_logits, b, out, stream):
        if self.fuse_route and self.expert_map is None and self.grouped is None:
            a1c = a1s = None
            if self.afmt != A_BF16:
                a1c, a1s = moe_quant_act(x, self.afmt, b["a1"][0], b["a1"][1], stream)
            out, b["workspace"] = moe_layer_forward(
                x, router_logits, self.w1, self.w1_scale, self.w2, self.w2_scale, b["ids"], b["w"], b["sort"],
                self.wfmt, self.afmt, b["bm"], self.E_local, self.I, self.score, True, self.n_shared,
                self.shared_weight, out, b["workspace"], a1c, a1s, stream, self.weight_layout, self.act)
            return out
        if self.expert_map is not None:
            moe_route_topk(router_logits, self.topk, self.score, True, self.n_shared, self.shared_weight,
                           b["ids_global"], b["w"], stream)
            moe_map_experts(b["ids_global"], self.expert_map, self.E_total, None, b["ids"], stream)
            moe_align_sort(b["ids"], self.E_local, b["bm"], b["sort"], stream)
        elif self.grouped is None:
            moe_route_align(router_logits, self.topk, b["bm"], self.score, True, self.n_shared, self.shared_weight,
                            b["ids"], b["w"], b["sort"], stream)
        else:
            g = self.grouped
            moe_route_grouped_topk(router_logits, self.topk, g["num_expert_group"], g["topk_group"],
                                   g.get("correction_bias"), self.score, True, g.get("routed_scaling_factor", 1.0),
                                   self.n_shared, self.shared_weight, b["ids"], b["w"], stream)
            moe_align_sort(b["ids"], self.E_total, b["bm"], b["sort"], stream)
        a1c = a1s = None
        if self.afmt != A_BF16:
            a1c, a1s = moe_quant_act(x, self.afmt, b["a1"][0], b["a1"][1], stream)
        out, b["workspace"] = moe_experts_forward(
            x, self.w1, self.w1_scale, self.w2, self.w2_scale, b["ids"], b["w"], b["sort"], self.wfmt, self.afmt,
            b["bm"], self.E_local, self.I, out, b["workspace"], a1c, a1s, stream, self.weight_layout, self.act)
        return out
