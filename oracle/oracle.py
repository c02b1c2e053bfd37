"""ctypes binding of the C oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the CPU
baseline leg of bench.py may import this module.  The product path (the HIP
library and its Python binding) never imports or calls it, and the oracle shares
no code with that path.

All arrays are numpy host arrays.  bf16 values are numpy uint16 bit patterns.

Which test pins which oracle function (tests/test_oracle_*.py, all CPU):
  orc_e2m1_value / orc_e8m0_value / orc_e4m3_value
      literal e2m1 table and sign rule; 2**(e-127); torch.float8_e4m3fn and
      torch.float8_e8m0fnu casts (library routines) on all 256 codes.
  orc_f64_to_bf16 / orc_f32_to_bf16
      torch's float32 -> bfloat16 cast on random and boundary values.
  orc_e4m3_encode / orc_e2m1_encode
      brute-force nearest-code search over every finite code (ties to even),
      golden tie and saturation table, torch.float8_e4m3fn cast.
  orc_mx_shared_exp
      math.frexp closed form and golden boundary table.
  orc_route_topk
      brute-force full stable sort; weights sum to 1; top-1 weight exactly 1;
      softmax of the chosen logits equals the renormalised full softmax.
  orc_route_grouped_topk
      hand-worked golden examples (tests/golden/grouped_router_examples.txt);
      one group without bias equals orc_route_topk; the same reading written with
      numpy sort/lexsort on random inputs with exact ties; slots from at most
      topk_group groups; weights are the unbiased scores and sum to the scaling
      factor; a uniform bias shift keeps the ids.
  router weight on the input (orc_layer.weight_on_input, top-1)
      weight 1 equals the ordinary layer bit for bit; weight w equals W2 . act(w Wg a,
      w Wu a) written with numpy matmul on weights decoded from the literal tables.
  orc_map_experts
      numpy fancy indexing of the map; the expert-parallel shares of a layer (each
      device's local weights, local ids) add up to the whole layer's output.
  orc_align_sort
      numpy.argsort(kind="stable") of the flattened ids; offsets multiples of
      block_m; every slot exactly once.
  orc_quant_act
      brute force per element, golden worked groups, dequantised error bounds;
      per-tensor FP8 equals the per-row rule on the flattened tensor.
  FP8 per-tensor weights / activations (orc_layer formats)
      per-tensor weights equal per-channel weights with the scale broadcast over rows;
      a one-token, one-slot batch with per-tensor activations equals per-token ones;
      numpy brute force (torch e4m3 casts, one amax per tensor) on a whole batch.
  orc_stage1 / orc_stage2 / orc_forward
      top-1 weight-1 routing equals a dense gated MLP computed with numpy.matmul
      on weights decoded from the literal tables; closed-form all-equal example;
      fp64 brute force on tiny shapes; token-permutation and expert-relabelling
      invariance; +1 on every w2 E8M0 byte doubles the output; zero weight slot
      contributes nothing.
  SwiGLU-OAI, biases, interleaved gate/up rows (orc_stage1 / orc_stage2 options)
      alpha 1, beta 0, no limit equals the SiLU layer bit for bit; interleaved rows
      (codes, scales, biases permuted with numpy) equal separated rows bit for bit, and
      the unpermuted rows do not; the down-projection bias adds sum_j w_j * b2[e_j]
      (numpy einsum); with zero w1 codes (gate and up = biases) the clamp's
      invariances: gate clamped from above only, up on both sides, none at limit 0,
      zero at up = -beta or gate = 0, increasing in the gate below the limit.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

W_MXFP4, W_FP8_BLOCK128, W_FP8_CHANNEL, W_FP8_TENSOR, W_BF16 = 0, 1, 2, 3, 4
A_BF16, A_MXFP4_G32, A_FP8_G128, A_FP8_TOKEN, A_FP8_TENSOR = 0, 1, 2, 3, 4
SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    import subprocess

    src = os.path.join(_HERE, "moe_oracle.c")
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(src):
        cmd = [
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
            "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
            src, "-o", LIB_PATH + ".tmp", "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_uint]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [ctypes.c_uint]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f64_to_bf16.restype = ctypes.c_uint16
        L.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.restype = ctypes.c_uint
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e2m1_encode.restype = ctypes.c_uint
        L.orc_e2m1_encode.argtypes = [ctypes.c_float]
        L.orc_mx_shared_exp.restype = I
        L.orc_mx_shared_exp.argtypes = [ctypes.c_float]
        L.orc_route_topk.restype = I
        L.orc_route_topk.argtypes = [P, I, I, I, I, I, I, ctypes.c_float, P, P]
        L.orc_map_experts.restype = I
        L.orc_map_experts.argtypes = [P, P, I, I, I, I, P]
        L.orc_route_grouped_topk.restype = I
        L.orc_route_grouped_topk.argtypes = [P, P, I, I, I, I, I, I, I, ctypes.c_float, I, ctypes.c_float, P, P]
        L.orc_sort_capacity.restype = ctypes.c_int64
        L.orc_sort_capacity.argtypes = [I, I, I, I]
        L.orc_align_sort.restype = I
        L.orc_align_sort.argtypes = [P, I, I, I, I, P, P, P, P, P]
        L.orc_quant_act.restype = I
        L.orc_quant_act.argtypes = [P, I, I, I, P, P]
        L.orc_stage1.restype = I
        L.orc_stage1.argtypes = [P, P, P, P, P, I, P]
        L.orc_stage2.restype = I
        L.orc_stage2.argtypes = [P, P, P, P, P, I, P]
        L.orc_forward.restype = I
        L.orc_forward.argtypes = [P, P, P, P, P, I, P]
        L.orc_num_threads.restype = I
        L.orc_num_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None) -> int | None:
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


# ---------------------------------------------------------------- codecs
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e8m0_value(byte: int) -> float:
    return lib().orc_e8m0_value(byte)


def e4m3_value(byte: int) -> float:
    return lib().orc_e4m3_value(byte)


def bf16_to_f32(b: int) -> float:
    return lib().orc_bf16_to_f32(b)


def f64_to_bf16(v: float) -> int:
    return lib().orc_f64_to_bf16(v)


def f32_to_bf16(v: float) -> int:
    return lib().orc_f32_to_bf16(v)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(v)


def e2m1_encode(v: float) -> int:
    return lib().orc_e2m1_encode(v)


def mx_shared_exp(amax: float) -> int:
    return lib().orc_mx_shared_exp(amax)


def num_threads() -> int:
    return lib().orc_num_threads()


# ---------------------------------------------------------------- router / sort / quant
def route_topk(logits: np.ndarray, topk: int, score: int = SCORE_SOFTMAX, renormalize: bool = True,
               n_shared: int = 0, shared_weight: float = 1.0):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    KP = topk + n_shared
    ids = np.empty((T, KP), np.int32)
    w = np.empty((T, KP), np.float32)
    rc = lib().orc_route_topk(_ptr(logits), T, E, topk, score, int(renormalize), n_shared,
                              shared_weight, _ptr(ids), _ptr(w))
    if rc:
        raise ValueError("orc_route_topk: bad arguments")
    return ids, w


def route_grouped_topk(logits: np.ndarray, topk: int, n_group: int, topk_group: int, bias: np.ndarray | None = None,
                       score: int = SCORE_SIGMOID, renormalize: bool = True, scaling: float = 1.0, n_shared: int = 0,
                       shared_weight: float = 1.0):
    """Grouped top-k router with an optional score-correction bias (see
    orc_route_grouped_topk for the reading of the pages)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    KP = topk + n_shared
    ids = np.empty((T, KP), np.int32)
    w = np.empty((T, KP), np.float32)
    rc = lib().orc_route_grouped_topk(_ptr(logits), _ptr(b), T, E, topk, n_group, topk_group, score,
                                      int(renormalize), scaling, n_shared, shared_weight, _ptr(ids), _ptr(w))
    if rc:
        raise ValueError("orc_route_grouped_topk: bad arguments")
    return ids, w


def map_experts(topk_ids: np.ndarray, expert_map: np.ndarray | None, E_global: int,
                num_local_tokens: int | None = None) -> np.ndarray:
    """Local ids of an expert-parallel share (see orc_map_experts)."""
    topk_ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    T, K = topk_ids.shape
    m = None if expert_map is None else np.ascontiguousarray(expert_map, dtype=np.int32)
    out = np.empty((T, K), np.int32)
    rc = lib().orc_map_experts(_ptr(topk_ids), _ptr(m), -1 if num_local_tokens is None else num_local_tokens, T, K,
                               E_global, _ptr(out))
    if rc:
        raise ValueError("orc_map_experts: bad arguments")
    return out


def sort_capacity(T: int, K: int, E_total: int, block_m: int) -> int:
    return lib().orc_sort_capacity(T, K, E_total, block_m)


def align_sort(topk_ids: np.ndarray, E_total: int, block_m: int):
    topk_ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    T, K = topk_ids.shape
    cap = sort_capacity(T, K, E_total, block_m)
    counts = np.empty(E_total, np.int32)
    offsets = np.empty(E_total + 1, np.int32)
    sorted_slots = np.empty(cap, np.int32)
    block_expert = np.empty(cap // block_m, np.int32)
    num_padded = np.empty(1, np.int32)
    rc = lib().orc_align_sort(_ptr(topk_ids), T, K, E_total, block_m, _ptr(counts), _ptr(offsets),
                              _ptr(sorted_slots), _ptr(block_expert), _ptr(num_padded))
    if rc:
        raise ValueError("orc_align_sort: bad arguments")
    return dict(expert_counts=counts, expert_offsets=offsets, sorted_slots=sorted_slots,
                block_expert=block_expert, num_padded=int(num_padded[0]))


def quant_act(x_bf16: np.ndarray, fmt: int):
    """Returns (codes, scales) in the layouts documented in moe_oracle.c."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x_bf16.shape
    if fmt == A_FP8_G128:
        codes = np.empty((rows, cols), np.uint8)
        scales = np.empty((rows, (cols + 127) // 128), np.float32)
    elif fmt == A_FP8_TOKEN:
        codes = np.empty((rows, cols), np.uint8)
        scales = np.empty((rows,), np.float32)
    elif fmt == A_FP8_TENSOR:
        codes = np.empty((rows, cols), np.uint8)
        scales = np.empty((1,), np.float32)
    elif fmt == A_MXFP4_G32:
        codes = np.empty((rows, cols // 2), np.uint8)
        scales = np.empty((rows, cols // 32), np.uint8)
    else:
        raise ValueError("quant_act: bf16 has no quantiser")
    rc = lib().orc_quant_act(_ptr(x_bf16), rows, cols, fmt, _ptr(codes), _ptr(scales))
    if rc:
        raise ValueError("orc_quant_act: bad arguments")
    return codes, scales


# ---------------------------------------------------------------- expert layer
class _Layer(ctypes.Structure):
    _fields_ = [
        ("H", ctypes.c_int), ("I", ctypes.c_int), ("E_total", ctypes.c_int), ("K", ctypes.c_int),
        ("wfmt", ctypes.c_int), ("afmt", ctypes.c_int),
        ("w1", ctypes.c_void_p), ("w1_scale", ctypes.c_void_p),
        ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
        ("act", ctypes.c_int), ("alpha", ctypes.c_double), ("beta", ctypes.c_double), ("limit", ctypes.c_double),
        ("gate_up_interleaved", ctypes.c_int),
        ("w1_bias", ctypes.c_void_p), ("w2_bias", ctypes.c_void_p),
        ("weight_on_input", ctypes.c_int),
    ]


ACT_SILU, ACT_SWIGLU_OAI = 0, 1


@dataclass
class Layer:
    """Weights of the expert layer (numpy arrays, layouts as in moe_oracle.h)."""
    H: int
    I: int
    E_total: int
    K: int
    wfmt: int
    afmt: int
    w1: np.ndarray
    w1_scale: np.ndarray
    w2: np.ndarray
    w2_scale: np.ndarray
    act: int = ACT_SILU
    alpha: float = 1.702
    beta: float = 1.0
    limit: float = 7.0
    gate_up_interleaved: bool = False
    w1_bias: np.ndarray | None = None  # bf16 bits [E_total, 2I] in w1 row order
    w2_bias: np.ndarray | None = None  # bf16 bits [E_total, H]
    weight_on_input: bool = False      # top-k weight on FC1 (top-1 routing), unweighted sum

    def _c(self) -> _Layer:
        for a in (self.w1, self.w1_scale, self.w2, self.w2_scale, self.w1_bias, self.w2_bias):
            assert a is None or a.flags["C_CONTIGUOUS"]
        for b, n in ((self.w1_bias, 2 * self.I), (self.w2_bias, self.H)):
            assert b is None or (b.dtype == np.uint16 and b.shape == (self.E_total, n))
        return _Layer(self.H, self.I, self.E_total, self.K, self.wfmt, self.afmt,
                      _ptr(self.w1), _ptr(self.w1_scale), _ptr(self.w2), _ptr(self.w2_scale),
                      self.act, self.alpha, self.beta, self.limit, int(self.gate_up_interleaved),
                      _ptr(self.w1_bias), _ptr(self.w2_bias), int(self.weight_on_input))


def _tokens(T: int, tokens) -> np.ndarray:
    if tokens is None:
        return np.arange(T, dtype=np.int32)
    return np.ascontiguousarray(tokens, dtype=np.int32)


def _full_batch_only(L: Layer, tokens, T: int):
    if L.afmt == A_FP8_TENSOR and tokens is not None and not np.array_equal(np.asarray(tokens), np.arange(T)):
        raise ValueError("per-tensor activation scales need the whole batch (tokens=None)")


def stage1(L: Layer, x_bf16: np.ndarray, topk_ids: np.ndarray, tokens=None, topk_weights=None) -> np.ndarray:
    """topk_weights: needed (and used) only when L.weight_on_input."""
    _full_batch_only(L, tokens, x_bf16.shape[0])
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    topk_ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    tw = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    tk = _tokens(x_bf16.shape[0], tokens)
    h = np.empty((len(tk) * L.K, L.I), np.uint16)
    c = L._c()
    rc = lib().orc_stage1(ctypes.byref(c), _ptr(x_bf16), _ptr(topk_ids), _ptr(tw), _ptr(tk), len(tk), _ptr(h))
    if rc:
        raise ValueError("orc_stage1 failed")
    return h


def stage2(L: Layer, h: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray, tokens=None,
           T: int | None = None) -> np.ndarray:
    """h: [len(tokens)*K, I] bf16 bits, slot rows in (token list, slot) order."""
    _full_batch_only(L, tokens, topk_ids.shape[0] if T is None else T)
    h = np.ascontiguousarray(h, dtype=np.uint16)
    topk_ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    topk_weights = np.ascontiguousarray(topk_weights, dtype=np.float32)
    tk = _tokens(topk_ids.shape[0] if T is None else T, tokens)
    assert h.shape == (len(tk) * L.K, L.I)
    out = np.empty((len(tk), L.H), np.float64)
    c = L._c()
    rc = lib().orc_stage2(ctypes.byref(c), _ptr(h), _ptr(topk_ids), _ptr(topk_weights), _ptr(tk),
                          len(tk), _ptr(out))
    if rc:
        raise ValueError("orc_stage2 failed")
    return out


def forward(L: Layer, x_bf16: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray,
            tokens=None) -> np.ndarray:
    _full_batch_only(L, tokens, x_bf16.shape[0])
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    topk_ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    topk_weights = np.ascontiguousarray(topk_weights, dtype=np.float32)
    tk = _tokens(x_bf16.shape[0], tokens)
    out = np.empty((len(tk), L.H), np.float64)
    c = L._c()
    rc = lib().orc_forward(ctypes.byref(c), _ptr(x_bf16), _ptr(topk_ids), _ptr(topk_weights), _ptr(tk),
                           len(tk), _ptr(out))
    if rc:
        raise ValueError("orc_forward failed")
    return out
