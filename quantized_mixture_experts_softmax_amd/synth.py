"""Seeded synthetic inputs for the fused MoE expert layer.

This module only draws random numbers in the shapes and dtypes of the workloads;
it holds none of the layer's arithmetic (no routing, sorting, quantisation rule or
GEMM).  The same bytes feed the HIP path and the CPU oracle.  bf16 activations
come from fp32 normal draws through torch's bfloat16 cast (a library conversion,
not the layer's arithmetic).  MXFP4 weight codes are uniform random bytes (two
uniform e2m1 nibbles per byte).  FP8 weights are prepared the way a checkpoint's
would be: fp32 draws from N(0, 1/K), one fp32 scale per 128x128 block, output row or
expert equal to that block's max |w| / 448, and codes from torch's float8_e4m3fn
cast of w / scale (a library conversion), so every e4m3 code -- zero, subnormal,
+-448 -- occurs.  fp8_weights="uniform" keeps the older draw (uniform bytes with the
exponent field held in [4, 7]).

Each tensor has its own child generator of numpy's PCG64 (SeedSequence(seed)
spawned six ways: x, logits, w1, w1 scales, w2, w2 scales; weight codes spawn one
child per expert), so a tensor's values
do not depend on the shapes of the others, and activations/logits drawn for the
largest token count give the smaller counts as prefixes.

Workloads (shapes follow the pages: w1 = fused gate/up [E, 2I, H], w2 = [E, H, I];
MXFP4 packs two e2m1 codes per byte along K with one E8M0 byte per 32 elements;
FP8 weights are e4m3fn bytes with fp32 scales per 128x128 block or per output
channel):
  tiny      T=64   H=256  I=256   E=8       top-2  MXFP4 w4a16  softmax, logits N(0,1)
  decode    T=64   H=2880 I=2880  E=32      top-4  MXFP4 w4a16  softmax, logits N(0,1.5)
  prefill   T=8192 H=2880 I=2880  E=128     top-4  MXFP4 w4a16  softmax, Zipf(1.1)-skewed logits
  prefill-w4a4     same as prefill with MXFP4 activations
  fp8-block T=4096 H=7168 I=2048  E=256(+1) top-8(+1 shared, weight 1) FP8 128x128 / act g128, sigmoid
  fp8-channel T in {1,16,256,4096} H=4096 I=14336 E=8 top-2 FP8 per-channel / act per-token, softmax
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field

import numpy as np

W_MXFP4, W_FP8_BLOCK128, W_FP8_CHANNEL, W_FP8_TENSOR, W_BF16 = 0, 1, 2, 3, 4
A_BF16, A_MXFP4_G32, A_FP8_G128, A_FP8_TOKEN, A_FP8_TENSOR = 0, 1, 2, 3, 4
SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    topk: int
    wfmt: int
    afmt: int
    score: int = SCORE_SOFTMAX
    n_shared: int = 0
    shared_weight: float = 1.0
    logit_kind: str = "normal"      # "normal" or "zipf"
    logit_std: float = 1.0
    zipf_exponent: float = 1.1
    seed: int = 1000
    T_sweep: tuple = field(default_factory=tuple)
    fp8_weights: str = "gauss"      # "gauss": N(0, 1/K) quantised per scale block; "uniform": uniform codes

    @property
    def E_total(self) -> int:
        return self.E + self.n_shared

    @property
    def K(self) -> int:
        return self.topk + self.n_shared

    def with_T(self, T: int) -> "Workload":
        return Workload(**{**self.__dict__, "T": T})

    def scaled(self, **kw) -> "Workload":
        return Workload(**{**self.__dict__, **kw})


WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 256, 8, 2, W_MXFP4, A_BF16, seed=1000),
    "decode": Workload("decode", 64, 2880, 2880, 32, 4, W_MXFP4, A_BF16, logit_std=1.5, seed=1001),
    "prefill": Workload("prefill", 8192, 2880, 2880, 128, 4, W_MXFP4, A_BF16, logit_kind="zipf", seed=1002),
    "prefill-w4a4": Workload("prefill-w4a4", 8192, 2880, 2880, 128, 4, W_MXFP4, A_MXFP4_G32,
                             logit_kind="zipf", seed=1002),
    "fp8-block": Workload("fp8-block", 4096, 7168, 2048, 256, 8, W_FP8_BLOCK128, A_FP8_G128,
                          score=SCORE_SIGMOID, n_shared=1, shared_weight=1.0, seed=1003),
    "fp8-channel": Workload("fp8-channel", 4096, 4096, 14336, 8, 2, W_FP8_CHANNEL, A_FP8_TOKEN, seed=1004,
                            T_sweep=(1, 16, 256, 4096)),
    # per-tensor FP8 leaf at the fp8-channel shapes (not a configuration of its own)
    "bf16-decode": Workload("bf16-decode", 64, 2880, 2880, 32, 4, W_BF16, A_BF16, logit_std=1.5, seed=1006),
    "fp8-tensor": Workload("fp8-tensor", 4096, 4096, 14336, 8, 2, W_FP8_TENSOR, A_FP8_TENSOR, seed=1005,
                           T_sweep=(1, 16, 256, 4096)),
}

_FP8_MAG_MASK = np.uint64(0xBFBFBFBFBFBFBFBF)  # clear exponent bit 3 (bit 6 of the byte)
_FP8_MAG_SET = np.uint64(0x2020202020202020)   # set exponent bit 1 (bit 5): exponent field in [4, 7]
_FP8_RMS = 0.85                                 # approx. rms of the resulting code values


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rngs(seed: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(6)]


def make_activations(w: Workload, T: int | None = None) -> np.ndarray:
    """x [T, H] bf16 bits, N(0,1); a prefix of the draws for the largest T."""
    T = w.T if T is None else T
    rng = _rngs(w.seed)[0]
    return f32_to_bf16_bits(rng.standard_normal((T, w.H), dtype=np.float32))


def make_logits(w: Workload, T: int | None = None) -> np.ndarray:
    """Router logits [T, E] fp32.  "zipf": expert popularity p_e proportional to
    r_e^-s with ranks r a seeded permutation of 1..E, logits = ln p_e + Gumbel(0,1),
    so the top-1 choice is distributed exactly as p (Gumbel-max)."""
    T = w.T if T is None else T
    rng = _rngs(w.seed)[1]
    if w.logit_kind == "normal":
        return rng.normal(0.0, w.logit_std, (T, w.E)).astype(np.float32)
    ranks = rng.permutation(w.E).astype(np.float64) + 1.0
    logp = -w.zipf_exponent * np.log(ranks)
    logp -= np.log(np.exp(logp).sum())
    g = rng.gumbel(0.0, 1.0, (T, w.E))
    return (logp[None, :] + g).astype(np.float32)


def make_correction_bias(w: Workload) -> np.ndarray:
    """Score-correction bias [E] fp32 for the grouped router: N(0, 0.05^2), drawn from
    its own generator (seed + 7) so the other draws of the workload are unchanged."""
    return np.random.default_rng(w.seed + 7).normal(0.0, 0.05, w.E).astype(np.float32)


def make_biases(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """bf16 biases (bits) of the two projections, [E_total, 2I] and [E_total, H], N(0, 0.1^2),
    from their own generator (seed + 11) so the other draws are unchanged."""
    rng = np.random.default_rng(w.seed + 11)
    b1 = f32_to_bf16_bits(rng.normal(0.0, 0.1, (w.E_total, 2 * w.I)).astype(np.float32))
    b2 = f32_to_bf16_bits(rng.normal(0.0, 0.1, (w.E_total, w.H)).astype(np.float32))
    return b1, b2


def interleave_rows(a: np.ndarray, I: int) -> np.ndarray:
    """Reorders axis 1 of a [E, 2I, ...] tensor from [gate_0..gate_{I-1}, up_0..up_{I-1}]
    to gate_0, up_0, gate_1, up_1, ... (a pure permutation of rows)."""
    order = np.stack([np.arange(I), I + np.arange(I)], axis=1).reshape(-1)
    return np.ascontiguousarray(a[:, order])


def _expert_codes(seq, shape, fp8: bool) -> np.ndarray:
    """Uniform random bytes for one expert.  FP8: the e4m3 exponent field is held in
    [4, 7], so codes are finite (no NaN) with |value| in [0.125, 1.875] and a random
    sign, uniform over those 64 codes."""
    a = np.random.default_rng(seq).integers(0, 256, shape, dtype=np.uint8)
    if fp8:
        v = a.reshape(-1).view(np.uint64)
        v &= _FP8_MAG_MASK
        v |= _FP8_MAG_SET
    return a


def _weight(w: Workload, N: int, K: int, seq_codes, rng_scales):
    """One [E_total, N, K] weight tensor in the workload's format; one child generator
    per expert, filled by a thread pool (the result does not depend on scheduling)."""
    from concurrent.futures import ThreadPoolExecutor

    E = w.E_total
    if w.wfmt == W_BF16:
        # unquantised: N(0, 1/K) per expert, rounded to bf16 (the bit patterns, uint16)
        out = np.empty((E, N, K), np.uint16)
        seqs_b = seq_codes.spawn(E)

        def fill_b(e):
            v = np.random.default_rng(seqs_b[e]).standard_normal((N, K), dtype=np.float32) / np.float32(math.sqrt(K))
            out[e] = f32_to_bf16_bits(v)

        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill_b, range(E)))
        return out, None
    fp8 = w.wfmt != W_MXFP4
    if fp8 and w.fp8_weights == "gauss":
        return _fp8_gauss_weight(w, N, K, seq_codes)
    kb = K if fp8 else K // 2
    codes = np.empty((E, N, kb), np.uint8)
    seqs = seq_codes.spawn(E)

    def fill(e):
        codes[e] = _expert_codes(seqs[e], (N, kb), fp8)

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(E)))
    if not fp8:
        scales = rng_scales.integers(118, 127, (E, N, K // 32), dtype=np.uint8)  # E8M0 exponent in [118, 126]
        return codes, scales
    base = 1.0 / (_FP8_RMS * math.sqrt(K))
    if w.wfmt == W_FP8_BLOCK128:
        scales = (rng_scales.uniform(0.75, 1.25, (E, (N + 127) // 128, (K + 127) // 128)) * base).astype(np.float32)
    elif w.wfmt == W_FP8_TENSOR:
        scales = (rng_scales.uniform(0.75, 1.25, (E,)) * base).astype(np.float32)
    else:
        scales = (rng_scales.uniform(0.75, 1.25, (E, N)) * base).astype(np.float32)
    return codes, scales


def _fp8_gauss_weight(w: Workload, N: int, K: int, seq_codes):
    """FP8 weights [E, N, K] prepared like a checkpoint's: per expert, fp32 draws from
    N(0, 1/K); per scale block (128x128 block, output row, or the whole expert) the scale is
    that block's max |w| / 448 (1 for an all-zero block), and the codes are torch's
    float8_e4m3fn cast of w / scale clipped to +-448.  One child generator per expert."""
    from concurrent.futures import ThreadPoolExecutor

    import torch

    E = w.E_total
    codes = np.empty((E, N, K), np.uint8)
    if w.wfmt == W_FP8_BLOCK128:
        scales = np.empty((E, (N + 127) // 128, (K + 127) // 128), np.float32)
    elif w.wfmt == W_FP8_TENSOR:
        scales = np.empty((E,), np.float32)
    else:
        scales = np.empty((E, N), np.float32)
    seqs = seq_codes.spawn(E)
    inv_sqrt_k = np.float32(1.0 / math.sqrt(K))

    def fill(e):
        v = np.random.default_rng(seqs[e]).standard_normal((N, K), dtype=np.float32)
        v *= inv_sqrt_k
        a = np.abs(v)
        if w.wfmt == W_FP8_BLOCK128:
            nb, kb = (N + 127) // 128, (K + 127) // 128
            pad = np.zeros((nb * 128, kb * 128), np.float32)
            pad[:N, :K] = a
            amax = pad.reshape(nb, 128, kb, 128).max(axis=(1, 3))
            s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
            full = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:N, :K]
        elif w.wfmt == W_FP8_TENSOR:
            amax = a.max()
            s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
            full = s
        else:
            amax = a.max(axis=1)
            s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
            full = s[:, None]
        del a
        q = np.clip(v / full, -448.0, 448.0).astype(np.float32)
        codes[e] = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        scales[e] = s

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(E)))
    return codes, scales


def make_weights(w: Workload):
    """(w1, w1_scale, w2, w2_scale) host arrays; w1 rows [0, I) gate, [I, 2I) up."""
    seqs = np.random.SeedSequence(w.seed).spawn(6)
    r = _rngs(w.seed)
    w1, w1s = _weight(w, 2 * w.I, w.H, seqs[2], r[3])
    w2, w2s = _weight(w, w.H, w.I, seqs[4], r[5])
    return w1, w1s, w2, w2s


def make_all(w: Workload, T: int | None = None) -> dict:
    T = w.T if T is None else T
    w1, w1s, w2, w2s = make_weights(w)
    return dict(x=make_activations(w, T), logits=make_logits(w, T), w1=w1, w1_scale=w1s, w2=w2, w2_scale=w2s)
