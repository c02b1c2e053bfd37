/*
 * CPU oracle for the quantized fused MoE expert layer -- plain, slow, obviously
 * correct.  TEST INFRASTRUCTURE ONLY: the product path never includes, links,
 * loads or calls it (only tests, the package smoke check and the CPU-baseline leg
 * of the benchmark do).  It shares no code with the HIP library.
 *
 * Sources, cited by page and section (the pages are three vLLM pages):
 *   [rocm_aiter_moe]  API page "vllm.model_executor.layers.fused_moe.experts.rocm_aiter_moe"
 *   [mxfp4.py]        source page "vllm/model_executor/layers/quantization/mxfp4.py"
 *   [quark_moe]       API page "vllm.model_executor.layers.quantization.quark.quark_moe"
 * The pages fix tensor names, shapes and dtypes but not the numerics.  Element
 * codecs follow the public OCP Microscaling (MX) v1.0 and OCP 8-bit floating point
 * specifications that the dtype names on the pages refer to (float4_e2m1fn_x2,
 * float8_e8m0fnu, float8_e4m3fn).  Every other numeric choice is a stated reading.
 *
 * Precision: dot products, SiLU and the top-k combine are evaluated in fp64.  The
 * only roundings are the ones the method itself defines: the intermediate
 * activation h is bf16 (activations are bf16 on the MXFP4 path, [mxfp4.py]
 * Mxfp4Config), and the dynamic activation quantisers take their decisions in
 * fp32, the precision of the scales the pages carry.
 *
 * Parity pins: see the header comment of oracle/oracle.py for which test pins
 * which function.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Element codecs                                                             */
/* ------------------------------------------------------------------------- */

/* e2m1 (OCP MX FP4): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.
 * Exponent field 0 is subnormal: m * 0.5.  Otherwise (1 + m/2) * 2^(E-1). */
double orc_e2m1_value(unsigned code) {
  unsigned E = (code >> 1) & 3u, m = code & 1u;
  double mag = (E == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)E - 1);
  return (code & 8u) ? -mag : mag;
}

/* E8M0 (OCP MX shared scale): an unsigned biased exponent, value 2^(e-127);
 * 0xFF encodes NaN. */
double orc_e8m0_value(unsigned byte) {
  byte &= 0xFFu;
  if (byte == 0xFFu) return NAN;
  return ldexp(1.0, (int)byte - 127);
}

/* e4m3fn (OCP FP8): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities; S.1111.111 is NaN; largest finite magnitude 448. */
double orc_e4m3_value(unsigned byte) {
  byte &= 0xFFu;
  unsigned E = (byte >> 3) & 15u, m = byte & 7u;
  if (E == 15u && m == 7u) return NAN;
  double mag = (E == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)E - 7);
  return (byte & 0x80u) ? -mag : mag;
}

float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a double to the nearest bf16 (8 significant bits, fp32 exponent range),
 * ties to even, in one step (no intermediate fp32 rounding). */
uint16_t orc_f64_to_bf16(double v) {
  if (isnan(v)) return (uint16_t)0x7FC0u;
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (a == 0.0) return sign;
  /* largest finite bf16 is (2 - 2^-7) * 2^127; the rounding boundary above it is
   * (2 - 2^-8) * 2^127 */
  if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return sign | 0x7F80u;
  int e;
  frexp(a, &e);               /* a = f * 2^e, f in [0.5, 1) */
  int E = e - 1;              /* floor(log2 a) */
  if (E < -126) E = -126;     /* subnormal range shares the spacing of the smallest binade */
  double ulp = ldexp(1.0, E - 7);
  double q = nearbyint(a / ulp); /* exact quotient (power of two), ties to even */
  double r = q * ulp;
  /* re-encode r exactly as fp32 and keep the upper half (r has <= 8 significant bits) */
  float rf = (float)r;
  uint32_t u;
  memcpy(&u, &rf, sizeof u);
  return sign | (uint16_t)(u >> 16);
}

uint16_t orc_f32_to_bf16(float v) { return orc_f64_to_bf16((double)v); }

/* Nearest e4m3fn code to v, ties to the code with an even mantissa, magnitudes at
 * or above 448 saturate to 448.  The sign bit of the code is the sign bit of v
 * (so -0.0 and small negative values give 0x80). */
unsigned orc_e4m3_encode(float v) {
  unsigned sign = signbit(v) ? 0x80u : 0u;
  double a = fabs((double)v);
  if (isnan(v)) return 0x7Fu | sign;
  if (a >= 448.0) return sign | 0x7Eu;
  if (a < ldexp(1.0, -6)) {
    /* subnormal binade: spacing 2^-9, codes 0..7; a result of 8 is the smallest
     * normal (exponent field 1, mantissa 0), which is also code 8 */
    double q = nearbyint(ldexp(a, 9));
    return sign | (unsigned)q;
  }
  int e;
  frexp(a, &e);
  int E = e - 1;                       /* in [-6, 8] */
  double q = nearbyint(ldexp(a, 3 - E)); /* 8 <= q <= 16 */
  if (q == 16.0) {
    E += 1;
    q = 8.0;
  }
  if (E > 8 || (E == 8 && q > 14.0)) return sign | 0x7Eu;
  return sign | ((unsigned)(E + 7) << 3) | (unsigned)(q - 8.0);
}

/* Nearest e2m1 code to v, ties to the code with an even mantissa bit, magnitudes
 * at or above 6 saturate to 6; sign bit copied from v. */
unsigned orc_e2m1_encode(float v) {
  unsigned sign = signbit(v) ? 8u : 0u;
  double a = fabs((double)v);
  if (a >= 6.0) return sign | 7u;
  unsigned code;
  if (a < 2.0) {
    code = (unsigned)nearbyint(a * 2.0);            /* 0, 0.5, 1, 1.5, 2 -> codes 0..4 */
  } else if (a < 4.0) {
    code = 4u + (unsigned)(nearbyint(a) - 2.0);      /* 2, 3, 4 -> codes 4..6 */
  } else {
    code = 6u + (unsigned)(nearbyint(a / 2.0) - 2.0); /* 4, 6 -> codes 6..7 */
  }
  return sign | code;
}

/* OCP MX shared exponent for an FP4 (e2m1) block: floor(log2(amax)) minus the
 * largest e2m1 exponent (2), clamped to the E8M0 range; an all-zero block gets
 * the smallest scale. */
int orc_mx_shared_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e;
  frexp((double)amax, &e);
  int s = (e - 1) - 2;
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  return s;
}

/* ------------------------------------------------------------------------- */
/* Router                                                                     */
/* ------------------------------------------------------------------------- */

/* Top-k routing.  The pages name the router only through its products: topk_ids
 * (int32) and topk_weights (fp32) of shape [T, k + shared], cast so in
 * [rocm_aiter_moe] rocm_aiter_fused_experts, and router_logits as the input in
 * [mxfp4.py] Mxfp4MoEMethod.apply_monolithic.  Reading: the k largest logits
 * (equal logits: lower expert id first) in descending order; softmax weights
 * taken over the full logit row (equal to the softmax over the chosen k when
 * renormalised, since the full denominator cancels), or sigmoid scores;
 * renormalised to sum to one when asked.  Shared experts sit in slots
 * [k, k + n_shared) with ids E + s and the given weight, as
 * [rocm_aiter_moe] inject_shared_expert_weights lays out the combined buffer. */
int orc_route_topk(const float* logits, int T, int E, int topk, int score, int renormalize,
                   int n_shared, float shared_weight, int32_t* topk_ids, float* topk_weights) {
  if (T < 0 || E <= 0 || topk <= 0 || topk > E || n_shared < 0) return -1;
  if (score != ORC_SCORE_SOFTMAX && score != ORC_SCORE_SIGMOID) return -1;
  const int KP = topk + n_shared;
  int* taken = (int*)calloc((size_t)E, sizeof(int));
  double* sel = (double*)malloc(sizeof(double) * (size_t)topk);
  if (!taken || !sel) { free(taken); free(sel); return -1; }
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    memset(taken, 0, sizeof(int) * (size_t)E);
    for (int j = 0; j < topk; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: equal logits keep the lower id */
      }
      taken[best] = 1;
      topk_ids[(size_t)t * KP + j] = best;
      sel[j] = (double)l[best];
    }
    double denom = 0.0;
    if (score == ORC_SCORE_SOFTMAX) {
      const double lmax = sel[0];
      if (renormalize) {
        for (int j = 0; j < topk; ++j) denom += exp(sel[j] - lmax);
      } else {
        for (int e = 0; e < E; ++e) denom += exp((double)l[e] - lmax);
      }
      for (int j = 0; j < topk; ++j)
        topk_weights[(size_t)t * KP + j] = (float)(exp(sel[j] - lmax) / denom);
    } else {
      double sg[64];
      for (int j = 0; j < topk && j < 64; ++j) {
        sg[j] = 1.0 / (1.0 + exp(-sel[j]));
        denom += sg[j];
      }
      if (topk > 64) { free(taken); free(sel); return -1; }
      for (int j = 0; j < topk; ++j)
        topk_weights[(size_t)t * KP + j] = (float)(renormalize ? sg[j] / denom : sg[j]);
    }
    for (int s = 0; s < n_shared; ++s) {
      topk_ids[(size_t)t * KP + topk + s] = E + s;
      topk_weights[(size_t)t * KP + topk + s] = shared_weight;
    }
  }
  free(taken);
  free(sel);
  return 0;
}

/* Grouped top-k routing with a score-correction bias.  The pages name this router
 * only through its parameters (num_expert_group, topk_group, e_score_correction_bias,
 * routed_scaling_factor, passed to the monolithic kernel in [mxfp4.py]
 * Mxfp4MoEMethod.apply_monolithic and [quark_moe] QuarkMoEMethod.apply_monolithic)
 * and through its output buffer ([rocm_aiter_moe] inject_shared_expert_weights: the
 * grouped router already returns the combined routed + shared buffer).  Reading (the
 * published group-limited routing of the DeepSeek-V2/V3 models these parameters come
 * from), per token:
 *   s[e]   = sigmoid(l[e]), or the softmax of the whole logit row;
 *   key[e] = s[e] + bias[e] with a bias, else the logit itself (same order as s);
 *   experts form num_expert_group contiguous groups of E / num_expert_group; a
 *   group's score is the sum of its two largest keys with a bias, else its largest;
 *   the topk_group best groups are kept, and the topk best keys among their experts
 *   are the routed slots, best first (equal keys or group scores: lower id first);
 *   weight[j] = s[id_j], divided by the sum over the k slots (slot order) when
 *   renormalising, then times routed_scaling_factor.
 * Keys, group scores and weights are evaluated in fp64.  Shared slots follow as in
 * orc_route_topk. */
int orc_route_grouped_topk(const float* logits, const float* bias, int T, int E, int topk, int n_group,
                           int topk_group, int score, int renormalize, float scaling, int n_shared,
                           float shared_weight, int32_t* topk_ids, float* topk_weights) {
  if (T < 0 || E <= 0 || topk <= 0 || n_shared < 0 || n_group <= 0 || E % n_group != 0) return -1;
  if (topk_group <= 0 || topk_group > n_group || topk > topk_group * (E / n_group)) return -1;
  if (score != ORC_SCORE_SOFTMAX && score != ORC_SCORE_SIGMOID) return -1;
  const int KP = topk + n_shared, gs = E / n_group;
  double* s = (double*)malloc(sizeof(double) * (size_t)E);
  double* key = (double*)malloc(sizeof(double) * (size_t)E);
  double* gsc = (double*)malloc(sizeof(double) * (size_t)n_group);
  int* gsel = (int*)malloc(sizeof(int) * (size_t)n_group);
  int* taken = (int*)malloc(sizeof(int) * (size_t)E);
  if (!s || !key || !gsc || !gsel || !taken) {
    free(s); free(key); free(gsc); free(gsel); free(taken);
    return -1;
  }
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    if (score == ORC_SCORE_SIGMOID) {
      for (int e = 0; e < E; ++e) s[e] = 1.0 / (1.0 + exp(-(double)l[e]));
    } else {
      double m = (double)l[0], z = 0.0;
      for (int e = 1; e < E; ++e) if ((double)l[e] > m) m = (double)l[e];
      for (int e = 0; e < E; ++e) z += exp((double)l[e] - m);
      for (int e = 0; e < E; ++e) s[e] = exp((double)l[e] - m) / z;
    }
    for (int e = 0; e < E; ++e) key[e] = bias ? s[e] + (double)bias[e] : (double)l[e];
    /* group scores */
    for (int g = 0; g < n_group; ++g) {
      const double* kg = key + (size_t)g * gs;
      int b1 = 0;
      for (int i = 1; i < gs; ++i) if (kg[i] > kg[b1]) b1 = i;
      double v = kg[b1];
      if (bias && gs > 1) {
        int b2 = -1;
        for (int i = 0; i < gs; ++i) {
          if (i == b1) continue;
          if (b2 < 0 || kg[i] > kg[b2]) b2 = i;
        }
        v += kg[b2];
      }
      gsc[g] = v;
      gsel[g] = 0;
    }
    for (int r = 0; r < topk_group; ++r) {
      int best = -1;
      for (int g = 0; g < n_group; ++g) {
        if (gsel[g]) continue;
        if (best < 0 || gsc[g] > gsc[best]) best = g; /* strict: equal scores keep the lower id */
      }
      gsel[best] = 1;
    }
    /* experts of the kept groups */
    for (int e = 0; e < E; ++e) taken[e] = !gsel[e / gs];
    double denom = 0.0;
    for (int j = 0; j < topk; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || key[e] > key[best]) best = e;
      }
      taken[best] = 1;
      topk_ids[(size_t)t * KP + j] = best;
      denom += s[best];
    }
    for (int j = 0; j < topk; ++j) {
      const double w = s[topk_ids[(size_t)t * KP + j]];
      topk_weights[(size_t)t * KP + j] = (float)((renormalize ? w / denom : w) * (double)scaling);
    }
    for (int q = 0; q < n_shared; ++q) {
      topk_ids[(size_t)t * KP + topk + q] = E + q;
      topk_weights[(size_t)t * KP + topk + q] = shared_weight;
    }
  }
  free(s); free(key); free(gsc); free(gsel); free(taken);
  return 0;
}

/* Expert-parallel share of the layer on one device.  The pages hand an expert map
 * to the fused kernel as its expert mask ([rocm_aiter_moe] AiterExperts.apply:
 * expert_mask=expert_map) together with the per-rank count of valid tokens
 * (num_local_tokens = expert_tokens_meta.expert_num_tokens).  Reading: expert_map
 * [E_global] holds each global expert's local id on this device, or -1 when it lives
 * elsewhere; topk_ids keep global ids; token rows at or past num_local_tokens are not
 * valid here.  The local id of slot (t, j) is expert_map[topk_ids[t, j]] for a valid
 * row and an id in [0, E_global), else -1 (skipped by the sort and the combine, so the
 * layer's output is this device's partial sum).  expert_map NULL: identity;
 * num_local_tokens < 0: every row valid. */
int orc_map_experts(const int32_t* topk_ids, const int32_t* expert_map, int num_local_tokens, int T, int K,
                    int E_global, int32_t* local_ids) {
  if (T < 0 || K <= 0 || E_global <= 0) return -1;
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < K; ++j) {
      const int g = topk_ids[(size_t)t * K + j];
      int loc = -1;
      if ((num_local_tokens < 0 || t < num_local_tokens) && g >= 0 && g < E_global) loc = expert_map ? expert_map[g] : g;
      local_ids[(size_t)t * K + j] = loc;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Token -> expert sort                                                       */
/* ------------------------------------------------------------------------- */

/* Capacity of the padded sorted list: every slot plus at most block_m - 1 pad
 * rows per expert. */
int64_t orc_sort_capacity(int T, int K, int E_total, int block_m) {
  return (int64_t)T * K + (int64_t)E_total * (block_m - 1);
}

/* Stable counting sort of the flattened slots (slot = t*K + j) by expert id, each
 * expert's run padded up to a multiple of block_m.  The pages name this step only
 * as the "moe sorting" dispatch policy handed to the fused kernel and the
 * per-expert token counts ([rocm_aiter_moe] rocm_aiter_fused_experts,
 * AiterExperts.apply); the layout below is the plain reading.
 *   expert_counts[e]   slots routed to e
 *   expert_offsets[e]  first padded row of e; expert_offsets[E_total] = total padded rows
 *   sorted_slots[p]    slot id at padded row p, or the pad sentinel T*K
 *   block_expert[b]    expert owning rows [b*block_m, (b+1)*block_m), or -1 past the end
 *   num_padded[0]      expert_offsets[E_total]
 * Slots with an id outside [0, E_total) are not placed. */
int orc_align_sort(const int32_t* topk_ids, int T, int K, int E_total, int block_m,
                   int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
                   int32_t* block_expert, int32_t* num_padded) {
  if (T < 0 || K <= 0 || E_total <= 0 || block_m <= 0) return -1;
  const int64_t n = (int64_t)T * K;
  const int64_t cap = orc_sort_capacity(T, K, E_total, block_m);
  for (int e = 0; e < E_total; ++e) expert_counts[e] = 0;
  for (int64_t s = 0; s < n; ++s) {
    int e = topk_ids[s];
    if (e >= 0 && e < E_total) expert_counts[e]++;
  }
  expert_offsets[0] = 0;
  for (int e = 0; e < E_total; ++e) {
    int padded = (expert_counts[e] + block_m - 1) / block_m * block_m;
    expert_offsets[e + 1] = expert_offsets[e] + padded;
  }
  num_padded[0] = expert_offsets[E_total];
  for (int64_t p = 0; p < cap; ++p) sorted_slots[p] = (int32_t)n;
  /* place slots expert by expert, each in ascending slot order */
  for (int e = 0; e < E_total; ++e) {
    int64_t pos = expert_offsets[e];
    for (int64_t s = 0; s < n; ++s)
      if (topk_ids[s] == e) sorted_slots[pos++] = (int32_t)s;
  }
  for (int64_t b = 0; b < cap / block_m; ++b) {
    int64_t row = b * block_m;
    block_expert[b] = -1;
    for (int e = 0; e < E_total; ++e)
      if (row >= expert_offsets[e] && row < expert_offsets[e + 1]) block_expert[b] = e;
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Dynamic activation quantisation                                            */
/* ------------------------------------------------------------------------- */

/* Quantise one contiguous group of bf16 values to FP8 with a symmetric dynamic
 * scale: s = amax / 448 (fp32 division; s = 1 for an all-zero group), code =
 * nearest e4m3fn of x / s (fp32 division).  Returns s. */
static float quant_group_fp8(const uint16_t* x, int n, uint8_t* codes) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = fabsf(orc_bf16_to_f32(x[i]));
    if (a > amax) amax = a;
  }
  float s = (amax > 0.0f) ? amax / 448.0f : 1.0f;
  for (int i = 0; i < n; ++i) {
    float q = orc_bf16_to_f32(x[i]) / s;
    codes[i] = (uint8_t)orc_e4m3_encode(q);
  }
  return s;
}

/* Formats ([rocm_aiter_moe] AiterFp8BlockExperts: 128-grouped dynamic activation
 * scale; AiterFp8ChannelExperts: per-token dynamic scale; AiterMxfp4Experts:
 * MXFP4 dynamic activations, packed two per byte along the hidden dimension as in
 * [quark_moe] QuarkOCP_MX_MoEMethod.get_packed_dim):
 *   FP8_G128:  codes [rows][cols] e4m3, scales fp32 [rows][ceil(cols/128)]
 *   FP8_TOKEN: codes [rows][cols] e4m3, scales fp32 [rows]
 *   MXFP4_G32: codes [rows][cols/2] (low nibble = even column), scales E8M0 [rows][cols/32]
 * MXFP4: per 32-group, shared exponent es = orc_mx_shared_exp(amax); each value
 * is x * 2^-es (exact) rounded to the nearest e2m1 code, saturating at 6. */
int orc_quant_act(const uint16_t* x, int rows, int cols, int fmt, uint8_t* codes, void* scales) {
  if (rows < 0 || cols <= 0) return -1;
  if (fmt == ORC_A_FP8_G128) {
    const int ng = (cols + 127) / 128;
    float* sc = (float*)scales;
    for (int r = 0; r < rows; ++r)
      for (int g = 0; g < ng; ++g) {
        int c0 = g * 128, n = cols - c0 < 128 ? cols - c0 : 128;
        sc[(size_t)r * ng + g] = quant_group_fp8(x + (size_t)r * cols + c0, n, codes + (size_t)r * cols + c0);
      }
    return 0;
  }
  if (fmt == ORC_A_FP8_TOKEN) {
    float* sc = (float*)scales;
    for (int r = 0; r < rows; ++r) sc[r] = quant_group_fp8(x + (size_t)r * cols, cols, codes + (size_t)r * cols);
    return 0;
  }
  if (fmt == ORC_A_FP8_TENSOR) {
    /* one scale for the whole tensor: the per-group rule over all rows * cols values
     * ([rocm_aiter_moe] QuantMethod.PER_TENSOR, AiterFp8TensorExperts) */
    if ((long long)rows * cols > 0x7FFFFFFFLL) return -1;
    ((float*)scales)[0] = rows ? quant_group_fp8(x, rows * cols, codes) : 1.0f;
    return 0;
  }
  if (fmt == ORC_A_MXFP4_G32) {
    if (cols % 32) return -1;
    uint8_t* sc = (uint8_t*)scales;
    const int ng = cols / 32;
    for (int r = 0; r < rows; ++r)
      for (int g = 0; g < ng; ++g) {
        const uint16_t* xs = x + (size_t)r * cols + g * 32;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
          float a = fabsf(orc_bf16_to_f32(xs[i]));
          if (a > amax) amax = a;
        }
        int es = orc_mx_shared_exp(amax);
        sc[(size_t)r * ng + g] = (uint8_t)(es + 127);
        uint8_t* cb = codes + (size_t)r * (cols / 2) + g * 16;
        for (int i = 0; i < 16; ++i) {
          unsigned lo = orc_e2m1_encode((float)ldexp((double)orc_bf16_to_f32(xs[2 * i]), -es));
          unsigned hi = orc_e2m1_encode((float)ldexp((double)orc_bf16_to_f32(xs[2 * i + 1]), -es));
          cb[i] = (uint8_t)(lo | (hi << 4));
        }
      }
    return 0;
  }
  return -1;
}

/* Dequantised activation row (fp64) of one bf16 row of length n, through the
 * layer's activation format. */
static int activation_row(int afmt, const uint16_t* x, int n, double* out) {
  if (afmt == ORC_A_FP8_TENSOR) return -1; /* needs the whole tensor: tensor_rows */
  if (afmt == ORC_A_BF16) {
    for (int i = 0; i < n; ++i) out[i] = (double)orc_bf16_to_f32(x[i]);
    return 0;
  }
  uint8_t* codes = (uint8_t*)malloc((size_t)n);
  float* fsc = (float*)malloc(sizeof(float) * (size_t)((n + 31) / 32 + 1));
  if (!codes || !fsc) { free(codes); free(fsc); return -1; }
  int rc = orc_quant_act(x, 1, n, afmt, codes, fsc);
  if (rc == 0) {
    if (afmt == ORC_A_FP8_G128) {
      for (int i = 0; i < n; ++i) out[i] = orc_e4m3_value(codes[i]) * (double)fsc[i / 128];
    } else if (afmt == ORC_A_FP8_TOKEN) {
      for (int i = 0; i < n; ++i) out[i] = orc_e4m3_value(codes[i]) * (double)fsc[0];
    } else {
      const uint8_t* e8 = (const uint8_t*)fsc;
      for (int i = 0; i < n; ++i) {
        unsigned nib = (codes[i / 2] >> (4 * (i & 1))) & 15u;
        out[i] = orc_e2m1_value(nib) * orc_e8m0_value(e8[i / 32]);
      }
    }
  }
  free(codes);
  free(fsc);
  return rc;
}

/* Per-tensor FP8 activations: the n_rows x n values given (rows[i] points at row i)
 * quantised with one scale and dequantised into out[i * n + k]. */
static int tensor_rows(const uint16_t* const* rows, size_t n_rows, int n, double* out) {
  const size_t total = n_rows * (size_t)n;
  if (total > 0x7FFFFFFFu) return -1;
  uint16_t* buf = (uint16_t*)calloc(total + 1, sizeof(uint16_t));
  uint8_t* codes = (uint8_t*)malloc(total + 1);
  if (!buf || !codes) { free(buf); free(codes); return -1; }
  for (size_t i = 0; i < n_rows; ++i) memcpy(buf + i * n, rows[i], sizeof(uint16_t) * (size_t)n);
  float s = 1.0f;
  int rc = orc_quant_act(buf, (int)n_rows, n, ORC_A_FP8_TENSOR, codes, &s);
  for (size_t i = 0; rc == 0 && i < total; ++i) out[i] = orc_e4m3_value(codes[i]) * (double)s;
  free(buf);
  free(codes);
  return rc;
}

/* ------------------------------------------------------------------------- */
/* Expert weights                                                             */
/* ------------------------------------------------------------------------- */

/* Decode row n of expert e of a [E][N][K] weight tensor into fp64.
 * MXFP4 ([mxfp4.py] Mxfp4MoEMethod.create_weights: uint8 [E, N, K/2] with two
 * e2m1 values per byte and uint8 E8M0 scales [E, N, K/32]): value =
 * e2m1(nibble) * 2^(scale-127), exact.
 * FP8 block ([rocm_aiter_moe] AiterFp8BlockExperts: 128x128 weight blocks):
 * value = e4m3(code) * scale[e][n/128][k/128].
 * FP8 channel ([rocm_aiter_moe] AiterFp8ChannelExperts: per output channel):
 * value = e4m3(code) * scale[e][n].
 * bf16 (the unquantised leaf, [rocm_aiter_moe] AiterUnquantizedExperts):
 * value = the bf16 number itself, exact in fp64. */
static void weight_row(int wfmt, const uint8_t* w, const void* scale, int e, int n, int N, int K, double* out) {
  if (wfmt == ORC_W_BF16) {
    const uint16_t* row = (const uint16_t*)w + ((size_t)e * N + n) * (size_t)K;
    for (int k = 0; k < K; ++k) out[k] = (double)orc_bf16_to_f32(row[k]);
  } else if (wfmt == ORC_W_MXFP4) {
    const uint8_t* row = w + ((size_t)e * N + n) * (size_t)(K / 2);
    const uint8_t* srow = (const uint8_t*)scale + ((size_t)e * N + n) * (size_t)(K / 32);
    for (int k = 0; k < K; ++k) {
      unsigned nib = (row[k / 2] >> (4 * (k & 1))) & 15u;
      out[k] = orc_e2m1_value(nib) * orc_e8m0_value(srow[k / 32]);
    }
  } else if (wfmt == ORC_W_FP8_BLOCK128) {
    const int nbn = (N + 127) / 128, nbk = (K + 127) / 128;
    const uint8_t* row = w + ((size_t)e * N + n) * (size_t)K;
    const float* srow = (const float*)scale + ((size_t)e * nbn + n / 128) * (size_t)nbk;
    for (int k = 0; k < K; ++k) out[k] = orc_e4m3_value(row[k]) * (double)srow[k / 128];
  } else {
    /* FP8 channel: scale[e][n]; FP8 tensor ([rocm_aiter_moe] AiterFp8TensorExperts,
     * PER_TENSOR): one scale[e] per expert and projection */
    const uint8_t* row = w + ((size_t)e * N + n) * (size_t)K;
    const double s = (double)((const float*)scale)[wfmt == ORC_W_FP8_TENSOR ? (size_t)e : (size_t)e * N + n];
    for (int k = 0; k < K; ++k) out[k] = orc_e4m3_value(row[k]) * s;
  }
}

static double dot(const double* a, const double* b, int n) {
  double acc = 0.0;
  for (int i = 0; i < n; ++i) acc += a[i] * b[i];
  return acc;
}

/* The gated activation of one output column.
 * SILU ([rocm_aiter_moe] AiterExperts: activation SILU, act-and-mul only):
 *   h = silu(gate) * up with silu(z) = z / (1 + e^-z).
 * SWIGLU_OAI: the pages give only its name ([rocm_aiter_moe] _resolve_aiter_activation,
 * SWIGLUOAI mapped to the kernel's "swiglu") and its constants ([mxfp4.py]
 * Mxfp4MoEMethod.get_fused_moe_quant_config: gemm1_alpha 1.702, gemm1_beta 1.0,
 * swiglu_limit 7.0; rocm_aiter_fused_experts passes limit 0.0 when there is none).
 * Reading (the published gpt-oss activation these constants belong to): the gate is
 * clamped from above at the limit, the up value to [-limit, limit] (no clamping when
 * limit <= 0), and h = gate * sigmoid(alpha * gate) * (up + beta). */
static double glu(const orc_layer* L, double g, double u) {
  if (L->act == ORC_ACT_SILU) return g / (1.0 + exp(-g)) * u;
  if (L->limit > 0.0) {
    if (g > L->limit) g = L->limit;
    if (u > L->limit) u = L->limit;
    if (u < -L->limit) u = -L->limit;
  }
  return g / (1.0 + exp(-L->alpha * g)) * (u + L->beta);
}

/* bf16 bias value, 0 without a bias tensor. */
static double bias_at(const uint16_t* b, size_t i) { return b ? (double)orc_bf16_to_f32(b[i]) : 0.0; }

static int layer_ok(const orc_layer* L) {
  if (!L || L->H <= 0 || L->I <= 0 || L->E_total <= 0 || L->K <= 0) return 0;
  if (L->H % 32 || L->I % 32) return 0;
  if (L->wfmt < ORC_W_MXFP4 || L->wfmt > ORC_W_BF16) return 0;
  if (L->afmt < ORC_A_BF16 || L->afmt > ORC_A_FP8_TENSOR) return 0;
  if (L->act != ORC_ACT_SILU && L->act != ORC_ACT_SWIGLU_OAI) return 0;
  return 1;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Stage 1: for slot j of token t routed to expert e, gate_n = <a, W1[e][rg]> + b1[e][rg],
 * up_n = <a, W1[e][ru]> + b1[e][ru], h_n = bf16(act(gate_n, up_n)).  Rows: rg = n,
 * ru = I + n (gate rows then up rows, the SEPARATED gate/up layout of [rocm_aiter_moe]
 * rocm_aiter_fused_experts and [mxfp4.py] Mxfp4MoEMethod._setup_kernel_k3_situ), or
 * rg = 2n, ru = 2n + 1 (the INTERLEAVE gate mode [rocm_aiter_moe]
 * mxfp4_w4a16_extra_kwargs selects for MXFP4 w4a16).  Biases are bf16 [E, 2I] in the
 * same row order ([mxfp4.py] Mxfp4MoEMethod.create_weights: w13_bias). */
int orc_stage1(const orc_layer* L, const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
               const int32_t* tokens, int n_tok, uint16_t* h) {
  if (!layer_ok(L) || n_tok < 0 || (L->weight_on_input && !topk_weights)) return -1;
  const int H = L->H, I = L->I, K = L->K;
  int err = 0;
  /* per-tensor activations: one scale over the listed tokens (the whole batch) */
  double* a_all = NULL;
  if (L->afmt == ORC_A_FP8_TENSOR) {
    const uint16_t** rp = (const uint16_t**)malloc(sizeof(uint16_t*) * ((size_t)n_tok + 1));
    a_all = (double*)malloc(sizeof(double) * ((size_t)n_tok * H + 1));
    if (!rp || !a_all) { free(rp); free(a_all); return -1; }
    for (int i = 0; i < n_tok; ++i) rp[i] = x + (size_t)tokens[i] * H;
    const int rc = tensor_rows(rp, (size_t)n_tok, H, a_all);
    free(rp);
    if (rc) { free(a_all); return -1; }
  }
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)H);
    double* wr = (double*)malloc(sizeof(double) * (size_t)H);
    if (!a || !wr) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < n_tok; ++i) {
      if (!a || !wr) continue;
      const int t = tokens[i];
      if (a_all) {
        memcpy(a, a_all + (size_t)i * H, sizeof(double) * (size_t)H);
      } else if (activation_row(L->afmt, x + (size_t)t * H, H, a)) {
#pragma omp atomic write
        err = 1;
        continue;
      }
      for (int j = 0; j < K; ++j) {
        const int e = topk_ids[(size_t)t * K + j];
        uint16_t* hrow = h + ((size_t)i * K + j) * (size_t)I;
        if (e < 0 || e >= L->E_total) {
          for (int n = 0; n < I; ++n) hrow[n] = 0;
          continue;
        }
        /* router weight on the input: FC1 is linear, so scaling its input by the weight
         * scales both projections ([rocm_aiter_moe] AiterFp8TensorExperts.apply: tkw1
         * applies topk_weights to FC1's output instead of FC2's; top-1 only) */
        const double fc1w = L->weight_on_input ? (double)topk_weights[(size_t)t * K + j] : 1.0;
        for (int n = 0; n < I; ++n) {
          const int rg = L->gate_up_interleaved ? 2 * n : n;
          const int ru = L->gate_up_interleaved ? 2 * n + 1 : I + n;
          weight_row(L->wfmt, L->w1, L->w1_scale, e, rg, 2 * I, H, wr);
          const double g = fc1w * dot(a, wr, H) + bias_at(L->w1_bias, (size_t)e * 2 * I + rg);
          weight_row(L->wfmt, L->w1, L->w1_scale, e, ru, 2 * I, H, wr);
          const double u = fc1w * dot(a, wr, H) + bias_at(L->w1_bias, (size_t)e * 2 * I + ru);
          hrow[n] = orc_f64_to_bf16(glu(L, g, u));
        }
      }
    }
    free(a);
    free(wr);
  }
  free(a_all);
  return err ? -1 : 0;
}

/* Stage 2: y_m = <h_slot, W2[e][m]> + b2[e][m] (bf16 bias [E, H], [mxfp4.py]
 * Mxfp4MoEMethod.create_weights: w2_bias) and out_m = sum over the token's slots, in
 * ascending slot order, of topk_weight * y_m.  The weights multiply the down
 * projection's output and the reduction belongs to the expert computation itself
 * ([rocm_aiter_moe] AiterExperts.finalize_weight_and_reduce_impl is a no-op;
 * AiterFp8ChannelExperts.apply contrasts the default with weighting FC1). */
int orc_stage2(const orc_layer* L, const uint16_t* h, const int32_t* topk_ids, const float* topk_weights,
               const int32_t* tokens, int n_tok, double* out) {
  if (!layer_ok(L) || n_tok < 0) return -1;
  const int H = L->H, I = L->I, K = L->K;
  int err = 0;
  /* per-tensor activations: one scale over every slot row given (rows of slots that are
   * not routed are zero and leave the amax alone) */
  double* a_all = NULL;
  if (L->afmt == ORC_A_FP8_TENSOR) {
    const size_t nr = (size_t)n_tok * K;
    const uint16_t** rp = (const uint16_t**)malloc(sizeof(uint16_t*) * (nr + 1));
    a_all = (double*)malloc(sizeof(double) * (nr * I + 1));
    if (!rp || !a_all) { free(rp); free(a_all); return -1; }
    for (size_t r = 0; r < nr; ++r) rp[r] = h + r * (size_t)I;
    const int rc = tensor_rows(rp, nr, I, a_all);
    free(rp);
    if (rc) { free(a_all); return -1; }
  }
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    double* wr = (double*)malloc(sizeof(double) * (size_t)I);
    if (!a || !wr) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < n_tok; ++i) {
      if (!a || !wr) continue;
      const int t = tokens[i];
      double* orow = out + (size_t)i * H;
      for (int m = 0; m < H; ++m) orow[m] = 0.0;
      for (int j = 0; j < K; ++j) {
        const int e = topk_ids[(size_t)t * K + j];
        if (e < 0 || e >= L->E_total) continue;
        if (a_all) {
          memcpy(a, a_all + ((size_t)i * K + j) * (size_t)I, sizeof(double) * (size_t)I);
        } else if (activation_row(L->afmt, h + ((size_t)i * K + j) * (size_t)I, I, a)) {
#pragma omp atomic write
          err = 1;
          continue;
        }
        const double wj = L->weight_on_input ? 1.0 : (double)topk_weights[(size_t)t * K + j];
        for (int m = 0; m < H; ++m) {
          weight_row(L->wfmt, L->w2, L->w2_scale, e, m, H, I, wr);
          orow[m] += wj * (dot(a, wr, I) + bias_at(L->w2_bias, (size_t)e * H + m));
        }
      }
    }
    free(a);
    free(wr);
  }
  free(a_all);
  return err ? -1 : 0;
}

int orc_forward(const orc_layer* L, const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                const int32_t* tokens, int n_tok, double* out) {
  if (!layer_ok(L) || n_tok < 0) return -1;
  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n_tok * L->K * L->I + 1);
  if (!h) return -1;
  int rc = orc_stage1(L, x, topk_ids, topk_weights, tokens, n_tok, h);
  if (rc == 0) rc = orc_stage2(L, h, topk_ids, topk_weights, tokens, n_tok, out);
  free(h);
  return rc;
}
