/*
 * libmoe -- quantized fused Mixture-of-Experts expert layer for AMD MI355X (gfx950).
 *
 * C ABI.  Pages cited by title and section:
 *   [rocm_aiter_moe]  vLLM API page "vllm.model_executor.layers.fused_moe.experts.rocm_aiter_moe"
 *   [mxfp4.py]        vLLM source page "vllm/model_executor/layers/quantization/mxfp4.py"
 *   [quark_moe]       vLLM API page "vllm.model_executor.layers.quantization.quark.quark_moe"
 *
 * General rules for every entry point below:
 *   - Tensor pointers are DEVICE pointers owned by the caller; tensors are dense
 *     row-major.  The library keeps no pointer after a call returns.
 *   - Calls only enqueue work on `stream` (NULL = the null stream).  They never
 *     allocate device memory, never synchronise the host and never read device
 *     data on the host, so a call may be captured into a HIP graph.  (The one
 *     exception is checked mode, off unless moe_set_checked_mode turns it on.)
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     non-MOE_OK status nothing was enqueued (in checked mode: nothing after the
 *     table check) and moe_last_error() returns a message for the calling thread.
 *     Invalid DEVICE data (an expert id out of range in topk_ids, NaN logits) is not
 *     an error: such slots are dropped as documented per call.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Results are deterministic: the same inputs give bit-identical outputs on
 *     every call (no floating-point atomics anywhere).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* bad shape, pointer, alignment or enum */
  MOE_EUNSUPPORTED = 2,  /* valid request this library does not implement */
  MOE_EWORKSPACE = 3,    /* workspace missing or smaller than moe_experts_workspace_bytes() */
  MOE_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} moe_status;

/* Router score function.  The pages name the softmax top-k router only through its
 * products ([rocm_aiter_moe] inject_shared_expert_weights, rocm_aiter_fused_experts);
 * sigmoid scoring is the DeepSeek-style variant. */
typedef enum moe_score { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

/* Weight formats ([rocm_aiter_moe] derive_aiter_quant_method):
 *   MOE_W_MXFP4        BLOCK_1X32: w1 uint8 [E, 2I, H/2] (two e2m1 codes per byte, the low
 *                      nibble holds the even K index), w1_scale uint8 E8M0 [E, 2I, H/32];
 *                      w2 [E, H, I/2], w2_scale [E, H, I/32]  ([mxfp4.py] Mxfp4MoEMethod.create_weights)
 *   MOE_W_FP8_BLOCK128 BLOCK_128x128: w1 e4m3fn [E, 2I, H], w1_scale fp32 [E, ceil(2I/128), ceil(H/128)];
 *                      w2 [E, H, I], w2_scale fp32 [E, ceil(H/128), ceil(I/128)]  ([rocm_aiter_moe] AiterFp8BlockExperts)
 *   MOE_W_FP8_CHANNEL  PER_TOKEN (per output channel): codes as above, w1_scale fp32 [E, 2I],
 *                      w2_scale fp32 [E, H]  ([rocm_aiter_moe] AiterFp8ChannelExperts)
 *   MOE_W_FP8_TENSOR   PER_TENSOR: codes as above, one fp32 scale per expert and projection:
 *                      w1_scale [E], w2_scale [E]  ([rocm_aiter_moe] AiterFp8TensorExperts)
 *   MOE_W_BF16         unquantised: w1 bf16 [E, 2I, H], w2 bf16 [E, H, I], no scales (pass
 *                      NULL); with MOE_A_BF16 only, the canonical layout only, and block_m
 *                      64 or 128, or 16 when H, I <= 2944 (the 16-row activation tile is
 *                      kept in LDS)  ([rocm_aiter_moe] AiterUnquantizedExperts)
 * In w1 rows [0, I) are the gate projection and rows [I, 2I) the up projection. */
typedef enum moe_wfmt {
  MOE_W_MXFP4 = 0, MOE_W_FP8_BLOCK128 = 1, MOE_W_FP8_CHANNEL = 2, MOE_W_FP8_TENSOR = 3, MOE_W_BF16 = 4
} moe_wfmt;

/* Activation (GEMM input) formats, quantised dynamically ([rocm_aiter_moe]
 * AiterMxfp4Experts, AiterFp8BlockExperts, AiterFp8ChannelExperts):
 *   MOE_A_BF16       no quantisation (w4a16)
 *   MOE_A_MXFP4_G32  codes uint8 [rows, cols/2] (two e2m1 per byte, low nibble = even column),
 *                    scales uint8 E8M0 [rows, cols/32]
 *   MOE_A_FP8_G128   codes e4m3fn [rows, cols], scales fp32 [rows, ceil(cols/128)]
 *   MOE_A_FP8_TOKEN  codes e4m3fn [rows, cols], scales fp32 [rows]
 *   MOE_A_FP8_TENSOR codes e4m3fn [rows, cols], scales fp32 [1]: one scale for the whole
 *                    tensor, the FP8 rule applied to all rows * cols values (the per-tensor
 *                    activation quantisation of PER_TENSOR); used with MOE_W_FP8_TENSOR */
typedef enum moe_afmt {
  MOE_A_BF16 = 0, MOE_A_MXFP4_G32 = 1, MOE_A_FP8_G128 = 2, MOE_A_FP8_TOKEN = 3, MOE_A_FP8_TENSOR = 4
} moe_afmt;

/* Weight memory layout.
 *   MOE_LAYOUT_CANONICAL  the row-major tensors described under moe_wfmt.
 *   MOE_LAYOUT_TILED      the kernel layout written by moe_tile_weights: a one-time
 *                         permutation of the same codes (and, for MXFP4, of the E8M0
 *                         scales) into 16-row x 128-K blocks in the lane order of the MFMA
 *                         operands, so every wavefront load is one contiguous 1 KB run.
 *                         The pages shuffle expert weights into a kernel format once, after
 *                         loading ([mxfp4.py] Mxfp4MoEMethod._setup_kernel,
 *                         process_weights_after_loading); this is that step for this library. */
typedef enum moe_weight_layout { MOE_LAYOUT_CANONICAL = 0, MOE_LAYOUT_TILED = 1 } moe_weight_layout;

/* Gated activation of stage 1 (gate and up are the two w13 rows of an output column,
 * each plus its bias when w1_bias is given):
 *   MOE_ACT_SILU        h = silu(gate) * up, silu(z) = z / (1 + e^-z)
 *                       ([rocm_aiter_moe] AiterExperts: SILU activation, act-and-mul only)
 *   MOE_ACT_SWIGLU_OAI  gate = min(gate, limit), up = clamp(up, -limit, limit) (no clamping
 *                       when limit <= 0), h = gate * sigmoid(alpha * gate) * (up + beta).
 *                       The pages name it (SWIGLUOAI, [rocm_aiter_moe]
 *                       _resolve_aiter_activation) and give alpha 1.702, beta 1.0, limit 7.0
 *                       ([mxfp4.py] Mxfp4MoEMethod.get_fused_moe_quant_config); the formula is
 *                       the published gpt-oss activation those constants belong to. */
typedef enum moe_act { MOE_ACT_SILU = 0, MOE_ACT_SWIGLU_OAI = 1 } moe_act;

/* ------------------------------------------------------------------------------------
 * moe_route_topk -- softmax / sigmoid top-k router with optional shared-expert slots.
 *
 * For every token t: the `topk` largest logits of router_logits[t, 0:E] in descending
 * order (equal logits: lower expert id first).  Weights:
 *   softmax: exp(l_j - l_max) / sum, the sum over the chosen k when `renormalize`
 *            (equal to the renormalised full softmax), else over all E logits;
 *   sigmoid: 1 / (1 + exp(-l_j)), divided by their sum over the chosen k when `renormalize`.
 * Then n_shared shared-expert slots follow: slot topk + s holds expert id E + s with
 * weight shared_weight, the combined routed+shared layout of [rocm_aiter_moe]
 * inject_shared_expert_weights.
 *   router_logits  [T, E] fp32 (input of [mxfp4.py] Mxfp4MoEMethod.apply_monolithic)
 *   topk_ids       [T, topk + n_shared] int32   (written)
 *   topk_weights   [T, topk + n_shared] fp32    (written; dtypes as cast in
 *                  [rocm_aiter_moe] rocm_aiter_fused_experts)
 * Limits: 1 <= E <= 1024, 1 <= topk <= min(E, 32), 0 <= n_shared <= 32, T >= 0.
 * T == 0 enqueues nothing.  Logits must be finite (NaN rows give unspecified ids).
 * ---------------------------------------------------------------------------------- */
moe_status moe_route_topk(const float* router_logits, int T, int E, int topk, moe_score score,
                          int renormalize, int n_shared, float shared_weight,
                          int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_route_grouped_topk -- group-limited top-k router with a score-correction bias.
 *
 * The pages name this router only through the parameters handed to the monolithic
 * kernel ([mxfp4.py] Mxfp4MoEMethod.apply_monolithic: num_expert_group, topk_group,
 * e_score_correction_bias, routed_scaling_factor) and its combined routed + shared
 * output ([rocm_aiter_moe] inject_shared_expert_weights).  Reading (group-limited
 * routing of the DeepSeek-V2/V3 models these parameters come from), per token t:
 *   s[e]    = 1 / (1 + exp(-l[e])) (sigmoid) or the softmax of the whole row;
 *   key[e]  = s[e] + correction_bias[e], or l[e] itself when correction_bias is NULL;
 *   the E experts form num_expert_group contiguous groups of E / num_expert_group; a
 *   group's score is the sum of its two largest keys (with a bias) or its largest key;
 *   the topk_group best groups are kept and the topk best keys among their experts are
 *   the routed slots, best first; equal keys or group scores: lower id first;
 *   weight[j] = s[id_j], divided by the sum of the k weights when `renormalize`, then
 *   multiplied by routed_scaling_factor.
 * Keys, group scores and weights are computed in fp64 (the ids follow the fp64 order).
 * Shared slots follow as in moe_route_topk.
 *   router_logits     [T, E] fp32;  correction_bias [E] fp32 or NULL
 *   topk_ids          [T, topk + n_shared] int32 (written)
 *   topk_weights      [T, topk + n_shared] fp32  (written)
 * Limits: 1 <= E <= 1024; 1 <= num_expert_group <= 64 dividing E; 1 <= topk_group <=
 * num_expert_group; 1 <= topk <= min(32, topk_group * E / num_expert_group);
 * 0 <= n_shared <= 32; T >= 0 (T == 0 enqueues nothing).  Logits must be finite.
 * Errors: MOE_EINVAL for any argument outside these limits, NULL or misaligned pointers.
 * ---------------------------------------------------------------------------------- */
moe_status moe_route_grouped_topk(const float* router_logits, const float* correction_bias, int T, int E,
                                  int topk, int num_expert_group, int topk_group, moe_score score,
                                  int renormalize, float routed_scaling_factor, int n_shared,
                                  float shared_weight, int32_t* topk_ids, float* topk_weights,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_map_experts -- this device's share of an expert-parallel layer.
 *
 * The pages hand an expert map to the fused kernel as its expert mask, with the count of
 * valid token rows ([rocm_aiter_moe] AiterExperts.apply: expert_mask=expert_map,
 * num_local_tokens = expert_tokens_meta.expert_num_tokens).  For every slot (t, j):
 *   local_ids[t, j] = expert_map[topk_ids[t, j]]  if topk_ids[t, j] is in [0, E_global)
 *                                                 and t < *num_local_tokens,
 *                   = -1                          otherwise.
 * expert_map [E_global] int32 holds each global expert's local id on this device (its
 * row in this device's w1/w2) or -1; NULL means the identity.  num_local_tokens is a
 * device int32 scalar or NULL (every row valid).  Feed local_ids to moe_align_sort and
 * moe_experts_forward with E_total = the local expert count: slots with -1 are skipped
 * and the layer's output is this device's partial sum (rows with no local slot are 0).
 *   topk_ids [T, K] int32 (global ids);  local_ids [T, K] int32 (written)
 * Limits: T >= 0, 1 <= K <= 64, 1 <= E_global <= 2^20, T*K < 2^31; map entries must be
 * -1 or valid local ids.  Errors: MOE_EINVAL for arguments outside these limits, NULL or
 * misaligned pointers.
 * ---------------------------------------------------------------------------------- */
moe_status moe_map_experts(const int32_t* topk_ids, const int32_t* expert_map, const int32_t* num_local_tokens,
                           int T, int K, int E_global, int32_t* local_ids, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_align_sort -- stable token->expert sort padded to the GEMM row tile.
 *
 * The flattened slots s = t*K + j (K = slots per token, routed + shared) are grouped by
 * expert id in ascending slot order; each expert's run is padded up to a multiple of
 * block_m rows.  The pages hand this step to the fused kernel as its "moe sorting"
 * dispatch policy and per-expert token counts ([rocm_aiter_moe] rocm_aiter_fused_experts,
 * AiterExperts.apply: expert_num_tokens).
 *   topk_ids        [T, K] int32 (input)
 *   expert_counts   [E_total] int32: slots routed to each expert
 *   expert_offsets  [E_total + 1] int32: first padded row of each expert; the last entry
 *                   is the total number of padded rows
 *   sorted_slots    [moe_sort_capacity(T,K,E_total,block_m)] int32: slot id per padded row,
 *                   T*K for pad rows and for every row past the total
 *   block_expert    [moe_sort_capacity(...) / block_m] int32: owning expert of each
 *                   block of block_m rows, -1 past the total
 *   num_padded      [1] int32: total padded rows (= expert_offsets[E_total])
 * Limits: E_total <= 1024, block_m in {16, 32, 64, 128}, T*K < 2^31 - E_total*block_m.
 * Ids outside [0, E_total) are not placed (their slots are skipped by the layer).
 * ---------------------------------------------------------------------------------- */
size_t moe_sort_capacity(int T, int K, int E_total, int block_m); /* = T*K + E_total*(block_m-1) */
moe_status moe_align_sort(const int32_t* topk_ids, int T, int K, int E_total, int block_m,
                          int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
                          int32_t* block_expert, int32_t* num_padded, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_route_align -- moe_route_topk followed by moe_align_sort (K = topk + n_shared,
 * E_total = E + n_shared), with the same outputs bit for bit.  When E <= 64, T*K <= 4096
 * and T*E <= 8192 both steps run in one launch of one workgroup (logits and ids stay on
 * chip); other shapes take the two separate launches.  Arguments, layouts and limits are those of
 * the two calls, plus E + n_shared <= 1024.  Device pointers; enqueued on `stream`.
 * ---------------------------------------------------------------------------------- */
moe_status moe_route_align(const float* router_logits, int T, int E, int topk, moe_score score,
                           int renormalize, int n_shared, float shared_weight, int block_m,
                           int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                           int32_t* expert_offsets, int32_t* sorted_slots, int32_t* block_expert,
                           int32_t* num_padded, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_quant_act -- dynamic activation quantisation of a bf16 matrix [rows, cols].
 *
 * FP8 (e4m3fn) formats: per group (128 columns, the whole row for MOE_A_FP8_TOKEN, the
 * whole tensor for MOE_A_FP8_TENSOR; the last 128-group of a row may be shorter),
 * s = amax / 448 in IEEE fp32 (s = 1 for an
 * all-zero group) and code = nearest e4m3fn value of x / s (IEEE fp32 division), ties to
 * even, saturating at +-448 ([rocm_aiter_moe] AiterFp8BlockExperts: 128-grouped dynamic
 * activation scale; AiterFp8ChannelExperts: per-token dynamic scale).
 * MXFP4: per 32 columns, shared exponent es = floor(log2 amax) - 2 clamped to [-127, 127]
 * (es = -127 for an all-zero group), scale byte es + 127, code = nearest e2m1 of
 * x * 2^-es, ties to even, saturating at +-6 ([rocm_aiter_moe] AiterMxfp4Experts,
 * MXFP4 dynamic activations; two codes per byte as [quark_moe]
 * QuarkOCP_MX_MoEMethod.get_packed_dim).  The code's sign bit is the sign of x.
 *   x       [rows, cols] bf16;  codes / scales: layouts of moe_afmt above.
 * MOE_A_FP8_TENSOR runs four launches (the scale slot holds the amax until the last one)
 * and needs rows * cols < 2^31.
 * Limits: cols % 32 == 0, cols <= 65536, rows >= 0.  x and codes 16-byte aligned, scales
 * 4-byte aligned.  fmt == MOE_A_BF16 is MOE_EINVAL.
 * ---------------------------------------------------------------------------------- */
moe_status moe_quant_act(const uint16_t* x, int rows, int cols, moe_afmt fmt,
                         uint8_t* codes, void* scales, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_experts_forward -- the expert computation of the fused MoE layer.
 *
 * For every slot (t, j) routed to expert e = topk_ids[t, j] (shared experts are ordinary
 * experts with ids >= the routed count, carried as extra slots):
 *   stage 1  [g | u] = a1[t] . w1[e]^T (+ w1_bias[e])  (g: rows [0, I) of w1, u: rows
 *            [I, 2I); with gate_up_interleaved g and u of column n are rows 2n and 2n+1)
 *            h = bf16( act(g, u) )        fused into the GEMM epilogue (see moe_act)
 *            for quantised activation formats h is re-quantised (a2) in the same format
 *   stage 2  y = a2 . w2[e]^T (+ w2_bias[e]), scaled by topk_weights[t, j]
 *   out[t] = bf16( sum over j = 0..K-1, in ascending j, of the weighted y )
 * (the weighted reduction is part of the expert computation: [rocm_aiter_moe]
 * AiterExperts.finalize_weight_and_reduce_impl is a no-op and the weights apply to the
 * second GEMM's output by default, per AiterFp8ChannelExperts.apply.)
 * a1 is hidden_states itself (MOE_A_BF16) or its quantisation; pass a1_codes/a1_scales
 * from moe_quant_act, or NULL to quantise inside this call.
 * Rows come from moe_align_sort run with the same T, K, E_total and block_m.
 * The workspace holds the intermediate h, the a1/a2 codes and an fp32 per-slot buffer
 * [T*K, H] of unweighted y rows (each product w * y is rounded to fp32 before it is
 * added); its layout is reported by moe_workspace_layout().
 * Limits: H % 32 == 0, I % 32 == 0, H, I <= 65536, 1 <= K <= 64, E_total <= 1024,
 * block_m in {16, 32, 64, 128}; (wfmt, afmt) one of
 *   (MXFP4, BF16) (MXFP4, MXFP4_G32) (FP8_BLOCK128, FP8_G128) (FP8_CHANNEL, FP8_TOKEN)
 *   (FP8_TENSOR, FP8_TENSOR) (BF16, BF16: canonical layout; block_m 64, 128, or 16 with H, I <= 2944)
 * (others: MOE_EUNSUPPORTED).  Pointers to 16-byte aligned memory.
 * ---------------------------------------------------------------------------------- */
typedef struct moe_forward_args {
  int T, H, I, E_total, K, block_m;
  moe_wfmt wfmt;
  moe_afmt afmt;
  moe_act act;
  const uint16_t* hidden_states;                 /* [T, H] bf16 */
  const uint8_t* a1_codes; const void* a1_scales; /* optional pre-quantised hidden_states */
  const uint8_t* w1; const void* w1_scale;       /* see moe_wfmt */
  const uint8_t* w2; const void* w2_scale;
  const int32_t* topk_ids;                       /* [T, K] */
  const float* topk_weights;                     /* [T, K] */
  const int32_t* sorted_slots;                   /* from moe_align_sort */
  const int32_t* block_expert;
  const int32_t* num_padded;
  uint16_t* out;                                 /* [T, H] bf16, written */
  void* workspace;
  size_t workspace_bytes;
  moe_weight_layout weight_layout;               /* layout of w1 and w2 (both the same) */
  float act_alpha, act_beta, act_limit;          /* MOE_ACT_SWIGLU_OAI parameters (else unused) */
  int gate_up_interleaved;                       /* 0: w1 rows [gate_0..gate_{I-1}, up_0..up_{I-1}];
                                                    1: gate_n, up_n alternate (the INTERLEAVE gate
                                                    mode of [rocm_aiter_moe]
                                                    mxfp4_w4a16_extra_kwargs); not for FP8_BLOCK128 */
  const uint16_t* w1_bias;                       /* bf16 [E_total, 2I] in w1 row order, or NULL;
                                                    4-byte aligned (bias pairs are loaded as words) */
  const uint16_t* w2_bias;                       /* bf16 [E_total, H], or NULL, 4-byte aligned
                                                    ([mxfp4.py] create_weights: w13_bias, w2_bias) */
  int apply_router_weight_on_input;              /* 1: topk_weights scale both stage-1
                                                    projections and the sum over slots is
                                                    unweighted; needs K == 1 ([rocm_aiter_moe]
                                                    AiterFp8TensorExperts.apply: tkw1) */
} moe_forward_args;

/* Byte offsets into the workspace (each 256-byte aligned); 0 size = not used. */
typedef struct moe_workspace_layout_t {
  size_t h_off, h_bytes;           /* bf16 [cap, I]: stage-1 output in sorted-row order */
  size_t a1_codes_off, a1_codes_bytes, a1_scales_off, a1_scales_bytes; /* quantised hidden_states */
  size_t a2_codes_off, a2_codes_bytes, a2_scales_off, a2_scales_bytes; /* quantised h, sorted rows */
  size_t ybuf_off, ybuf_bytes;     /* fp32 [T*K, H]: stage-2 rows (unweighted) by slot id */
  size_t total;
} moe_workspace_layout_t;

size_t moe_experts_workspace_bytes(const moe_forward_args* a);
moe_status moe_workspace_layout(const moe_forward_args* a, moe_workspace_layout_t* layout);
moe_status moe_experts_forward(const moe_forward_args* a, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_experts_forward_noalloc -- moe_experts_forward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, launches and results bit for bit, with the workspace
 * taken from a scratch area the library owns instead of a->workspace (a->workspace and
 * a->workspace_bytes are ignored).  The call allocates nothing, ever.
 * The scratch is MOE_NOALLOC_SCRATCH_BYTES (64 MiB) of device memory per device the
 * library runs on, held until the process ends; it fits a call whose
 * moe_experts_workspace_bytes() is at most that (e.g. the decode shapes: T = 64, H = I =
 * 2880, 32 experts, top-4 need about 7 MB).  Larger calls return MOE_EWORKSPACE with
 * nothing enqueued.  Every call on one device shares that device's scratch and leaves the
 * last call's intermediates in it: calls that may overlap on one device (two streams, two
 * host threads) race and must be ordered by the caller.  Arguments, limits and errors are
 * otherwise those of moe_experts_forward.
 * ---------------------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_experts_forward_noalloc(const moe_forward_args* a, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_set_checked_mode -- a debugging aid for callers that build the routing tables
 * themselves.  With `on` nonzero (process-wide; off by default), moe_experts_forward and
 * moe_experts_forward_noalloc first check, on the device, the tables the expert kernels
 * index with: num_padded in [0, capacity] and a multiple of block_m; every sorted_slots
 * entry below num_padded in [0, T*K] (T*K is the pad sentinel); every block_expert entry
 * below num_padded / block_m in [-1, E_total).  The call then waits for the stream; tables
 * that fail return MOE_EINVAL (moe_last_error() names the first entry found) with nothing
 * further enqueued, so a corrupt table is reported instead of being read out of bounds.
 * Each checked call costs one small kernel and a stream synchronisation, and is therefore
 * not capturable in a HIP graph.  moe_layer_forward's fused small-batch path builds its
 * tables inside the first GEMM kernel and is not checked.  Returns MOE_OK.
 * ---------------------------------------------------------------------------------- */
moe_status moe_set_checked_mode(int on);

/* ------------------------------------------------------------------------------------
 * moe_layer_forward -- the whole layer from router logits: moe_route_align (E = E_total -
 * n_shared routed experts, topk = K - n_shared, the block_m of `a`) writing into the
 * routing buffers that `a` names, then moe_experts_forward(a).  The pages' layer takes
 * router_logits and performs the top-k selection before the expert kernels
 * ([rocm_aiter_moe] rocm_aiter_fused_experts; [mxfp4.py] Mxfp4MoEMethod.apply_monolithic).
 *   router_logits   [T, E] fp32
 *   a->topk_ids, a->topk_weights, a->sorted_slots, a->block_expert, a->num_padded
 *                   OUTPUTS here (layouts of moe_route_align / moe_align_sort), despite
 *                   the const in the struct, which describes moe_experts_forward
 *   expert_counts [E_total], expert_offsets [E_total + 1]: outputs as moe_align_sort
 * Every output equals that of the two separate calls bit for bit.  For a batch with
 * block_m == 16, E <= 64, T*K <= 4096, T*E <= 8192 and the stage-1 LDS budget met (no
 * apply_router_weight_on_input) the stage-1 kernel routes and sorts the batch itself,
 * saving a launch; otherwise the separate launches run.  Limits: those of the two calls,
 * 0 <= n_shared < K.  Device pointers; enqueued on `stream`.
 * ---------------------------------------------------------------------------------- */
moe_status moe_layer_forward(const moe_forward_args* a, const float* router_logits, moe_score score,
                             int renormalize, int n_shared, float shared_weight, int32_t* expert_counts,
                             int32_t* expert_offsets, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_tile_weights -- one-time permutation of one weight tensor ([E, N, K] codes in the
 * canonical layout of `wfmt`, i.e. w1 with N = 2I, K = H or w2 with N = H, K = I) into
 * MOE_LAYOUT_TILED.  Block (e, n16, c) holds rows [16*n16, 16*n16+16) and K elements
 * [128c, 128c+128) (zero past K); lane l = 16*g + r of a wavefront owns row r, elements
 * [128c + 32g, +32):
 *   MXFP4: 1088 bytes per block = 64 lanes x 16 code bytes, then 64 E8M0 bytes (lane order);
 *          w_scale must be the canonical [E, N, K/32] bytes and is folded into `out`
 *          (forward calls on tiled MXFP4 weights ignore w1_scale / w2_scale).
 *   FP8:   2048 bytes per block = 64 lanes x 16 bytes (elements 32g..32g+15), then
 *          64 lanes x 16 bytes (32g+16..32g+31); scales stay in their canonical arrays and
 *          are still passed to moe_experts_forward.
 * Blocks are ordered [E][N/16][ceil(K/128)].  `out` holds moe_tiled_weight_bytes() bytes.
 * Limits: N % 16 == 0, K % 32 == 0.  Device pointers; enqueued on `stream`.
 * ---------------------------------------------------------------------------------- */
size_t moe_tiled_weight_bytes(moe_wfmt wfmt, int E, int N, int K);
moe_status moe_tile_weights(moe_wfmt wfmt, int E, int N, int K, const uint8_t* w, const void* w_scale,
                            uint8_t* out, hipStream_t stream);

/* Whether a (wfmt, afmt, act, H, I) combination is implemented (MOE_OK) or not
 * (MOE_EUNSUPPORTED / MOE_EINVAL, with the reason in moe_last_error()); the analogue of
 * [rocm_aiter_moe] AiterExperts.is_supported_config. */
moe_status moe_supports(moe_wfmt wfmt, moe_afmt afmt, moe_act act, int H, int I);

/* A row tile for moe_align_sort / moe_experts_forward suited to T*K slots over E_total
 * experts, weight format wfmt and weight layout (host-side heuristic; any value in
 * {16, 32, 64, 128} is valid): 16 rows for up to 16 rows per expert on average (FP8
 * 128x128-block weights: up to 1), else 64, except 128 for FP8 block weights in the
 * tiled layout with at least 64 rows per expert, where the LDS-staged 128-row kernel is
 * the faster one.  32-row blocks are never picked (measured slower than 64). */
int moe_pick_block_m(int T, int K, int E_total, moe_wfmt wfmt, moe_weight_layout layout);

/* Profiling hook.  While enabled (count == 4), moe_experts_forward calls made on this
 * thread record, on their stream, events[0] just before the stage-1 GEMM, events[1] just
 * after it, events[2] after the stage-2 GEMM and events[3] after the combine, so a caller
 * can time the kernels inside a running pipeline.  count == 0 disables it.  The events are
 * created and owned by the caller and must stay valid while enabled. */
moe_status moe_profile_events(hipEvent_t* events, int count);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
