// C-ABI entry points of libmoe: host-side validation, workspace layout and the
// launch sequence.  Nothing here allocates, synchronises or reads device memory.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/moe.h"
#include "moe_internal.h"

// Workspace of moe_experts_forward_noalloc: device memory the library owns, one copy per
// device (the code object's copy on that device), held until the process ends.  Host code
// never names this array as an address: its device address comes from hipGetSymbolAddress
// (scratch_ptr below).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];
// Checked mode: the verdict of the last table check on this device (code, entry index).
static __device__ int32_t check_result[2];

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_prof[4] = {nullptr, nullptr, nullptr, nullptr};
thread_local bool g_prof_on = false;

hipError_t prof_mark(int i, hipStream_t stream) {
  return g_prof_on ? hipEventRecord(g_prof[i], stream) : hipSuccess;
}

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

moe_status ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_bm(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// bytes of codes / scales of a [rows, cols] matrix in activation format f
size_t code_bytes(int f, size_t rows, size_t cols) {
  if (f == MOE_A_MXFP4_G32) return rows * cols / 2;
  if (f == MOE_A_FP8_G128 || f == MOE_A_FP8_TOKEN || f == MOE_A_FP8_TENSOR) return rows * cols;
  return 0;
}
size_t scale_bytes(int f, size_t rows, size_t cols) {
  if (f == MOE_A_MXFP4_G32) return rows * (cols / 32);
  if (f == MOE_A_FP8_G128) return rows * ((cols + 127) / 128) * 4;
  if (f == MOE_A_FP8_TOKEN) return rows * 4;
  if (f == MOE_A_FP8_TENSOR) return 4;
  return 0;
}

bool pair_supported(int wf, int af) {
  return (wf == MOE_W_MXFP4 && (af == MOE_A_BF16 || af == MOE_A_MXFP4_G32)) ||
         (wf == MOE_W_FP8_BLOCK128 && af == MOE_A_FP8_G128) || (wf == MOE_W_FP8_CHANNEL && af == MOE_A_FP8_TOKEN) ||
         (wf == MOE_W_FP8_TENSOR && af == MOE_A_FP8_TENSOR) || (wf == MOE_W_BF16 && af == MOE_A_BF16);
}

moe_status check_shapes(const moe_forward_args* a) {
  if (!a) return fail(MOE_EINVAL, "moe_experts_forward: args is NULL");
  if (a->T < 0) return fail(MOE_EINVAL, "T must be >= 0 (got %d)", a->T);
  if (a->H <= 0 || a->H % 32 || a->H > 65536) return fail(MOE_EINVAL, "H must be a positive multiple of 32 <= 65536 (got %d)", a->H);
  if (a->I <= 0 || a->I % 32 || a->I > 65536) return fail(MOE_EINVAL, "I must be a positive multiple of 32 <= 65536 (got %d)", a->I);
  if (a->E_total < 1 || a->E_total > 1024) return fail(MOE_EINVAL, "E_total must be in [1, 1024] (got %d)", a->E_total);
  if (a->K < 1 || a->K > 64) return fail(MOE_EINVAL, "K must be in [1, 64] (got %d)", a->K);
  if (!valid_bm(a->block_m)) return fail(MOE_EINVAL, "block_m must be 16, 32, 64 or 128 (got %d)", a->block_m);
  if ((long long)a->T * a->K + (long long)a->E_total * a->block_m >= 0x7FFFFFFFLL)
    return fail(MOE_EINVAL, "T*K too large");
  if (a->act != MOE_ACT_SILU && a->act != MOE_ACT_SWIGLU_OAI)
    return fail(MOE_EUNSUPPORTED, "activation %d is not implemented (SiLU-and-mul, SwiGLU-OAI)", (int)a->act);
  if (a->gate_up_interleaved != 0 && a->gate_up_interleaved != 1)
    return fail(MOE_EINVAL, "gate_up_interleaved must be 0 or 1 (got %d)", a->gate_up_interleaved);
  if (a->apply_router_weight_on_input != 0 && a->apply_router_weight_on_input != 1)
    return fail(MOE_EINVAL, "apply_router_weight_on_input must be 0 or 1 (got %d)", a->apply_router_weight_on_input);
  if (a->apply_router_weight_on_input && a->K != 1)
    return fail(MOE_EINVAL, "the router weight goes on the input only with one slot per token (K = %d)", a->K);
  if (a->gate_up_interleaved && a->wfmt == MOE_W_FP8_BLOCK128)
    return fail(MOE_EUNSUPPORTED, "interleaved gate/up rows would split FP8 128x128 scale blocks");
  if (a->wfmt < MOE_W_MXFP4 || a->wfmt > MOE_W_BF16) return fail(MOE_EINVAL, "unknown weight format %d", (int)a->wfmt);
  if (a->afmt < MOE_A_BF16 || a->afmt > MOE_A_FP8_TENSOR) return fail(MOE_EINVAL, "unknown activation format %d", (int)a->afmt);
  if (!pair_supported(a->wfmt, a->afmt))
    return fail(MOE_EUNSUPPORTED, "weight format %d with activation format %d is not implemented", (int)a->wfmt,
                (int)a->afmt);
  if (a->weight_layout != MOE_LAYOUT_CANONICAL && a->weight_layout != MOE_LAYOUT_TILED)
    return fail(MOE_EINVAL, "unknown weight layout %d", (int)a->weight_layout);
  if (a->wfmt == MOE_W_BF16 && a->weight_layout != MOE_LAYOUT_CANONICAL)
    return fail(MOE_EUNSUPPORTED, "bf16 weights use the canonical layout");
  if (a->wfmt == MOE_W_BF16 && a->block_m == 32)
    return fail(MOE_EUNSUPPORTED, "bf16 weights run on 16-, 64- or 128-row blocks (block_m %d)", a->block_m);
  if (a->wfmt == MOE_W_BF16 && a->block_m == 16 &&
      !(moe::persist_launch_fits(moe::kABf16, 1, a->H, 2 * a->I, a->w1_bias != nullptr) &&
        moe::persist_launch_fits(moe::kABf16, 2, a->I, a->H, a->w2_bias != nullptr)))
    return fail(MOE_EUNSUPPORTED, "bf16 weights on 16-row blocks need H, I <= 2944 (the activation tile in LDS)");
  return ok();
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

moe_status moe_profile_events(hipEvent_t* events, int count) {
  if (count == 0) {
    g_prof_on = false;
    return ok();
  }
  if (count != 4 || !events) return fail(MOE_EINVAL, "moe_profile_events: pass 4 events, or count 0 to disable");
  for (int i = 0; i < 4; ++i) g_prof[i] = events[i];
  g_prof_on = true;
  return ok();
}

size_t moe_tiled_weight_bytes(moe_wfmt wfmt, int E, int N, int K) {
  if (E < 0 || N < 0 || K < 0 || N % 16 || K % 32) return 0;
  const size_t blocks = (size_t)E * (N / 16) * ((K + 127) / 128);
  if (wfmt == MOE_W_MXFP4) return blocks * 1088;
  if (wfmt == MOE_W_FP8_BLOCK128 || wfmt == MOE_W_FP8_CHANNEL || wfmt == MOE_W_FP8_TENSOR) return blocks * 2048;
  return 0;
}

moe_status moe_tile_weights(moe_wfmt wfmt, int E, int N, int K, const uint8_t* w, const void* w_scale, uint8_t* out,
                            hipStream_t stream) {
  if (wfmt < MOE_W_MXFP4 || wfmt > MOE_W_FP8_TENSOR) return fail(MOE_EINVAL, "moe_tile_weights: unknown weight format %d", (int)wfmt);
  if (E < 0 || N <= 0 || K <= 0 || N % 16 || K % 32 || K > 65536)
    return fail(MOE_EINVAL, "moe_tile_weights: need N %% 16 == 0, K %% 32 == 0, K <= 65536 (got N=%d, K=%d)", N, K);
  if (E > 0 && (!w || !out || (wfmt == MOE_W_MXFP4 && !w_scale))) return fail(MOE_EINVAL, "moe_tile_weights: NULL pointer");
  if (!aligned(w, 16) || !aligned(out, 16)) return fail(MOE_EINVAL, "moe_tile_weights: w and out must be 16-byte aligned");
  return hip_status(moe::launch_tile_weights((int)wfmt, E, N, K, w, w_scale, out, stream), "moe_tile_weights launch");
}

moe_status moe_supports(moe_wfmt wfmt, moe_afmt afmt, moe_act act, int H, int I) {
  if (act != MOE_ACT_SILU && act != MOE_ACT_SWIGLU_OAI)
    return fail(MOE_EUNSUPPORTED, "activation %d is not implemented (SiLU-and-mul, SwiGLU-OAI)", (int)act);
  if (wfmt < MOE_W_MXFP4 || wfmt > MOE_W_BF16) return fail(MOE_EINVAL, "unknown weight format %d", (int)wfmt);
  if (afmt < MOE_A_BF16 || afmt > MOE_A_FP8_TENSOR) return fail(MOE_EINVAL, "unknown activation format %d", (int)afmt);
  if (!pair_supported(wfmt, afmt))
    return fail(MOE_EUNSUPPORTED, "weight format %d with activation format %d is not implemented", (int)wfmt, (int)afmt);
  if (H <= 0 || H % 32 || I <= 0 || I % 32 || H > 65536 || I > 65536)
    return fail(MOE_EINVAL, "H and I must be positive multiples of 32 <= 65536 (got %d, %d)", H, I);
  return ok();
}

int moe_pick_block_m(int T, int K, int E_total, moe_wfmt wfmt, moe_weight_layout layout) {
  if (E_total <= 0) return 16;
  // Measured on MI355X (bench steps, every format): 16-row blocks win up to ~16 rows per
  // expert (the persistent kernel, with the route fused in), except for FP8 block weights
  // with more than one row per expert (T = 32 .. 256 over 257 experts: 64 rows 12-22%
  // faster); above that 64-row blocks win everywhere, 32-row blocks never (1.1-2.6x slower
  // than 64 at 20-36 rows per expert).
  const double rows = (double)T * K / E_total;
  if (rows <= 16 && !(wfmt == MOE_W_FP8_BLOCK128 && rows > 1)) return 16;
  // FP8 block weights, tiled: the 128-row LDS-staged kernel (4.13 against 4.30 ms per step
  // at T = 4096, 257 experts, top-8 + 1 shared; 2.85 against 2.91 at T = 2048)
  if (wfmt == MOE_W_FP8_BLOCK128 && layout == MOE_LAYOUT_TILED && rows >= 64) return 128;
  return 64;  // 64-row blocks keep two waves per SIMD resident (measured faster than 128)
}

moe_status moe_route_topk(const float* router_logits, int T, int E, int topk, moe_score score, int renormalize,
                          int n_shared, float shared_weight, int32_t* topk_ids, float* topk_weights,
                          hipStream_t stream) {
  if (T < 0) return fail(MOE_EINVAL, "moe_route_topk: T must be >= 0 (got %d)", T);
  if (E < 1 || E > 1024) return fail(MOE_EINVAL, "moe_route_topk: E must be in [1, 1024] (got %d)", E);
  if (topk < 1 || topk > E || topk > 32) return fail(MOE_EINVAL, "moe_route_topk: topk must be in [1, min(E, 32)] (got %d)", topk);
  if (n_shared < 0 || n_shared > 32) return fail(MOE_EINVAL, "moe_route_topk: n_shared must be in [0, 32] (got %d)", n_shared);
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return fail(MOE_EINVAL, "moe_route_topk: unknown score %d", (int)score);
  if (T > 0 && (!router_logits || !topk_ids || !topk_weights)) return fail(MOE_EINVAL, "moe_route_topk: NULL pointer");
  if (!aligned(router_logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
    return fail(MOE_EINVAL, "moe_route_topk: pointers must be 4-byte aligned");
  return hip_status(moe::launch_route_topk(router_logits, T, E, topk, (int)score, renormalize ? 1 : 0, n_shared,
                                           shared_weight, topk_ids, topk_weights, stream),
                    "moe_route_topk launch");
}

moe_status moe_route_grouped_topk(const float* router_logits, const float* correction_bias, int T, int E, int topk,
                                  int num_expert_group, int topk_group, moe_score score, int renormalize,
                                  float routed_scaling_factor, int n_shared, float shared_weight, int32_t* topk_ids,
                                  float* topk_weights, hipStream_t stream) {
  const char* fn = "moe_route_grouped_topk";
  if (T < 0) return fail(MOE_EINVAL, "%s: T must be >= 0 (got %d)", fn, T);
  if (E < 1 || E > 1024) return fail(MOE_EINVAL, "%s: E must be in [1, 1024] (got %d)", fn, E);
  if (num_expert_group < 1 || num_expert_group > 64 || E % num_expert_group != 0)
    return fail(MOE_EINVAL, "%s: num_expert_group must be in [1, 64] and divide E (got %d, E = %d)", fn,
                num_expert_group, E);
  if (topk_group < 1 || topk_group > num_expert_group)
    return fail(MOE_EINVAL, "%s: topk_group must be in [1, num_expert_group] (got %d)", fn, topk_group);
  if (topk < 1 || topk > 32 || topk > topk_group * (E / num_expert_group))
    return fail(MOE_EINVAL, "%s: topk must be in [1, min(32, topk_group * E / num_expert_group)] (got %d)", fn, topk);
  if (n_shared < 0 || n_shared > 32) return fail(MOE_EINVAL, "%s: n_shared must be in [0, 32] (got %d)", fn, n_shared);
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return fail(MOE_EINVAL, "%s: unknown score %d", fn, (int)score);
  if (T > 0 && (!router_logits || !topk_ids || !topk_weights)) return fail(MOE_EINVAL, "%s: NULL pointer", fn);
  if (!aligned(router_logits, 4) || !aligned(correction_bias, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
    return fail(MOE_EINVAL, "%s: pointers must be 4-byte aligned", fn);
  return hip_status(moe::launch_route_grouped_topk(router_logits, correction_bias, T, E, topk, num_expert_group,
                                                   topk_group, (int)score, renormalize ? 1 : 0, routed_scaling_factor,
                                                   n_shared, shared_weight, topk_ids, topk_weights, stream),
                    "moe_route_grouped_topk launch");
}

moe_status moe_map_experts(const int32_t* topk_ids, const int32_t* expert_map, const int32_t* num_local_tokens,
                           int T, int K, int E_global, int32_t* local_ids, hipStream_t stream) {
  const char* fn = "moe_map_experts";
  if (T < 0) return fail(MOE_EINVAL, "%s: T must be >= 0 (got %d)", fn, T);
  if (K < 1 || K > 64) return fail(MOE_EINVAL, "%s: K must be in [1, 64] (got %d)", fn, K);
  if (E_global < 1 || E_global > (1 << 20)) return fail(MOE_EINVAL, "%s: E_global must be in [1, 2^20] (got %d)", fn, E_global);
  if (T > 0 && (!topk_ids || !local_ids)) return fail(MOE_EINVAL, "%s: NULL pointer", fn);
  if ((long long)T * K > 0x7FFFFFFFLL) return fail(MOE_EINVAL, "%s: T*K too large", fn);
  if (!aligned(topk_ids, 4) || !aligned(expert_map, 4) || !aligned(num_local_tokens, 4) || !aligned(local_ids, 4))
    return fail(MOE_EINVAL, "%s: pointers must be 4-byte aligned", fn);
  return hip_status(moe::launch_map_experts(topk_ids, expert_map, num_local_tokens, T, K, E_global, local_ids, stream),
                    "moe_map_experts launch");
}

size_t moe_sort_capacity(int T, int K, int E_total, int block_m) {
  if (T < 0 || K < 0 || E_total < 0 || block_m < 1) return 0;
  return (size_t)T * K + (size_t)E_total * (block_m - 1);
}

moe_status moe_align_sort(const int32_t* topk_ids, int T, int K, int E_total, int block_m, int32_t* expert_counts,
                          int32_t* expert_offsets, int32_t* sorted_slots, int32_t* block_expert, int32_t* num_padded,
                          hipStream_t stream) {
  if (T < 0) return fail(MOE_EINVAL, "moe_align_sort: T must be >= 0 (got %d)", T);
  if (K < 1 || K > 64) return fail(MOE_EINVAL, "moe_align_sort: K must be in [1, 64] (got %d)", K);
  if (E_total < 1 || E_total > 1024) return fail(MOE_EINVAL, "moe_align_sort: E_total must be in [1, 1024] (got %d)", E_total);
  if (!valid_bm(block_m)) return fail(MOE_EINVAL, "moe_align_sort: block_m must be 16, 32, 64 or 128 (got %d)", block_m);
  if ((long long)T * K + (long long)E_total * block_m >= 0x7FFFFFFFLL) return fail(MOE_EINVAL, "moe_align_sort: T*K too large");
  if (!expert_counts || !expert_offsets || !sorted_slots || !block_expert || !num_padded || (T > 0 && !topk_ids))
    return fail(MOE_EINVAL, "moe_align_sort: NULL pointer");
  return hip_status(moe::launch_align_sort(topk_ids, T, K, E_total, block_m, expert_counts, expert_offsets,
                                           sorted_slots, block_expert, num_padded, stream),
                    "moe_align_sort launch");
}

}  // extern "C"

namespace {

moe_status check_route_align(const char* fn, const float* router_logits, int T, int E, int topk, moe_score score,
                             int n_shared, int block_m, const int32_t* topk_ids, const float* topk_weights,
                             const int32_t* expert_counts, const int32_t* expert_offsets, const int32_t* sorted_slots,
                             const int32_t* block_expert, const int32_t* num_padded) {
  if (T < 0) return fail(MOE_EINVAL, "%s: T must be >= 0 (got %d)", fn, T);
  if (E < 1 || E > 1024) return fail(MOE_EINVAL, "%s: E must be in [1, 1024] (got %d)", fn, E);
  if (topk < 1 || topk > E || topk > 32) return fail(MOE_EINVAL, "%s: topk must be in [1, min(E, 32)] (got %d)", fn, topk);
  if (n_shared < 0 || n_shared > 32) return fail(MOE_EINVAL, "%s: n_shared must be in [0, 32] (got %d)", fn, n_shared);
  if (E + n_shared > 1024) return fail(MOE_EINVAL, "%s: E + n_shared must be <= 1024 (got %d)", fn, E + n_shared);
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return fail(MOE_EINVAL, "%s: unknown score %d", fn, (int)score);
  if (!valid_bm(block_m)) return fail(MOE_EINVAL, "%s: block_m must be 16, 32, 64 or 128 (got %d)", fn, block_m);
  const int K = topk + n_shared, E_total = E + n_shared;
  if ((long long)T * K + (long long)E_total * block_m >= 0x7FFFFFFFLL) return fail(MOE_EINVAL, "%s: T*K too large", fn);
  if (!expert_counts || !expert_offsets || !sorted_slots || !block_expert || !num_padded ||
      (T > 0 && (!router_logits || !topk_ids || !topk_weights)))
    return fail(MOE_EINVAL, "%s: NULL pointer", fn);
  if (!aligned(router_logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
    return fail(MOE_EINVAL, "%s: pointers must be 4-byte aligned", fn);
  return ok();
}

}  // namespace

extern "C" {

moe_status moe_route_align(const float* router_logits, int T, int E, int topk, moe_score score, int renormalize,
                           int n_shared, float shared_weight, int block_m, int32_t* topk_ids, float* topk_weights,
                           int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
                           int32_t* block_expert, int32_t* num_padded, hipStream_t stream) {
  moe_status st0 = check_route_align("moe_route_align", router_logits, T, E, topk, score, n_shared, block_m, topk_ids,
                                     topk_weights, expert_counts, expert_offsets, sorted_slots, block_expert, num_padded);
  if (st0 != MOE_OK) return st0;
  const int K = topk + n_shared, E_total = E + n_shared;
  if (moe::route_sort_fusable(T, E, K))
    return hip_status(moe::launch_route_sort(router_logits, T, E, topk, (int)score, renormalize ? 1 : 0, n_shared,
                                             shared_weight, block_m, topk_ids, topk_weights, expert_counts,
                                             expert_offsets, sorted_slots, block_expert, num_padded, stream),
                      "moe_route_align launch");
  moe_status st = hip_status(moe::launch_route_topk(router_logits, T, E, topk, (int)score, renormalize ? 1 : 0,
                                                    n_shared, shared_weight, topk_ids, topk_weights, stream),
                             "moe_route_align route launch");
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_align_sort(topk_ids, T, K, E_total, block_m, expert_counts, expert_offsets,
                                           sorted_slots, block_expert, num_padded, stream),
                    "moe_route_align sort launch");
}

moe_status moe_quant_act(const uint16_t* x, int rows, int cols, moe_afmt fmt, uint8_t* codes, void* scales,
                         hipStream_t stream) {
  if (fmt != MOE_A_MXFP4_G32 && fmt != MOE_A_FP8_G128 && fmt != MOE_A_FP8_TOKEN && fmt != MOE_A_FP8_TENSOR)
    return fail(MOE_EINVAL, "moe_quant_act: format %d has no quantiser", (int)fmt);
  if (rows < 0) return fail(MOE_EINVAL, "moe_quant_act: rows must be >= 0 (got %d)", rows);
  if (cols <= 0 || cols % 32 || cols > 65536) return fail(MOE_EINVAL, "moe_quant_act: cols must be a positive multiple of 32 <= 65536 (got %d)", cols);
  if (rows > 0 && (!x || !codes || !scales)) return fail(MOE_EINVAL, "moe_quant_act: NULL pointer");
  if (fmt == MOE_A_FP8_TENSOR && (long long)rows * cols >= 0x7FFFFFFFLL)
    return fail(MOE_EINVAL, "moe_quant_act: per-tensor quantisation needs rows * cols < 2^31");
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return fail(MOE_EINVAL, "moe_quant_act: x and codes must be 16-byte aligned, scales 4-byte aligned");
  return hip_status(moe::launch_quant_act(x, rows, cols, (int)fmt, nullptr, codes, scales, stream), "moe_quant_act launch");
}

moe_status moe_workspace_layout(const moe_forward_args* a, moe_workspace_layout_t* L) {
  moe_status st = check_shapes(a);
  if (st != MOE_OK) return st;
  if (!L) return fail(MOE_EINVAL, "moe_workspace_layout: layout is NULL");
  memset(L, 0, sizeof *L);
  const size_t cap = moe_sort_capacity(a->T, a->K, a->E_total, a->block_m);
  size_t off = 0;
  auto take = [&](size_t bytes, size_t& o, size_t& b) {
    b = bytes;
    o = bytes ? off : 0;
    off = round_up(off + bytes, 256);
  };
  take(cap * (size_t)a->I * 2, L->h_off, L->h_bytes);
  if (a->afmt != MOE_A_BF16 && a->a1_codes == nullptr) {
    take(code_bytes(a->afmt, a->T, a->H), L->a1_codes_off, L->a1_codes_bytes);
    take(scale_bytes(a->afmt, a->T, a->H), L->a1_scales_off, L->a1_scales_bytes);
  }
  if (a->afmt != MOE_A_BF16) {
    take(code_bytes(a->afmt, cap, a->I), L->a2_codes_off, L->a2_codes_bytes);
    take(scale_bytes(a->afmt, cap, a->I), L->a2_scales_off, L->a2_scales_bytes);
  }
  take((size_t)a->T * a->K * a->H * 4, L->ybuf_off, L->ybuf_bytes);
  L->total = off;
  return ok();
}

size_t moe_experts_workspace_bytes(const moe_forward_args* a) {
  moe_workspace_layout_t L;
  if (moe_workspace_layout(a, &L) != MOE_OK) return 0;
  return L.total;
}

}  // extern "C"

namespace {

std::atomic<int> g_checked{0};  // moe_set_checked_mode

// Checked mode: the routing tables a forward call reads, against the bounds its kernels
// index with (the weights by block owner, the token rows and per-slot rows by slot).  One
// workgroup; result[0] = 0 (valid) or the code of the first violation claimed (1: padded
// total, 2: sorted slot, 3: block owner), result[1] = the offending value or entry.  Reads
// only sorted[0, num_padded) and owner[0, num_padded / bm), after num_padded is checked
// against the capacity the caller's buffers hold.
__global__ __launch_bounds__(1024) void check_tables_kernel(const int32_t* __restrict__ sorted,
                                                            const int32_t* __restrict__ owner,
                                                            const int32_t* __restrict__ num_padded, int cap, int bm,
                                                            int TK, int E, int32_t* __restrict__ result) {
  __shared__ int code, where;
  const int tid = (int)threadIdx.x;
  const int np = num_padded[0];
  if (tid == 0) {
    const bool bad = np < 0 || np > cap || np % bm != 0;
    code = bad ? 1 : 0;
    where = np;
  }
  __syncthreads();
  if (code == 0) {
    for (int q = tid; q < np; q += (int)blockDim.x) {
      const int s = sorted[q];
      if ((s < 0 || s > TK) && atomicCAS(&code, 0, 2) == 0) where = q;
    }
    for (int b = tid; b < np / bm; b += (int)blockDim.x) {
      const int e = owner[b];
      if ((e < -1 || e >= E) && atomicCAS(&code, 0, 3) == 0) where = b;
    }
  }
  __syncthreads();
  if (tid == 0) {
    result[0] = code;
    result[1] = where;
  }
}

// Device address of check_result on the current device (looked up once per device).
int32_t* check_result_ptr(hipError_t* err) {
  static std::atomic<void*> ptrs[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_result));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    ptrs[dev].store(p, std::memory_order_release);
  }
  *err = hipSuccess;
  return (int32_t*)p;
}

// Runs check_tables_kernel on the call's tables and waits for its verdict.
moe_status check_tables(const moe_forward_args* a, size_t cap, hipStream_t stream) {
  hipError_t e = hipSuccess;
  int32_t* res = check_result_ptr(&e);
  if (!res) return hip_status(e, "checked mode: result address");
  check_tables_kernel<<<1, 1024, 0, stream>>>(a->sorted_slots, a->block_expert, a->num_padded, (int)cap, a->block_m,
                                              a->T * a->K, a->E_total, res);
  if ((e = hipGetLastError()) != hipSuccess) return hip_status(e, "checked mode: table check launch");
  int32_t host[2] = {0, 0};
  if ((e = hipMemcpyAsync(host, res, sizeof host, hipMemcpyDeviceToHost, stream)) != hipSuccess ||
      (e = hipStreamSynchronize(stream)) != hipSuccess)
    return hip_status(e, "checked mode: table check result");
  switch (host[0]) {
    case 0:
      return ok();
    case 1:
      return fail(MOE_EINVAL, "checked mode: num_padded = %d, but it must be a multiple of block_m %d in [0, %zu]",
                  host[1], a->block_m, cap);
    case 2:
      return fail(MOE_EINVAL, "checked mode: sorted_slots[%d] is outside [0, T*K = %d]", host[1], a->T * a->K);
    default:
      return fail(MOE_EINVAL, "checked mode: block_expert[%d] is outside [-1, E_total = %d)", host[1], a->E_total);
  }
}

// Routing that stage 1 performs itself (moe_layer_forward on a small batch).
struct FusedRoute {
  const float* logits;
  int E, topk, score, renorm, n_shared;
  float shared_w;
  int32_t *counts, *offsets;
};

moe_status experts_forward(const moe_forward_args* a, const FusedRoute* r, hipStream_t stream) {
  moe_workspace_layout_t L;
  moe_status st = moe_workspace_layout(a, &L);
  if (st != MOE_OK) return st;
  if (a->T == 0) return ok();
  // tiled MXFP4 weights carry their scales inside the blocks
  const bool scales_needed =
      !(a->wfmt == MOE_W_MXFP4 && a->weight_layout == MOE_LAYOUT_TILED) && a->wfmt != MOE_W_BF16;
  if (!a->hidden_states || !a->w1 || !a->w2 || (scales_needed && (!a->w1_scale || !a->w2_scale)) || !a->topk_ids ||
      !a->topk_weights || !a->sorted_slots || !a->block_expert || !a->num_padded || !a->out)
    return fail(MOE_EINVAL, "moe_experts_forward: NULL pointer");
  if (!aligned(a->hidden_states, 16) || !aligned(a->w1, 16) || !aligned(a->w2, 16) || !aligned(a->out, 16) ||
      !aligned(a->topk_weights, 4) || !aligned(a->w1_scale, a->wfmt == MOE_W_MXFP4 ? 1 : 4) ||
      !aligned(a->w2_scale, a->wfmt == MOE_W_MXFP4 ? 1 : 4) || (a->a1_codes && !aligned(a->a1_codes, 16)) ||
      (a->a1_scales && !aligned(a->a1_scales, 4)) || !aligned(a->w1_bias, 4) || !aligned(a->w2_bias, 4))
    return fail(MOE_EINVAL, "moe_experts_forward: misaligned pointer (16 B for tensors, 4 B for fp32 arrays, "
                            "4 B for biases)");
  if (a->afmt != MOE_A_BF16 && (a->a1_codes == nullptr) != (a->a1_scales == nullptr))
    return fail(MOE_EINVAL, "moe_experts_forward: a1_codes and a1_scales go together");
  if (!a->workspace || a->workspace_bytes < L.total)
    return fail(MOE_EWORKSPACE, "moe_experts_forward: workspace of %zu bytes needed, %zu given", L.total,
                a->workspace ? a->workspace_bytes : (size_t)0);
  if (!aligned(a->workspace, 256)) return fail(MOE_EINVAL, "moe_experts_forward: workspace must be 256-byte aligned");

  uint8_t* ws = (uint8_t*)a->workspace;
  const size_t cap = moe_sort_capacity(a->T, a->K, a->E_total, a->block_m);
  // checked mode: caller-built tables are verified before anything reads them (the fused
  // route builds its own in stage 1)
  if (!r && g_checked.load(std::memory_order_relaxed) && (st = check_tables(a, cap, stream)) != MOE_OK) return st;
  const int afmt = (int)a->afmt;
  uint16_t* h = (uint16_t*)(ws + L.h_off);
  const void* a1 = a->hidden_states;
  const void* a1s = nullptr;
  hipError_t e = hipSuccess;
  if (afmt != MOE_A_BF16) {
    if (a->a1_codes) {
      a1 = a->a1_codes;
      a1s = a->a1_scales;
    } else {
      a1 = ws + L.a1_codes_off;
      a1s = ws + L.a1_scales_off;
      e = moe::launch_quant_act(a->hidden_states, a->T, a->H, afmt, nullptr, ws + L.a1_codes_off,
                                ws + L.a1_scales_off, stream);
      if (e != hipSuccess) return hip_status(e, "moe_experts_forward: a1 quantisation");
    }
  }
  moe::GemmParams p{};
  p.T = a->T;
  p.slots_per_token = a->K;
  p.sorted_slots = a->sorted_slots;
  p.block_expert = a->block_expert;
  p.num_padded = a->num_padded;
  p.num_blocks = (int)(cap / a->block_m);
  p.topk_weights = a->topk_weights;
  p.weight_layout = (int)a->weight_layout;
  p.act = a->act == MOE_ACT_SWIGLU_OAI ? moe::kActSwigluOai : moe::kActSilu;
  p.act_alpha = a->act_alpha;
  p.act_beta = a->act_beta;
  p.act_limit = a->act_limit;

  // stage 1: gate/up GEMM + SiLU-and-mul -> h (bf16, sorted rows)
  p.a = a1;
  p.a_scale = a1s;
  p.a_gather = 1;
  p.w = a->w1;
  p.w_scale = a->w1_scale;
  p.N = a->I;
  p.K = a->H;
  p.Nw = 2 * a->I;
  p.h = h;
  p.interleaved = a->gate_up_interleaved;
  p.bias = a->w1_bias;
  p.weight_on_input = a->apply_router_weight_on_input;
  p.wsc_es = a->wfmt == MOE_W_FP8_TENSOR ? 1 : p.Nw;  // FP8 weight scales: per tensor or per channel
  p.wsc_rs = a->wfmt == MOE_W_FP8_TENSOR ? 0 : 1;
  p.asc_rs = a->afmt == MOE_A_FP8_TENSOR ? 0 : 1;
  if (r) {  // stage 1 routes and sorts; its workgroup 0 writes the tables read below
    p.route = 1;
    p.logits = r->logits;
    p.route_E = r->E;
    p.route_topk = r->topk;
    p.route_score = r->score;
    p.route_renorm = r->renorm;
    p.route_n_shared = r->n_shared;
    p.route_shared_w = r->shared_w;
    p.route_cap = (int)cap;
    p.out_ids = const_cast<int32_t*>(a->topk_ids);
    p.out_weights = const_cast<float*>(a->topk_weights);
    p.out_counts = r->counts;
    p.out_offsets = r->offsets;
    p.out_sorted = const_cast<int32_t*>(a->sorted_slots);
    p.out_block_expert = const_cast<int32_t*>(a->block_expert);
    p.out_num_padded = const_cast<int32_t*>(a->num_padded);
  }
  if ((e = prof_mark(0, stream)) != hipSuccess) return hip_status(e, "moe_experts_forward: profiling event");
  e = moe::launch_gemm(1, (int)a->wfmt, afmt, a->block_m, p, stream);
  if (e != hipSuccess) return hip_status(e, "moe_experts_forward: stage 1");
  if ((e = prof_mark(1, stream)) != hipSuccess) return hip_status(e, "moe_experts_forward: profiling event");
  p.route = 0;

  // a2: re-quantise h in the activation format
  const void* a2 = h;
  const void* a2s = nullptr;
  if (afmt != MOE_A_BF16) {
    e = moe::launch_quant_act(h, (int)cap, a->I, afmt, a->num_padded, ws + L.a2_codes_off, ws + L.a2_scales_off,
                              stream);
    if (e != hipSuccess) return hip_status(e, "moe_experts_forward: a2 quantisation");
    a2 = ws + L.a2_codes_off;
    a2s = ws + L.a2_scales_off;
  }

  // stage 2: down GEMM, weighted by topk_weights -> per-slot fp32 rows
  float* ybuf = (float*)(ws + L.ybuf_off);
  p.a = a2;
  p.a_scale = a2s;
  p.a_gather = 0;
  p.w = a->w2;
  p.w_scale = a->w2_scale;
  p.N = a->H;
  p.K = a->I;
  p.Nw = a->H;
  p.h = nullptr;
  p.ybuf = ybuf;
  p.interleaved = 0;
  p.bias = a->w2_bias;
  p.weight_on_input = 0;
  p.wsc_es = a->wfmt == MOE_W_FP8_TENSOR ? 1 : p.Nw;
  e = moe::launch_gemm(2, (int)a->wfmt, afmt, a->block_m, p, stream);
  if (e != hipSuccess) return hip_status(e, "moe_experts_forward: stage 2");
  if ((e = prof_mark(2, stream)) != hipSuccess) return hip_status(e, "moe_experts_forward: profiling event");

  // ordered top-k combine
  e = moe::launch_combine(ybuf, a->topk_ids, a->apply_router_weight_on_input ? nullptr : a->topk_weights, a->T, a->K,
                          a->H, a->E_total, a->out, stream);
  if (e != hipSuccess) return hip_status(e, "moe_experts_forward: combine");
  return hip_status(prof_mark(3, stream), "moe_experts_forward: profiling event");
}

// Device address of `scratch` on the current device: looked up once per device (with that
// device current) and kept; NULL with the HIP error in *err when the lookup fails.
void* scratch_ptr(hipError_t* err) {
  static std::atomic<void*> ptrs[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    ptrs[dev].store(p, std::memory_order_release);  // two threads racing store the same address
  }
  *err = hipSuccess;
  return p;
}

}  // namespace

extern "C" {

moe_status moe_set_checked_mode(int on) {
  g_checked.store(on ? 1 : 0, std::memory_order_relaxed);
  return ok();
}

moe_status moe_experts_forward(const moe_forward_args* a, hipStream_t stream) {
  return experts_forward(a, nullptr, stream);
}

moe_status moe_experts_forward_noalloc(const moe_forward_args* a, hipStream_t stream) {
  moe_status st = check_shapes(a);
  if (st != MOE_OK) return st;
  moe_forward_args c = *a;
  c.workspace = nullptr;
  c.workspace_bytes = 0;
  moe_workspace_layout_t L;
  if ((st = moe_workspace_layout(&c, &L)) != MOE_OK) return st;
  if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_EWORKSPACE, "moe_experts_forward_noalloc: this call needs a workspace of %zu bytes, more than "
                                "the library's scratch of %zu bytes (use moe_experts_forward with a caller workspace)",
                L.total, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  if (a->T == 0) return ok();
  hipError_t e = hipSuccess;
  void* ws = scratch_ptr(&e);
  if (!ws) return hip_status(e, "moe_experts_forward_noalloc: scratch address");
  c.workspace = ws;
  c.workspace_bytes = MOE_NOALLOC_SCRATCH_BYTES;
  return experts_forward(&c, nullptr, stream);
}

moe_status moe_layer_forward(const moe_forward_args* a, const float* router_logits, moe_score score, int renormalize,
                             int n_shared, float shared_weight, int32_t* expert_counts, int32_t* expert_offsets,
                             hipStream_t stream) {
  moe_status st = check_shapes(a);
  if (st != MOE_OK) return st;
  if (n_shared < 0 || n_shared >= a->K || n_shared >= a->E_total)
    return fail(MOE_EINVAL, "moe_layer_forward: n_shared must be in [0, min(K, E_total)) (got %d)", n_shared);
  const int E = a->E_total - n_shared, topk = a->K - n_shared;
  st = check_route_align("moe_layer_forward", router_logits, a->T, E, topk, score, n_shared, a->block_m, a->topk_ids,
                         a->topk_weights, expert_counts, expert_offsets, a->sorted_slots, a->block_expert,
                         a->num_padded);
  if (st != MOE_OK) return st;
  // stage 1 on the persistent 16-row kernel routes and sorts the batch itself; the
  // router weight on the input is read by stage 1 and so needs the weights first
  if (a->block_m == 16 && !a->apply_router_weight_on_input &&
      moe::route_stage1_fusable((int)a->afmt, a->H, a->I, a->T, E, topk, n_shared, a->w1_bias != nullptr)) {
    const FusedRoute r{router_logits, E, topk, (int)score, renormalize ? 1 : 0, n_shared, shared_weight,
                       expert_counts, expert_offsets};
    return experts_forward(a, &r, stream);
  }
  st = moe_route_align(router_logits, a->T, E, topk, score, renormalize, n_shared, shared_weight, a->block_m,
                       const_cast<int32_t*>(a->topk_ids), const_cast<float*>(a->topk_weights), expert_counts,
                       expert_offsets, const_cast<int32_t*>(a->sorted_slots), const_cast<int32_t*>(a->block_expert),
                       const_cast<int32_t*>(a->num_padded), stream);
  if (st != MOE_OK) return st;
  return experts_forward(a, nullptr, stream);
}

}  // extern "C"
