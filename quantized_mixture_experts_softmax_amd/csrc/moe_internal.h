// Internal (non-ABI) declarations shared by the libmoe translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Activation formats (values match moe_afmt in include/moe.h).
// kAFp8Tensor is quantised by its own kernels; the GEMMs read it as kAFp8Token with a
// row stride of 0 in the scale array.
enum { kABf16 = 0, kAMxfp4 = 1, kAFp8G128 = 2, kAFp8Token = 3, kAFp8Tensor = 4 };
// Weight formats (values match moe_wfmt).  kWFp8Tensor runs as kWFp8Channel with scale
// strides (expert 1, row 0).
enum { kWMxfp4 = 0, kWFp8Block = 1, kWFp8Channel = 2, kWFp8Tensor = 3, kWBf16 = 4 };

// One grouped-GEMM launch over the padded sorted rows.
struct GemmParams {
  // A operand: bf16 [rows, K] or quantised codes + scales (layouts of moe_afmt).
  const void* a;
  const void* a_scale;
  int a_gather;        // 1: A row = token of the sorted slot (stage 1); 0: A row = sorted row (stage 2)
  // Weights of all experts: [E, Nw, K] in the weight format; Nw = 2I (stage 1) or H (stage 2).
  const uint8_t* w;
  const void* w_scale;
  int N;               // output columns: I (stage 1, gate/up pairs) or H (stage 2)
  int K;               // reduction length: H (stage 1) or I (stage 2)
  int Nw;              // weight rows per expert
  int T, slots_per_token;
  const int32_t* sorted_slots;
  const int32_t* block_expert;
  const int32_t* num_padded;
  int num_blocks;      // grid rows: capacity / block_m
  // stage 1 output: h bf16 [cap, I]
  uint16_t* h;
  // stage 2 output: ybuf fp32 [T*K, H] by slot id (the combine applies topk_weights)
  float* ybuf;
  const float* topk_weights;
  int strips_per_wg;   // small-block kernel: consecutive column strips one workgroup streams
  int weight_layout;   // 0 canonical, 1 tiled (moe_tile_weights)
  // Stage 1: gated activation and the order of w13's rows; both stages: optional bf16
  // bias [E, Nw] indexed by weight row.
  int act;             // kActSilu or kActSwigluOai
  float act_alpha, act_beta, act_limit;
  int interleaved;     // stage 1: w13 rows alternate gate_n, up_n (else gate rows, then up rows)
  const uint16_t* bias;
  int weight_on_input;  // stage 1: the slot's top-k weight scales both projections (top-1)
  // FP8 channel-path scale strides: weight scale of (expert e, row n) at e * wsc_es + n *
  // wsc_rs (per channel: Nw, 1; per tensor: 1, 0); activation scale of row r at r * asc_rs
  // (per token 1, per tensor 0).
  int wsc_es, wsc_rs, asc_rs;
  // Stage 1 with the router + align-sort fused in (the persistent 16-row kernel): every
  // workgroup routes and sorts the batch in LDS; workgroup 0 writes the results.
  int route;                 // 0: sorted_slots / block_expert / num_padded are inputs
  const float* logits;       // [T, route_E] fp32
  int route_E, route_topk, route_score, route_renorm, route_n_shared;
  float route_shared_w;
  int route_cap;             // T * (topk + n_shared) + (route_E + n_shared) * 15
  int route_keep_off;        // LDS offset of the kept tables (set by the launcher)
  int bias_lds_off;          // persistent kernel with biases: LDS offset of a phase's bias slice (launcher)
  int32_t* out_ids;
  float* out_weights;
  int32_t *out_counts, *out_offsets, *out_sorted, *out_block_expert, *out_num_padded;
};

__device__ __forceinline__ size_t wsc_index(const GemmParams& p, int e, int row) {
  return (size_t)e * p.wsc_es + (size_t)row * p.wsc_rs;
}

constexpr int kActSilu = 0, kActSwigluOai = 1;

// h = act(gate, up) of one output column (stage-1 epilogue).  SiLU: silu(g) * u.
// SwiGLU-OAI: gate clamped from above at the limit, up to [-limit, limit] (no clamp
// for limit <= 0), h = g * sigmoid(alpha * g) * (u + beta).
__device__ __forceinline__ float glu_act(const GemmParams& p, float g, float u) {
  if (p.act == kActSilu) return g / (1.0f + __expf(-g)) * u;
  if (p.act_limit > 0.0f) {
    g = fminf(g, p.act_limit);
    u = fminf(fmaxf(u, -p.act_limit), p.act_limit);
  }
  return g / (1.0f + __expf(-p.act_alpha * g)) * (u + p.act_beta);
}

// Stage-1 factor of a sorted row's projections: its slot's top-k weight when the router
// weight goes on the input, else 1 (pad rows: 0, their activations are zero anyway).
__device__ __forceinline__ float fc1_weight(const GemmParams& p, int slot) {
  if (!p.weight_on_input) return 1.0f;
  return slot < p.T * p.slots_per_token ? p.topk_weights[slot] : 0.0f;
}

// bf16 bias of weight row `row` of expert e (0 without a bias tensor).
__device__ __forceinline__ float bias_of(const GemmParams& p, int e, int row) {
  return p.bias ? __uint_as_float((uint32_t)p.bias[(size_t)e * p.Nw + row] << 16) : 0.0f;
}

hipError_t launch_route_topk(const float* logits, int T, int E, int topk, int score, int renorm, int n_shared,
                             float shared_w, int32_t* ids, float* weights, hipStream_t stream);
hipError_t launch_route_grouped_topk(const float* logits, const float* bias, int T, int E, int topk, int n_group,
                                     int topk_group, int score, int renorm, float scaling, int n_shared,
                                     float shared_w, int32_t* ids, float* weights, hipStream_t stream);
hipError_t launch_map_experts(const int32_t* ids, const int32_t* emap, const int32_t* n_valid, int T, int K,
                              int E_global, int32_t* out, hipStream_t stream);
hipError_t launch_align_sort(const int32_t* ids, int T, int K, int E, int bm, int32_t* counts, int32_t* offsets,
                             int32_t* sorted, int32_t* block_expert, int32_t* num_padded, hipStream_t stream);
// Router + align-sort in a single one-workgroup launch; only when route_sort_fusable(T, E, K)
// (E routed experts, K = topk + n_shared), else hipErrorInvalidValue.
bool route_sort_fusable(int T, int E, int K);
// Whether stage 1 can run with the router + sort fused in (16-row blocks, the persistent
// kernel, LDS for the tile, the bias slice, the route scratch and the kept tables); K_dim
// = H, N = I, T tokens, E routed experts, topk, n_shared, bias: w1 biases present.
// Whether 16-row blocks of this activation format run on the persistent kernel for one
// stage (K_dim: the GEMM's K; N: its output columns; bias: the stage has a bias slice).
bool persist_launch_fits(int afmt, int stage, int K_dim, int N, bool bias);
bool route_stage1_fusable(int afmt, int K_dim, int N, int T, int E, int topk, int n_shared, bool bias);
hipError_t launch_route_sort(const float* logits, int T, int E, int topk, int score, int renorm, int n_shared,
                             float shared_w, int bm, int32_t* ids, float* weights, int32_t* counts, int32_t* offsets,
                             int32_t* sorted, int32_t* block_expert, int32_t* num_padded, hipStream_t stream);
// rows_dev (optional): device row count; rows at or past it are skipped.
hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, int fmt, const int32_t* rows_dev,
                            uint8_t* codes, void* scales, hipStream_t stream);
hipError_t launch_tile_weights(int wfmt, int E, int N, int K, const uint8_t* w, const void* ws, uint8_t* out,
                               hipStream_t stream);
hipError_t launch_gemm(int stage, int wfmt, int afmt, int block_m, const GemmParams& p, hipStream_t stream);
// 128-row blocks on tiled weights with both operands staged in LDS (gemm_lds.hip); epi: the
// general epilogue (biases, SwiGLU-OAI, interleaved rows, router weight on the input).
hipError_t launch_gemm_lds(int stage, int wfmt, int afmt, int epi, const GemmParams& p, hipStream_t stream);
hipError_t launch_combine(const float* ybuf, const int32_t* topk_ids, const float* topk_weights, int T, int K,
                          int H, int E_total, uint16_t* out, hipStream_t stream);

}  // namespace moe
