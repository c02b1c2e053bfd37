/*
 * CPU oracle for the quantized fused MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the test-suite, the package smoke check and the
 * CPU-baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * Conventions (all pointers are host memory owned by the caller):
 *   bf16 values travel as uint16_t bit patterns (upper half of an IEEE fp32).
 *   MXFP4 weights: w[E][N][K/2] bytes, element k of a row is nibble (k & 1) of
 *   byte k/2 (low nibble = even k); scales s[E][N][K/32] are E8M0 bytes.
 *   FP8 weights: w[E][N][K] e4m3fn bytes; block scales [E][ceil(N/128)][ceil(K/128)]
 *   fp32, channel scales [E][N] fp32.
 *   bf16 weights (unquantised): w[E][N][K] bf16 bit patterns (2 bytes each), no scales.
 *   w1 holds the fused gate/up projection: rows [0, I) are gate, [I, 2I) are up.
 *
 * Return value of every int function: 0 on success, -1 on bad arguments.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* weight formats */
enum { ORC_W_MXFP4 = 0, ORC_W_FP8_BLOCK128 = 1, ORC_W_FP8_CHANNEL = 2, ORC_W_FP8_TENSOR = 3, ORC_W_BF16 = 4 };
/* activation (GEMM input) formats */
enum { ORC_A_BF16 = 0, ORC_A_MXFP4_G32 = 1, ORC_A_FP8_G128 = 2, ORC_A_FP8_TOKEN = 3, ORC_A_FP8_TENSOR = 4 };
/* router score functions */
enum { ORC_SCORE_SOFTMAX = 0, ORC_SCORE_SIGMOID = 1 };

/* ---- element codecs ---- */
double orc_e2m1_value(unsigned code);        /* low 4 bits used */
double orc_e8m0_value(unsigned byte);        /* 2^(byte-127); NaN for 255 */
double orc_e4m3_value(unsigned byte);        /* OCP e4m3fn; NaN for 0x7F/0xFF */
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f64_to_bf16(double v);          /* round to nearest even */
uint16_t orc_f32_to_bf16(float v);           /* round to nearest even */
unsigned orc_e4m3_encode(float v);           /* nearest, ties to even, saturating at 448 */
unsigned orc_e2m1_encode(float v);           /* nearest, ties to even, saturating at 6 */
int orc_mx_shared_exp(float amax);           /* floor(log2 amax) - 2 clamped to [-127,127]; amax==0 -> -127 */

/* ---- router ---- */
int orc_route_topk(const float* logits, int T, int E, int topk, int score, int renormalize,
                   int n_shared, float shared_weight, int32_t* topk_ids, float* topk_weights);
int orc_route_grouped_topk(const float* logits, const float* bias, int T, int E, int topk, int n_group,
                           int topk_group, int score, int renormalize, float scaling, int n_shared,
                           float shared_weight, int32_t* topk_ids, float* topk_weights);
int orc_map_experts(const int32_t* topk_ids, const int32_t* expert_map, int num_local_tokens, int T, int K,
                    int E_global, int32_t* local_ids);

/* ---- token -> expert sort, padded per expert to block_m rows ---- */
int64_t orc_sort_capacity(int T, int K, int E_total, int block_m);
int orc_align_sort(const int32_t* topk_ids, int T, int K, int E_total, int block_m,
                   int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
                   int32_t* block_expert, int32_t* num_padded);

/* ---- dynamic activation quantisation ---- */
int orc_quant_act(const uint16_t* x, int rows, int cols, int fmt, uint8_t* codes, void* scales);

/* ---- expert layer ---- */
/* Gated activations. */
enum { ORC_ACT_SILU = 0, ORC_ACT_SWIGLU_OAI = 1 };

typedef struct {
  int H, I, E_total, K;       /* hidden, intermediate, experts in the weight tensors, slots per token */
  int wfmt, afmt;
  const uint8_t* w1; const void* w1_scale;   /* [E_total][2I][..] */
  const uint8_t* w2; const void* w2_scale;   /* [E_total][H][..]  */
  int act;                    /* ORC_ACT_SILU or ORC_ACT_SWIGLU_OAI */
  double alpha, beta, limit;  /* SwiGLU-OAI parameters (limit <= 0: no clamping) */
  int gate_up_interleaved;    /* 0: w13 rows [gate_0..gate_{I-1}, up_0..up_{I-1}]; 1: gate_n, up_n alternate */
  const uint16_t* w1_bias;    /* bf16 [E_total][2I] in w13 row order, or NULL */
  const uint16_t* w2_bias;    /* bf16 [E_total][H], or NULL */
  int weight_on_input;        /* 1: the top-k weight scales the gate/up projections (stage 1)
                                 and the sum over slots is unweighted (top-1 routing) */
} orc_layer;

/* Stage 1 for the tokens listed in `tokens` (n_tok of them):
 *   h[(i*K + j)*I + n] = bf16( act(g, u) ) for slot j of token tokens[i], g and u the
 *   gate and up rows' dot products (times the slot's top-k weight when weight_on_input;
 *   topk_weights is read only then) plus their biases.
 * Activations are x (bf16) or, for quantised formats, x quantised and dequantised
 * per row with the layer's activation format. */
int orc_stage1(const orc_layer* L, const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
               const int32_t* tokens, int n_tok, uint16_t* h);

/* Stage 2: takes the per-slot intermediate h (bf16, layout as orc_stage1 writes
 * it), quantises each slot row with the layer's activation format where that is
 * not bf16, multiplies by w2 and sums over the token's slots in ascending slot
 * order, weighting slot j by topk_weights.  out[i*H + m] in fp64. */
int orc_stage2(const orc_layer* L, const uint16_t* h, const int32_t* topk_ids, const float* topk_weights,
               const int32_t* tokens, int n_tok, double* out);

/* Stage 1 followed by stage 2. */
int orc_forward(const orc_layer* L, const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                const int32_t* tokens, int n_tok, double* out);

/* Number of threads the parallel loops of orc_stage1/orc_stage2 use. */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
