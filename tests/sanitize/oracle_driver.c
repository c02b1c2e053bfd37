/* Exercises every oracle entry point on small seeded inputs, for every weight / activation
 * format pair and the edge cases (empty batch, bad arguments), so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer checks the oracle's memory accesses and
 * arithmetic.  Prints "oracle-sanitize ok" and exits 0 when every call returned as expected. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/moe_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12; rng_state ^= rng_state << 25; rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float unif(void) { return (float)(rnd() >> 8) / 16777216.0f * 2.0f - 1.0f; }

#define CHECK(cond) do { if (!(cond)) { fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); exit(1); } } while (0)

static void layer_case(int wfmt, int afmt, int act, int interleaved, int bias, int on_input) {
  const int T = 7, H = 96, I = 64, E = 3, k = on_input ? 1 : 2, K = k;
  const int N1 = 2 * I;
  size_t w1b, w2b, s1b = 0, s2b = 0;
  if (wfmt == ORC_W_MXFP4) { w1b = (size_t)E * N1 * H / 2; w2b = (size_t)E * H * I / 2; s1b = (size_t)E * N1 * H / 32; s2b = (size_t)E * H * I / 32; }
  else if (wfmt == ORC_W_BF16) { w1b = (size_t)E * N1 * H * 2; w2b = (size_t)E * H * I * 2; }
  else {
    w1b = (size_t)E * N1 * H; w2b = (size_t)E * H * I;
    if (wfmt == ORC_W_FP8_BLOCK128) { s1b = (size_t)E * ((N1 + 127) / 128) * ((H + 127) / 128) * 4; s2b = (size_t)E * ((H + 127) / 128) * ((I + 127) / 128) * 4; }
    else if (wfmt == ORC_W_FP8_CHANNEL) { s1b = (size_t)E * N1 * 4; s2b = (size_t)E * H * 4; }
    else { s1b = (size_t)E * 4; s2b = (size_t)E * 4; }
  }
  uint8_t* w1 = malloc(w1b); uint8_t* w2 = malloc(w2b);
  uint8_t* s1 = s1b ? malloc(s1b) : NULL; uint8_t* s2 = s2b ? malloc(s2b) : NULL;
  for (size_t i = 0; i < w1b; ++i) w1[i] = (uint8_t)rnd();
  for (size_t i = 0; i < w2b; ++i) w2[i] = (uint8_t)rnd();
  if (wfmt != ORC_W_MXFP4) {  /* keep FP8 / bf16 codes finite: clear the top exponent bit */
    for (size_t i = 0; i < w1b; ++i) w1[i] &= (wfmt == ORC_W_BF16 && (i & 1) == 0) ? 0xFF : 0xBF;
    for (size_t i = 0; i < w2b; ++i) w2[i] &= (wfmt == ORC_W_BF16 && (i & 1) == 0) ? 0xFF : 0xBF;
  }
  if (wfmt == ORC_W_MXFP4) {
    for (size_t i = 0; i < s1b; ++i) s1[i] = (uint8_t)(118 + rnd() % 9);
    for (size_t i = 0; i < s2b; ++i) s2[i] = (uint8_t)(118 + rnd() % 9);
  } else if (s1) {
    for (size_t i = 0; i < s1b / 4; ++i) ((float*)s1)[i] = 0.01f + 0.001f * (float)(rnd() % 7);
    for (size_t i = 0; i < s2b / 4; ++i) ((float*)s2)[i] = 0.01f + 0.001f * (float)(rnd() % 7);
  }
  uint16_t* b1 = NULL; uint16_t* b2 = NULL;
  if (bias) {
    b1 = malloc(sizeof(uint16_t) * E * N1); b2 = malloc(sizeof(uint16_t) * E * H);
    for (int i = 0; i < E * N1; ++i) b1[i] = orc_f32_to_bf16(0.1f * unif());
    for (int i = 0; i < E * H; ++i) b2[i] = orc_f32_to_bf16(0.1f * unif());
  }
  uint16_t* x = malloc(sizeof(uint16_t) * T * H);
  for (int i = 0; i < T * H; ++i) x[i] = orc_f32_to_bf16(unif());
  float* logits = malloc(sizeof(float) * T * E);
  for (int i = 0; i < T * E; ++i) logits[i] = unif();
  int32_t* ids = malloc(sizeof(int32_t) * T * K); float* wts = malloc(sizeof(float) * T * K);
  CHECK(orc_route_topk(logits, T, E, k, on_input ? ORC_SCORE_SIGMOID : ORC_SCORE_SOFTMAX, !on_input, 0, 1.0f, ids, wts) == 0);
  orc_layer L;
  memset(&L, 0, sizeof L);
  L.H = H; L.I = I; L.E_total = E; L.K = K; L.wfmt = wfmt; L.afmt = afmt;
  L.w1 = w1; L.w1_scale = s1; L.w2 = w2; L.w2_scale = s2;
  L.act = act; L.alpha = 1.702; L.beta = 1.0; L.limit = 7.0; L.gate_up_interleaved = interleaved;
  L.w1_bias = b1; L.w2_bias = b2; L.weight_on_input = on_input;
  int32_t tokens[7] = {0, 1, 2, 3, 4, 5, 6};
  double* out = malloc(sizeof(double) * T * H);
  uint16_t* h = malloc(sizeof(uint16_t) * T * K * I);
  CHECK(orc_forward(&L, x, ids, wts, tokens, T, out) == 0);
  for (int i = 0; i < T * H; ++i) CHECK(isfinite(out[i]));
  CHECK(orc_stage1(&L, x, ids, wts, tokens + 2, 3, h) == 0);
  CHECK(orc_stage2(&L, h, ids, wts, tokens + 2, 3, out) == 0);
  CHECK(orc_forward(&L, x, ids, wts, tokens, 0, out) == 0); /* empty */
  ids[0] = -1;                                                /* a dropped slot */
  CHECK(orc_forward(&L, x, ids, wts, tokens, T, out) == 0);
  free(w1); free(w2); free(s1); free(s2); free(b1); free(b2); free(x); free(logits); free(ids); free(wts);
  free(out); free(h);
}

int main(void) {
  /* codecs over every code */
  for (unsigned c = 0; c < 256; ++c) { (void)orc_e4m3_value(c); (void)orc_e8m0_value(c); (void)orc_e2m1_value(c & 15); }
  for (int i = 0; i < 4096; ++i) {
    const float v = unif() * 600.0f;
    (void)orc_e4m3_encode(v); (void)orc_e2m1_encode(v / 64.0f); (void)orc_mx_shared_exp(fabsf(v));
    (void)orc_f32_to_bf16(v); (void)orc_f64_to_bf16((double)v);
  }
  /* routers, map, sort */
  const int T = 33, E = 20, k = 3, KP = 4;
  float lg[33 * 20], bias[20];
  for (int i = 0; i < T * E; ++i) lg[i] = unif();
  for (int i = 0; i < E; ++i) bias[i] = 0.05f * unif();
  int32_t ids[33 * 4], loc[33 * 4], map[21];
  float wts[33 * 4];
  CHECK(orc_route_topk(lg, T, E, k, ORC_SCORE_SOFTMAX, 1, 1, 1.0f, ids, wts) == 0);
  CHECK(orc_route_grouped_topk(lg, bias, T, E, k, 4, 2, ORC_SCORE_SIGMOID, 1, 2.5f, 1, 1.0f, ids, wts) == 0);
  CHECK(orc_route_topk(lg, T, E, 0, ORC_SCORE_SOFTMAX, 1, 0, 1.0f, ids, wts) == -1); /* bad topk */
  for (int i = 0; i < 21; ++i) map[i] = i % 2 ? i / 2 : -1;
  CHECK(orc_map_experts(ids, map, 20, T, KP, 21, loc) == 0);
  for (int bm = 16; bm <= 128; bm *= 2) {
    const int64_t cap = orc_sort_capacity(T, KP, 21, bm);
    int32_t* sorted = malloc(sizeof(int32_t) * cap);
    int32_t* owner = malloc(sizeof(int32_t) * (cap / bm + 1));
    int32_t cnt[21], offs[22], npad;
    CHECK(orc_align_sort(ids, T, KP, 21, bm, cnt, offs, sorted, owner, &npad) == 0);
    CHECK(orc_align_sort(loc, T, KP, 21, bm, cnt, offs, sorted, owner, &npad) == 0);
    free(sorted); free(owner);
  }
  /* quantisers, ragged groups included */
  const int rows = 5, cols = 160;
  uint16_t xq[5 * 160];
  uint8_t codes[5 * 160];
  float scl[5 * 2];
  uint8_t e8[5 * 5];
  for (int i = 0; i < rows * cols; ++i) xq[i] = orc_f32_to_bf16(unif() * 10.0f);
  CHECK(orc_quant_act(xq, rows, cols, ORC_A_FP8_G128, codes, scl) == 0);
  CHECK(orc_quant_act(xq, rows, cols, ORC_A_FP8_TOKEN, codes, scl) == 0);
  CHECK(orc_quant_act(xq, rows, cols, ORC_A_FP8_TENSOR, codes, scl) == 0);
  CHECK(orc_quant_act(xq, rows, cols, ORC_A_MXFP4_G32, codes, e8) == 0);
  /* the layer, every format pair and the activation options */
  const int pairs[6][2] = {{ORC_W_MXFP4, ORC_A_BF16}, {ORC_W_MXFP4, ORC_A_MXFP4_G32}, {ORC_W_FP8_BLOCK128, ORC_A_FP8_G128},
                           {ORC_W_FP8_CHANNEL, ORC_A_FP8_TOKEN}, {ORC_W_FP8_TENSOR, ORC_A_FP8_TENSOR}, {ORC_W_BF16, ORC_A_BF16}};
  for (int p = 0; p < 6; ++p) {
    layer_case(pairs[p][0], pairs[p][1], ORC_ACT_SILU, 0, 0, 0);
    layer_case(pairs[p][0], pairs[p][1], ORC_ACT_SWIGLU_OAI, pairs[p][0] != ORC_W_FP8_BLOCK128, 1, 0);
    layer_case(pairs[p][0], pairs[p][1], ORC_ACT_SILU, 0, 0, 1);
  }
  printf("oracle-sanitize ok\n");
  return 0;
}
