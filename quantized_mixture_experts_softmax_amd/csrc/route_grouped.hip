// Grouped top-k router with a score-correction bias (pages: "mxfp4.py",
// Mxfp4MoEMethod.apply_monolithic, which hands num_expert_group, topk_group,
// e_score_correction_bias and routed_scaling_factor to the monolithic kernel;
// "rocm_aiter_moe", inject_shared_expert_weights, for the combined routed + shared
// output).  The routing rule is the one documented for moe_route_grouped_topk.
//
// One wave64 per token, four tokens per 256-thread workgroup.  Lane l holds experts
// l, l + 64, ...; keys (score + bias, or the logit without a bias) are compared in
// fp64.  The token's keys are staged in LDS so that lane g can scan group g for its
// best one or two keys; the kept groups are a 64-bit ballot of "fewer than topk_group
// groups rank before mine"; the k winners are found by k rounds of a wave argmax over
// the keys of the kept groups (equal keys: lower id), and lane j keeps winner j.
#include "moe_device.h"
#include "moe_internal.h"

#include <math.h>

namespace moe {

constexpr int kGroupedWaves = 4;

__device__ __forceinline__ bool better_key(double v1, int i1, double v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <int VPL>  // experts per lane; E <= 64 * VPL
__global__ __launch_bounds__(64 * kGroupedWaves) void route_grouped_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int topk, int n_group,
    int topk_group, int score, int renorm, float scaling, int n_shared, float shared_w, int32_t* __restrict__ ids,
    float* __restrict__ weights) {
  __shared__ double lkey[kGroupedWaves][64 * VPL];
  __shared__ double lgsc[kGroupedWaves][64];
  const int wv = (int)(threadIdx.x / kWave), lane = lane_id();
  const int t = (int)blockIdx.x * kGroupedWaves + wv;
  const bool live = t < T;  // every wave stays to the barriers
  const float* row = logits + (size_t)(live ? t : 0) * E;

  float lv[VPL];
  double s[VPL], key[VPL];
  float lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    lv[i] = (live && e < E) ? row[e] : -INFINITY;
    lmax = fmaxf(lmax, lv[i]);
  }
  if (score == 0) {  // softmax over the whole row, fp64
    const double m = (double)wave_max(lmax);
    double z = 0.0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) z += (lane + kWave * i < E) ? exp((double)lv[i] - m) : 0.0;
    z = wave_sum_f64(z);
#pragma unroll
    for (int i = 0; i < VPL; ++i) s[i] = (lane + kWave * i < E) ? exp((double)lv[i] - m) / z : 0.0;
  } else {
#pragma unroll
    for (int i = 0; i < VPL; ++i) s[i] = 1.0 / (1.0 + exp(-(double)lv[i]));
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    key[i] = e < E ? (bias ? s[i] + (double)bias[e] : (double)lv[i]) : -INFINITY;
    if (e < E) lkey[wv][e] = key[i];
  }
  __syncthreads();

  // group scores: lane g scans group g
  const int gs = E / n_group;
  if (lane < n_group) {
    const double* kg = &lkey[wv][lane * gs];
    int b1 = 0;
    for (int i = 1; i < gs; ++i)
      if (kg[i] > kg[b1]) b1 = i;
    double v = kg[b1];
    if (bias && gs > 1) {
      int b2 = b1 == 0 ? 1 : 0;
      for (int i = b2 + 1; i < gs; ++i)
        if (i != b1 && kg[i] > kg[b2]) b2 = i;
      v += kg[b2];
    }
    lgsc[wv][lane] = v;
  }
  __syncthreads();
  bool gkeep = false;
  if (lane < n_group) {
    const double mine = lgsc[wv][lane];
    int rank = 0;
    for (int h = 0; h < n_group; ++h) rank += better_key(lgsc[wv][h], h, mine, lane) ? 1 : 0;
    gkeep = rank < topk_group;
  }
  const uint64_t keep = __ballot(gkeep);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    if (e >= E || !((keep >> (e / gs)) & 1ull)) key[i] = -INFINITY;
  }

  // k rounds of wave argmax; the winner's unbiased score travels with it
  uint32_t taken = 0;
  int my_id = 0;
  double my_s = 0.0;
  for (int j = 0; j < topk; ++j) {
    double bk = -INFINITY, bs = 0.0;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !((taken >> i) & 1u) && better_key(key[i], e, bk, bi)) {
        bk = key[i];
        bi = e;
        bs = s[i];
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ok = __shfl_xor(bk, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      const double os = __shfl_xor(bs, o, kWave);
      if (better_key(ok, oi, bk, bi)) {
        bk = ok;
        bi = oi;
        bs = os;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == j) {
      my_id = bi;
      my_s = bs;
    }
  }
  const double w = lane < topk ? my_s : 0.0;
  const double denom = renorm ? wave_sum_f64(w) : 1.0;
  const int KP = topk + n_shared;
  if (live && lane < KP) {
    ids[(size_t)t * KP + lane] = lane < topk ? my_id : E + (lane - topk);
    weights[(size_t)t * KP + lane] = lane < topk ? (float)(w / denom * (double)scaling) : shared_w;
  }
}

hipError_t launch_route_grouped_topk(const float* logits, const float* bias, int T, int E, int topk, int n_group,
                                     int topk_group, int score, int renorm, float scaling, int n_shared,
                                     float shared_w, int32_t* ids, float* weights, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 block(64 * kGroupedWaves), grid((unsigned)((T + kGroupedWaves - 1) / kGroupedWaves));
#define MOE_ROUTE_G(VPL)                                                                                          \
  route_grouped_kernel<VPL><<<grid, block, 0, stream>>>(logits, bias, T, E, topk, n_group, topk_group, score, renorm, \
                                                        scaling, n_shared, shared_w, ids, weights)
  if (E <= 64) MOE_ROUTE_G(1);
  else if (E <= 128) MOE_ROUTE_G(2);
  else if (E <= 256) MOE_ROUTE_G(4);
  else if (E <= 512) MOE_ROUTE_G(8);
  else MOE_ROUTE_G(16);
#undef MOE_ROUTE_G
  return hipGetLastError();
}

}  // namespace moe
