// Router bodies shared by the router kernels and the fused router + sort kernel.
// E <= 64 (route_tile_small): one thread per (token, expert) counts the experts that
// rank before it (value desc, id asc) in the token's logits staged in LDS, and the
// expert of rank j < k fills slot j; then one thread per slot computes the weight.
// No step depends on another lane, so a tile of tokens is routed in the latency of
// one E-long loop.  Larger E (route_token): one wave64 per token, each lane holding
// E/64 logits; the k winners are found by k rounds of a wave-wide argmax and lane j
// keeps the j-th winner.  The routing rule follows
// the reading documented for moe_route_topk (pages: "rocm_aiter_moe",
// inject_shared_expert_weights and rocm_aiter_fused_experts; "mxfp4.py",
// Mxfp4MoEMethod.apply_monolithic).
#pragma once
#include "moe_device.h"

namespace moe {

// (v1, i1) ranks before (v2, i2): larger value first, equal values by lower id.
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

constexpr int kSmallE = 64;  // route_tile_small serves E <= kSmallE

// Weight of routed slot j of a token: sv = the token's k winning logits in rank order,
// row(i) = logit i of the token (the full softmax sum runs over them in id order).
template <class Row>
__device__ __forceinline__ float slot_weight(const float* sv, int j, int topk, int score, int renorm, Row row,
                                             int E) {
  const float top_v = sv[0];
  auto f = [&](float x) { return score == 0 ? expf(x - top_v) : 1.0f / (1.0f + expf(-x)); };
  const float s = f(sv[j]);
  float denom = 1.0f;
  if (renorm) {
    denom = 0.0f;
#pragma unroll 8
    for (int i = 0; i < topk; ++i) denom += f(sv[i]);
  } else if (score == 0) {
    denom = 0.0f;
#pragma unroll 8
    for (int i = 0; i < E; ++i) denom += expf(row(i) - top_v);
  }
  return (score == 0 || renorm) ? s / denom : s;
}

// Routes tokens [t0, t0 + nt) with the nthreads threads of the workgroup (all must
// call).  lg: the tokens' logits staged in LDS, [nt][E]; sel_v: LDS scratch of nt*topk
// floats.  ids_copy (optional, LDS) receives the same ids as ids, at the same index
// relative to t0.  Weights follow the same rule as route_token; a renormalised sum runs
// over the k winners in rank order, the full softmax sum over the experts in id order.
__device__ __forceinline__ void route_tile_small(const float* lg, int t0, int nt, int E, int topk, int score,
                                                 int renorm, int n_shared, float shared_w, float* sel_v,
                                                 int32_t* __restrict__ ids, float* __restrict__ weights,
                                                 int32_t* ids_copy, int32_t* sel_id, int nthreads) {
  const int tid = (int)threadIdx.x;
  const int KP = topk + n_shared;
  for (int q = tid; q < nt * E; q += nthreads) {
    const int t = q / E, e = q - t * E;
    const float* row = lg + t * E;
    const float v = row[e];
    int rank = 0;
#pragma unroll 16
    for (int j = 0; j < E; ++j) rank += better(row[j], j, v, e) ? 1 : 0;
    if (rank < topk) {
      sel_id[t * KP + rank] = e;
      sel_v[t * topk + rank] = v;
    }
  }
  __syncthreads();
  for (int q = tid; q < nt * KP; q += nthreads) {
    const int t = q / KP, j = q - t * KP;
    int id;
    float wt;
    if (j < topk) {
      id = sel_id[t * KP + j];
      const float* lrow = lg + t * E;
      wt = slot_weight(sel_v + t * topk, j, topk, score, renorm, [&](int i) { return lrow[i]; }, E);
    } else {
      id = E + (j - topk);
      wt = shared_w;
    }
    ids[(size_t)(t0 + t) * KP + j] = id;
    weights[(size_t)(t0 + t) * KP + j] = wt;
    if (ids_copy) ids_copy[t * KP + j] = id;
  }
}

// Routes token t with the calling wave (all 64 lanes).  ids_copy (optional) receives
// the same ids as ids, at the same index.
template <int VPL>  // logits per lane; E <= 64 * VPL
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int topk, int score,
                                            int renorm, int n_shared, float shared_w, int32_t* __restrict__ ids,
                                            float* __restrict__ weights, int32_t* ids_copy) {
  const int lane = lane_id();
  const float* row = logits + (size_t)t * E;
  const int KP = topk + n_shared;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    v[i] = e < E ? row[e] : -INFINITY;
  }
  uint32_t taken = 0;
  float my_v = -INFINITY;  // lane j holds the j-th winner
  int my_id = 0x7FFFFFFF;
  float top_v = 0.0f;
  for (int j = 0; j < topk; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !((taken >> i) & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // every lane now holds the same winner
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == j) {
      my_v = bv;
      my_id = bi;
    }
    if (j == 0) top_v = bv;
  }
  float s = 0.0f;
  if (score == 0) {
    s = lane < topk ? expf(my_v - top_v) : 0.0f;
  } else {
    s = lane < topk ? 1.0f / (1.0f + expf(-my_v)) : 0.0f;
  }
  float denom = 1.0f;
  if (renorm) {
    denom = wave_sum(s);
  } else if (score == 0) {
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + kWave * i < E) part += expf(v[i] - top_v);
    denom = wave_sum(part);
  }
  if (lane < KP) {
    const int id = lane < topk ? my_id : E + (lane - topk);
    ids[(size_t)t * KP + lane] = id;
    weights[(size_t)t * KP + lane] = lane < topk ? ((score == 0 || renorm) ? s / denom : s) : shared_w;
    if (ids_copy) ids_copy[(size_t)t * KP + lane] = id;
  }
}

// Expands CALL(VPL) with the smallest logits-per-lane count that covers E (E > kSmallE).
#define MOE_ROUTE_DISPATCH(E, CALL) \
  do {                               \
    if ((E) <= 128) CALL(2);         \
    else if ((E) <= 256) CALL(4);    \
    else if ((E) <= 512) CALL(8);    \
    else CALL(16);                   \
  } while (0)

}  // namespace moe
