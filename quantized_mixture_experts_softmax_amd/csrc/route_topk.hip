// Wavefront-level softmax / sigmoid top-k router.
//
// One wave64 per token: each lane holds E/64 logits in registers, the k winners are
// found by k rounds of a wave-wide (value desc, id asc) argmax, and lane j keeps the
// j-th winner, so the weights are computed lane-parallel.  The routing rule follows
// the reading documented for moe_route_topk (pages: "rocm_aiter_moe",
// inject_shared_expert_weights and rocm_aiter_fused_experts; "mxfp4.py",
// Mxfp4MoEMethod.apply_monolithic).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// (v1, i1) ranks before (v2, i2): larger value first, equal values by lower id.
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

template <int VPL>  // logits per lane; E <= 64 * VPL
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int topk, int score, int renorm, int n_shared,
                                                         float shared_w, int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int lane = lane_id();
  const int t = blockIdx.x * (blockDim.x / kWave) + (int)(threadIdx.x / kWave);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
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
  const int KP = topk + n_shared;
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
  if (lane < topk) {
    ids[(size_t)t * KP + lane] = my_id;
    weights[(size_t)t * KP + lane] = (score == 0 || renorm) ? s / denom : s;
  } else if (lane < KP) {
    ids[(size_t)t * KP + lane] = E + (lane - topk);
    weights[(size_t)t * KP + lane] = shared_w;
  }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int topk, int score, int renorm,
                             int n_shared, float shared_w, int32_t* ids, float* weights, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 block(256), grid((unsigned)((T + 3) / 4));
#define MOE_ROUTE(VPL) \
  route_topk_kernel<VPL><<<grid, block, 0, stream>>>(logits, T, E, topk, score, renorm, n_shared, shared_w, ids, weights)
  if (E <= 64) MOE_ROUTE(1);
  else if (E <= 128) MOE_ROUTE(2);
  else if (E <= 256) MOE_ROUTE(4);
  else if (E <= 512) MOE_ROUTE(8);
  else MOE_ROUTE(16);
#undef MOE_ROUTE
  return hipGetLastError();
}

}  // namespace moe
