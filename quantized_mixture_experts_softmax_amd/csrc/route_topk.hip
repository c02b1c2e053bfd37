// Softmax / sigmoid top-k router (route_device.h): a tile of tokens per workgroup for
// E <= 64, one wave64 per token above.
#include "moe_device.h"
#include "moe_internal.h"
#include "route_device.h"

#include <algorithm>

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int topk, int score, int renorm, int n_shared,
                                                         float shared_w, int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int t = blockIdx.x * (blockDim.x / kWave) + (int)(threadIdx.x / kWave);
  if (t >= T) return;
  route_token<VPL>(logits, t, E, topk, score, renorm, n_shared, shared_w, ids, weights, nullptr);
}

// E <= kSmallE: nt tokens per 256-thread workgroup, logits staged in dynamic LDS as
// [nt][E] floats, then nt*topk winner values and nt*KP winner ids.
__global__ __launch_bounds__(256) void route_small_kernel(const float* __restrict__ logits, int T, int E, int topk,
                                                          int score, int renorm, int n_shared, float shared_w, int nt,
                                                          int32_t* __restrict__ ids, float* __restrict__ weights) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  const int t0 = (int)blockIdx.x * nt;
  const int n = min(nt, T - t0);
  float* lg = smem_f;
  float* sel_v = lg + nt * E;
  int32_t* sel_id = (int32_t*)(sel_v + nt * topk);
  for (int i = (int)threadIdx.x; i < n * E; i += 256) lg[i] = logits[(size_t)t0 * E + i];
  __syncthreads();
  route_tile_small(lg, t0, n, E, topk, score, renorm, n_shared, shared_w, sel_v, ids, weights, nullptr, sel_id, 256);
}

hipError_t launch_route_topk(const float* logits, int T, int E, int topk, int score, int renorm,
                             int n_shared, float shared_w, int32_t* ids, float* weights, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (E <= kSmallE) {
    const int nt = std::max(1, std::min(256, 1024 / E));
    const size_t lds = (size_t)nt * (E + topk + topk + n_shared) * 4;
    route_small_kernel<<<(unsigned)((T + nt - 1) / nt), 256, lds, stream>>>(logits, T, E, topk, score, renorm, n_shared,
                                                                           shared_w, nt, ids, weights);
    return hipGetLastError();
  }
  const dim3 block(256), grid((unsigned)((T + 3) / 4));
#define MOE_ROUTE(VPL) \
  route_topk_kernel<VPL><<<grid, block, 0, stream>>>(logits, T, E, topk, score, renorm, n_shared, shared_w, ids, weights)
  MOE_ROUTE_DISPATCH(E, MOE_ROUTE);
#undef MOE_ROUTE
  return hipGetLastError();
}

}  // namespace moe
