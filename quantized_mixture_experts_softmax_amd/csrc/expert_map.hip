// Expert-parallel share: global top-k ids -> this device's local expert ids (pages:
// "rocm_aiter_moe", AiterExperts.apply hands expert_map to the fused kernel as its
// expert mask, with num_local_tokens = expert_tokens_meta.expert_num_tokens).  The
// rule is the one documented for moe_map_experts.  One thread per slot.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void map_experts_kernel(const int32_t* __restrict__ ids,
                                                          const int32_t* __restrict__ emap,
                                                          const int32_t* __restrict__ n_valid, int T, int K,
                                                          int E_global, int32_t* __restrict__ out) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)T * K) return;
  const int t = (int)(i / K);
  const int g = ids[i];
  const bool row_ok = n_valid == nullptr || t < n_valid[0];
  int loc = -1;
  if (row_ok && g >= 0 && g < E_global) loc = emap ? emap[g] : g;
  out[i] = loc;
}

hipError_t launch_map_experts(const int32_t* ids, const int32_t* emap, const int32_t* n_valid, int T, int K,
                              int E_global, int32_t* out, hipStream_t stream) {
  const long n = (long)T * K;
  if (n == 0) return hipSuccess;
  map_experts_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(ids, emap, n_valid, T, K, E_global, out);
  return hipGetLastError();
}

}  // namespace moe
