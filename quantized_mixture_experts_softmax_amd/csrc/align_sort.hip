// Token -> expert align-sort: an LDS histogram + prefix scan + stable scatter,
// padded per expert to the GEMM row tile.
//
// One kernel, no inter-workgroup synchronisation.  Workgroup c owns the slot chunk
// [c*CH, (c+1)*CH).  Every workgroup builds, in LDS, the histogram of all slots and
// the histogram of the slots before its chunk (one pass over topk_ids, which is
// small and L2-resident), scans the padded counts into expert offsets, then places
// its own slots: the rank of a slot inside its expert is (slots of that expert
// before the chunk) + (earlier waves of this pass) + (lower lanes of its wave with
// the same expert), the last found by a ballot-based match over the id bits.  The
// result is the stable counting sort the oracle defines.  Each workgroup also fills
// a disjoint stride of the pad sentinels and of block_expert.
#include "moe_device.h"
#include "moe_internal.h"
#include "route_device.h"
#include "sort_device.h"

namespace moe {

constexpr int kMaxExperts = 1024;

// Lanes of this wave whose key equals mine (key < 2048).
__device__ __forceinline__ uint64_t match_key(int key) {
  uint64_t m = ~0ull;
#pragma unroll
  for (int b = 0; b < 11; ++b) {
    const uint64_t bal = __ballot((key >> b) & 1);
    m &= ((key >> b) & 1) ? bal : ~bal;
  }
  return m;
}

// The sort as run by workgroup `chunk` of `nchunks` (kSortThreads threads).  `ids` may
// point to global memory or to LDS.
__device__ __forceinline__ void align_sort_body(const int32_t* ids, int n, int E, int bm, int cap, int chunk,
                                                int nchunks, int32_t* __restrict__ counts_out,
                                                int32_t* __restrict__ offsets_out, int32_t* __restrict__ sorted,
                                                int32_t* __restrict__ block_expert, int32_t* __restrict__ num_padded) {
  __shared__ int total_cnt[kMaxExperts];
  __shared__ int before_cnt[kMaxExperts];  // becomes the running cursor
  __shared__ int offs[kMaxExperts + 1];
  __shared__ int wcnt[kSortWaves][kMaxExperts];
  __shared__ int wsum[kSortWaves];
  __shared__ int grand_total;

  const int tid = (int)threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int c0 = chunk * kSortChunk;
  for (int e = tid; e < E; e += kSortThreads) {
    total_cnt[e] = 0;
    before_cnt[e] = 0;
  }
  __syncthreads();
  // histograms of all slots and of the slots before this chunk
  for (int s = tid; s < n; s += kSortThreads) {
    const int e = ids[s];
    if (e >= 0 && e < E) {
      atomicAdd(&total_cnt[e], 1);
      if (s < c0) atomicAdd(&before_cnt[e], 1);
    }
  }
  __syncthreads();
  // exclusive scan of the padded counts (E <= kSortThreads)
  const int padded = tid < E ? (total_cnt[tid] + bm - 1) / bm * bm : 0;
  const int off = block_exclusive_scan(padded, wsum, &grand_total);
  if (tid < E) offs[tid] = off;
  if (tid == 0) offs[E] = grand_total;
  __syncthreads();
  const int total = grand_total;
  if (chunk == 0) {
    for (int e = tid; e < E; e += kSortThreads) {
      counts_out[e] = total_cnt[e];
      offsets_out[e] = offs[e];
    }
    if (tid == 0) {
      offsets_out[E] = total;
      num_padded[0] = total;
    }
  }
  // stable placement of this chunk's slots
  const int c1 = min(n, c0 + kSortChunk);
  for (int base = c0; base < c1; base += kSortThreads) {
    for (int i = tid; i < kSortWaves * E; i += kSortThreads) (&wcnt[0][0])[(i / E) * kMaxExperts + (i % E)] = 0;
    __syncthreads();
    const int s = base + tid;
    int e = s < c1 ? ids[s] : -1;
    if (e < 0 || e >= E) e = -1;
    const int key = e < 0 ? kMaxExperts : e;
    const uint64_t peers = match_key(key);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int rank = __popcll(peers & below);
    if (e >= 0 && rank == 0) wcnt[w][e] = __popcll(peers);
    __syncthreads();
    for (int x = tid; x < E; x += kSortThreads) {
      int run = before_cnt[x];
      for (int ww = 0; ww < kSortWaves; ++ww) {
        const int c = wcnt[ww][x];
        wcnt[ww][x] = run;
        run += c;
      }
      before_cnt[x] = run;
    }
    __syncthreads();
    if (e >= 0) sorted[offs[e] + wcnt[w][e] + rank] = s;
    __syncthreads();
  }
  // pad sentinels and block owners, a disjoint stride per workgroup
  fill_pads_owners(offs, total_cnt, E, total, n, bm, cap, chunk * kSortThreads + tid, nchunks * kSortThreads, sorted,
                   block_expert);
}

__global__ __launch_bounds__(kSortThreads) void align_sort_kernel(
    const int32_t* __restrict__ ids, int n, int E, int bm, int cap, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ sorted, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded) {
  align_sort_body(ids, n, E, bm, cap, (int)blockIdx.x, (int)gridDim.x, counts_out, offsets_out, sorted, block_expert,
                  num_padded);
}

// Router + sort in one workgroup (route_sort_fusable: E <= 64, small batch): the body is
// route_sort_block (sort_device.h).  The logits are staged in LDS with row stride E + 1,
// so the lanes of a wave, which hold different tokens, hit different banks.
__global__ __launch_bounds__(kSortThreads) void route_sort_kernel(
    const float* __restrict__ logits, int T, int E, int topk, int score, int renorm, int n_shared, float shared_w,
    int bm, int cap, int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ sorted, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded) {
  __shared__ __attribute__((aligned(16))) uint8_t scratch[kRouteSortLdsMax];
  RouteSortOut o{ids, weights, counts_out, offsets_out, sorted, block_expert, num_padded};
  route_sort_block(logits, T, E, topk, score, renorm, n_shared, shared_w, bm, cap, scratch, o);
}

bool route_sort_fusable(int T, int E, int K) {
  return E <= kSmallE && (long)T * K <= kSortChunk && (long)T * E <= kFuseLogits;
}

hipError_t launch_route_sort(const float* logits, int T, int E, int topk, int score, int renorm, int n_shared,
                             float shared_w, int bm, int32_t* ids, float* weights, int32_t* counts, int32_t* offsets,
                             int32_t* sorted, int32_t* block_expert, int32_t* num_padded, hipStream_t stream) {
  const int K = topk + n_shared, E_total = E + n_shared;
  if (!route_sort_fusable(T, E, K)) return hipErrorInvalidValue;
  const int cap = T * K + E_total * (bm - 1);
  route_sort_kernel<<<1, kSortThreads, 0, stream>>>(logits, T, E, topk, score, renorm, n_shared, shared_w, bm, cap, ids,
                                                    weights, counts, offsets, sorted, block_expert, num_padded);
  return hipGetLastError();
}

hipError_t launch_align_sort(const int32_t* ids, int T, int K, int E, int bm, int32_t* counts, int32_t* offsets,
                             int32_t* sorted, int32_t* block_expert, int32_t* num_padded, hipStream_t stream) {
  const int n = T * K;
  const int cap = n + E * (bm - 1);
  const int grid = n > 0 ? (n + kSortChunk - 1) / kSortChunk : 1;
  align_sort_kernel<<<grid, kSortThreads, 0, stream>>>(ids, n, E, bm, cap, counts, offsets, sorted, block_expert,
                                                       num_padded);
  return hipGetLastError();
}

}  // namespace moe
