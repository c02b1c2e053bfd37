// Sorting building blocks shared by the align-sort kernels and the fused router + sort
// (one 1024-thread workgroup): a block-wide scan, the pad / block-owner fill, and the
// route + sort of a small batch computed entirely in LDS.
#pragma once
#include "moe_device.h"
#include "route_device.h"

namespace moe {

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kSortChunk = 4096;
constexpr int kFuseLogits = 8192;  // T * E limit of the fused router + sort

// Block-wide exclusive scan of one value per thread (kSortThreads threads).
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = lane_id(), w = (int)threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  if (w == 0) {
    int x = lane < kSortWaves ? wsum[lane] : 0;
    int xi = x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int n = __shfl_up(xi, o, kWave);
      if (lane >= o) xi += n;
    }
    if (lane < kSortWaves) wsum[lane] = xi - x;  // exclusive wave base
    if (lane == kSortWaves - 1) *total = xi;
  }
  __syncthreads();
  return wsum[w] + inc - v;
}

// Rows p = start, start + stride, ... < cap: pad rows (past an expert's count inside its
// padded run, or past the total) get the sentinel n; the first row of every block gets
// the block's owner (-1 past the total).  offs [E + 1] and cnt [E] are the padded
// offsets and counts.
__device__ __forceinline__ void fill_pads_owners(const int* offs, const int* cnt, int E, int total, int n, int bm,
                                                 int cap, int start, int stride, int32_t* __restrict__ sorted,
                                                 int32_t* __restrict__ block_expert) {
  for (int p = start; p < cap; p += stride) {
    bool pad = p >= total;
    if (!pad) {
      int lo = 0, hi = E - 1;  // last e with offs[e] <= p
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offs[mid] <= p) lo = mid; else hi = mid - 1;
      }
      pad = p >= offs[lo] + cnt[lo];
      if ((p % bm) == 0) block_expert[p / bm] = lo;
    } else if ((p % bm) == 0 && p / bm < cap / bm) {
      block_expert[p / bm] = -1;
    }
    if (pad) sorted[p] = n;
  }
}

// Outputs of route_sort_block; any pointer may be null (not written).  `sorted` and
// `block_expert` may point to LDS.
struct RouteSortOut {
  int32_t* ids;
  float* weights;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* block_expert;
  int32_t* num_padded;
};

// LDS bytes route_sort_block needs: logits [T][E + 1], the winners [T * topk] (value and
// expert), selection masks and group prefixes [E][ceil(T / 64)], counts and offsets of
// the E + n_shared experts, and the scan's wave sums.
__host__ __device__ constexpr size_t route_sort_lds_bytes(int T, int E, int topk, int n_shared, int groups) {
  return ((size_t)T * (E + 1) * 4 + (size_t)T * topk * 8 + 8 + (size_t)E * groups * 12 +
          (size_t)(2 * (E + n_shared) + 1) * 4 + (size_t)kSortWaves * 4 + 4 + 15) / 16 * 16;
}
// Largest batch route_sort_block serves: T * E <= kFuseLogits, T * (topk + shared) <=
// kSortChunk, E <= kSmallE, shared <= 32, so T * (E + 1) <= kFuseLogits + kSortChunk and
// E * groups <= kFuseLogits / 64 + kSmallE.
constexpr size_t kRouteSortLdsMax =
    ((size_t)(kFuseLogits + kSortChunk) * 4 + (size_t)kSortChunk * 8 + 8 + (size_t)(kFuseLogits / 64 + kSmallE) * 12 +
     (size_t)(2 * (kSmallE + 32) + 1) * 4 + (size_t)kSortWaves * 4 + 4 + 15) / 16 * 16;

// Router + align-sort of a small batch (E <= kSmallE, T * K <= kSortChunk, T * E <=
// kFuseLogits) by one kSortThreads workgroup, all intermediates in the LDS at `lds`.
// Lane t of a wave task counts the experts ranking before e in its token (an expert
// j < e ranks before on >=, j > e on >: the id tie rule); an expert is chosen at most
// once per token, so the masks' popcount prefix is the slot's stable row.
// (route_sort_lds_bytes(T, E, topk, n_shared, ceil(T / 64)) bytes, 16-byte aligned).
// Expert-major: wave task
// (expert e, group of 64 tokens) ranks each token's logit of e against the token's row
// staged in LDS; the ballot of the winning lanes is the expert's selection mask for the
// group, so the stable row of slot (t, j) inside its expert is a popcount prefix of the
// masks.  Shared experts are chosen by every token, at position t.  The ids, weights and
// sort equal those of the separate router and align-sort kernels.
__device__ __forceinline__ void route_sort_block(const float* __restrict__ logits, int T, int E, int topk, int score,
                                                 int renorm, int n_shared, float shared_w, int bm, int cap,
                                                 uint8_t* lds, const RouteSortOut& o) {
  const int tid = (int)threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int KP = topk + n_shared, Et = E + n_shared, n = T * KP, G = (T + kWave - 1) / kWave, ld = E + 1;
  float* lg = (float*)lds;                                   // [T][E + 1]
  float* sel_v = lg + (size_t)T * ld;                        // [T][topk]
  int* sel_e = (int*)(sel_v + (size_t)T * topk);             // [T][topk]
  unsigned long long* mask = (unsigned long long*)(((uintptr_t)(sel_e + (size_t)T * topk) + 7) & ~(uintptr_t)7);
  int* pre = (int*)(mask + (size_t)E * G);                   // [E][G]
  int* cnt = pre + (size_t)E * G;                            // [Et]
  int* offs = cnt + Et;                                      // [Et + 1]
  int* wsum = offs + Et + 1;                                 // [kSortWaves]
  int* grand_total = wsum + kSortWaves;

  for (int i = tid; i < T * E; i += kSortThreads) {
    const int t = i / E;
    lg[t * ld + (i - t * E)] = logits[i];
  }
  __syncthreads();
  for (int task = w; task < E * G; task += kSortWaves) {  // wave-uniform
    const int e = task / G, g = task - e * G, t = g * kWave + lane;
    const bool ok = t < T;
    const float* row = lg + (ok ? t : 0) * ld;
    const float v = row[e];
    int rank = 0;
    for (int j = 0; j < e; ++j) rank += row[j] >= v ? 1 : 0;
    for (int j = e + 1; j < E; ++j) rank += row[j] > v ? 1 : 0;
    const bool sel = ok && rank < topk;
    const unsigned long long m = __ballot(sel);
    if (lane == 0) mask[task] = m;
    if (sel) {
      sel_e[t * topk + rank] = e;
      sel_v[t * topk + rank] = v;
    }
  }
  __syncthreads();
  // per-expert counts (shared experts: every token) and group prefixes
  if (tid < Et) {
    int c = T;
    if (tid < E) {
      c = 0;
      for (int g = 0; g < G; ++g) {
        pre[tid * G + g] = c;
        c += __popcll(mask[tid * G + g]);
      }
    }
    cnt[tid] = c;
  }
  __syncthreads();
  const int padded = tid < Et ? (cnt[tid] + bm - 1) / bm * bm : 0;
  const int off = block_exclusive_scan(padded, wsum, grand_total);
  if (tid < Et) offs[tid] = off;
  if (tid == 0) offs[Et] = *grand_total;
  __syncthreads();
  const int total = *grand_total;
  if (tid < Et) {
    if (o.counts) o.counts[tid] = cnt[tid];
    if (o.offsets) o.offsets[tid] = offs[tid];
  }
  if (tid == 0) {
    if (o.offsets) o.offsets[Et] = total;
    if (o.num_padded) o.num_padded[0] = total;
  }
  // slots: ids, weights and their sorted rows
  for (int q = tid; q < n; q += kSortThreads) {
    const int t = q / KP, j = q - t * KP;
    int e, pos;
    float wt;
    if (j < topk) {
      e = sel_e[t * topk + j];
      wt = slot_weight(sel_v + t * topk, j, topk, score, renorm, lg + t * ld, E);
      const int g = t / kWave, l = t % kWave;
      const unsigned long long below = l ? (~0ull >> (kWave - l)) : 0ull;
      pos = offs[e] + pre[e * G + g] + __popcll(mask[e * G + g] & below);
    } else {
      e = E + (j - topk);
      wt = shared_w;
      pos = offs[e] + t;
    }
    if (o.ids) o.ids[q] = e;
    if (o.weights) o.weights[q] = wt;
    if (o.sorted) o.sorted[pos] = q;
  }
  if (o.sorted) fill_pads_owners(offs, cnt, Et, total, n, bm, cap, tid, kSortThreads, o.sorted, o.block_expert);
}

}  // namespace moe
