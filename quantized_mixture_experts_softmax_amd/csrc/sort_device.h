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

// Rank key of expert e's logit v: larger keys rank first.  The high word is the logit's
// bits mapped to an unsigned order (-0 folded into +0, so equal logits have equal high
// words), the low word ~e, so of two equal logits the lower id ranks first: one 64-bit
// compare decides "ranks before" by value, then id.  Every key of a finite logit is > 0.
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  uint32_t u = __float_as_uint(v + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)~e;
}
// The logit a key was made from (+0 for -0: the weights computed from it are the same).
__device__ __forceinline__ float rank_key_value(uint64_t k) {
  uint32_t u = (uint32_t)(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

// LDS bytes route_sort_block needs: rank keys [T][E + 1], the winners [T * topk] (value
// and expert), selection masks and group prefixes [E][ceil(T / 64)], counts and offsets
// of the E + n_shared experts, the scan's wave sums, and 128 bytes of slack (the rank
// pass reads whole batches of 16 keys; reads past a row's end in the last batch are not
// used).
__host__ __device__ constexpr size_t route_sort_lds_bytes(int T, int E, int topk, int n_shared, int groups) {
  return ((size_t)T * (E + 1) * 8 + (size_t)T * topk * 8 + 8 + (size_t)E * groups * 12 +
          (size_t)(2 * (E + n_shared) + 1) * 4 + (size_t)kSortWaves * 4 + 4 + 128 + 15) / 16 * 16;
}
// Largest batch route_sort_block serves: T * E <= kFuseLogits, T * (topk + shared) <=
// kSortChunk, E <= kSmallE, shared <= 32, so T * (E + 1) <= kFuseLogits + kSortChunk and
// E * groups <= kFuseLogits / 64 + kSmallE.
constexpr size_t kRouteSortLdsMax =
    ((size_t)(kFuseLogits + kSortChunk) * 8 + (size_t)kSortChunk * 8 + 8 + (size_t)(kFuseLogits / 64 + kSmallE) * 12 +
     (size_t)(2 * (kSmallE + 32) + 1) * 4 + (size_t)kSortWaves * 4 + 4 + 128 + 15) / 16 * 16;

// Router + align-sort of a small batch (E <= kSmallE, T * K <= kSortChunk, T * E <=
// kFuseLogits) by one kSortThreads workgroup, all intermediates in the LDS at `lds`
// (route_sort_lds_bytes(T, E, topk, n_shared, ceil(T / 64)) bytes, 16-byte aligned).
// Expert-major: wave task (expert e, group of 64 tokens) counts, for each token (lane),
// the experts whose rank key exceeds e's (rank_key: a larger logit, or an equal one with a
// lower id); the ballot of the lanes with a count below topk is the expert's selection
// mask for the group.  An expert is chosen at most once per token, so the stable row of
// slot (t, j) inside its expert is a popcount prefix of the masks.  Shared experts are
// chosen by every token, at position t.  The ids, weights and sort equal those of the
// separate router and align-sort kernels.
// The logits a thread of route_sort_block stages: element tid + k * kSortThreads of the
// [T, E] array.
struct RouteLogits {
  float v[kFuseLogits / kSortThreads];
};
__device__ __forceinline__ void route_sort_load(const float* __restrict__ logits, int T, int E, RouteLogits& r) {
  const int tid = (int)threadIdx.x, n = T * E;
  if (n == 0) return;  // (uniform) logits may be NULL
  // clamped, unconditional loads: straight-line code keeps them all in flight together
  // (elements past n are loaded again and not used)
#pragma unroll
  for (int k = 0; k < kFuseLogits / kSortThreads; ++k) r.v[k] = logits[min(tid + k * kSortThreads, n - 1)];
}

// Its barriers order LDS only (all exchange between threads goes through LDS), so global
// loads in flight are not waited for there.
__device__ __forceinline__ void route_sort_block(const RouteLogits& lv, int T, int E, int topk, int score,
                                                 int renorm, int n_shared, float shared_w, int bm, int cap,
                                                 uint8_t* lds, const RouteSortOut& o) {
  const int tid = (int)threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: task bounds and addresses stay scalar
  const int KP = topk + n_shared, Et = E + n_shared, n = T * KP, G = (T + kWave - 1) / kWave;
  // (offsets from `lds`, which is 16-byte aligned: an integer round trip of the pointer
  // would lose its LDS address space and turn every access into a flat one)
  const int ld = E + 1;                                      // key row stride (spreads the lanes over banks)
  uint64_t* key = (uint64_t*)lds;                            // [T][E + 1]
  float* sel_v = (float*)(key + (size_t)T * ld + 16);        // [T][topk] (after 128 bytes of slack)
  int* sel_e = (int*)(sel_v + (size_t)T * topk);             // [T][topk]
  const size_t mask_off = ((size_t)T * ld * 8 + 128 + (size_t)T * topk * 8 + 7) & ~(size_t)7;
  unsigned long long* mask = (unsigned long long*)(lds + mask_off);  // [E][G]
  int* pre = (int*)(mask + (size_t)E * G);                   // [E][G]
  int* cnt = pre + (size_t)E * G;                            // [Et]
  int* offs = cnt + Et;                                      // [Et + 1]
  int* wsum = offs + Et + 1;                                 // [kSortWaves]
  int* grand_total = wsum + kSortWaves;

#pragma unroll
  for (int k = 0; k < kFuseLogits / kSortThreads; ++k) {
    const int i = tid + k * kSortThreads;
    if (i < T * E) {
      const int t = i / E, e = i - t * E;
      key[(size_t)t * ld + e] = rank_key(lv.v[k], e);
    }
  }
  lds_barrier();
  for (int task = w; task < E * G; task += kSortWaves) {  // wave-uniform
    const int e = task / G, g = task - e * G, t = g * kWave + lane;
    const bool ok = t < T;
    const uint64_t* row = key + (size_t)(ok ? t : 0) * ld;
    const uint64_t ke = row[e];
    // experts ranking before e: keys above e's.  Whole batches of 16 keys read with
    // immediate offsets from one base and counted without bound checks; only the last,
    // partial batch checks its (wave-uniform) bound, its reads past the row unused.
    int rank = 0;
    const int full = E & ~15;
    for (int j0 = 0; j0 < full; j0 += 16) {
      uint64_t x[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) x[k] = row[j0 + k];
#pragma unroll
      for (int k = 0; k < 16; ++k) rank += x[k] > ke ? 1 : 0;
    }
    if (full < E) {
      uint64_t x[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) x[k] = row[full + k];
#pragma unroll
      for (int k = 0; k < 16; ++k) rank += (full + k < E && x[k] > ke) ? 1 : 0;
    }
    const float v = rank_key_value(ke);
    const bool sel = ok && rank < topk;
    const unsigned long long m = __ballot(sel);
    if (lane == 0) mask[task] = m;
    if (sel) {
      sel_e[t * topk + rank] = e;
      sel_v[t * topk + rank] = v;
    }
  }
  lds_barrier();
  // Per-expert counts (shared experts: every token), group prefixes and padded offsets,
  // by wave 0 alone: Et <= kSmallE + 32 <= 2 * kWave experts, expert lane + 64 h in
  // element h of a lane, scanned lane by lane (h = 0 first), one barrier in all.
  if (w == 0) {
    int c[2], pd[2], s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = lane + kWave * h;
      int cc = e < Et ? T : 0;
      if (e < E) {
        cc = 0;
        for (int g = 0; g < G; ++g) {
          pre[e * G + g] = cc;
          cc += __popcll(mask[e * G + g]);
        }
      }
      c[h] = cc;
      pd[h] = (cc + bm - 1) / bm * bm;
      s[h] = pd[h];
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int n0 = __shfl_up(s[0], o, kWave), n1 = __shfl_up(s[1], o, kWave);
      if (lane >= o) {
        s[0] += n0;
        s[1] += n1;
      }
    }
    const int tot0 = __shfl(s[0], kWave - 1, kWave);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = lane + kWave * h;
      if (e < Et) {
        cnt[e] = c[h];
        offs[e] = (h ? tot0 : 0) + s[h] - pd[h];
      }
    }
    if (lane == kWave - 1) {
      offs[Et] = tot0 + s[1];
      *grand_total = tot0 + s[1];
    }
  }
  lds_barrier();
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
      const uint64_t* krow = key + (size_t)t * ld;
      wt = slot_weight(sel_v + t * topk, j, topk, score, renorm, [&](int i) { return rank_key_value(krow[i]); }, E);
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

namespace moe {
// Loads the logits, then routes and sorts (route_sort_load + route_sort_block).
__device__ __forceinline__ void route_sort_block(const float* __restrict__ logits, int T, int E, int topk, int score,
                                                 int renorm, int n_shared, float shared_w, int bm, int cap,
                                                 uint8_t* lds, const RouteSortOut& o) {
  RouteLogits lv;
  route_sort_load(logits, T, E, lv);
  route_sort_block(lv, T, E, topk, score, renorm, n_shared, shared_w, bm, cap, lds, o);
}
}  // namespace moe
