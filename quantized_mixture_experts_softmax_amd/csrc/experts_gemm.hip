// Grouped expert GEMMs on MFMA for gfx950, and the ordered top-k combine.
//
// Stage 1: per padded block of BM sorted rows of expert e, C = A . w1[e]^T over the
// gate rows and the matching up rows, with h = bf16(silu(gate) * up) in the
// epilogue (pages: "rocm_aiter_moe", AiterExperts -- SiLU, act-and-mul -- and
// rocm_aiter_fused_experts; w13 stacks gate rows over up rows).
// Stage 2: y = A . w2[e]^T, written as fp32 to a per-slot row; the combine kernel
// then multiplies each of a token's rows by the slot's top-k weight and sums them in
// ascending slot order (the top-k weighted reduction the pages place inside the
// expert computation: AiterExperts.finalize_weight_and_reduce_impl is a no-op).
//
// Work decomposition (one 256-thread workgroup = 4 wave64s):
//   * a workgroup owns one BM-row block (one expert) and a strip of output columns;
//     each wave owns NT 16-column MFMA tiles of that strip (in stage 1, NT/2 gate
//     tiles and the NT/2 matching up tiles, so the SiLU-and-mul stays in registers);
//   * K runs in chunks of 128.  The A tile (BM x 128) is shared by all waves and is
//     staged through LDS (double-buffered, padded rows); each weight element is used
//     by exactly one wave, so weights go from HBM straight to registers with 16-byte
//     loads, one chunk ahead of the MFMAs, and are never copied through LDS;
//   * within a chunk, lane l (group g = l/16) owns K elements [32g, 32g+32) for its
//     16 B MXFP4 / 32 B FP8 weight load; the bf16 MFMA consumes them as 4 K-steps of
//     8 and the A operand is read from LDS with the same K permutation, so A and B
//     agree on every K index.  One MXFP4 scale byte covers the lane's 32 elements,
//     which is also the K-block the scaled FP4 MFMA associates with that lane.
// MFMA per format: w4a16 dequantises MXFP4 to bf16 in registers with
// v_cvt_scalef32_pk_bf16_fp4 (exact) and runs v_mfma_f32_16x16x32_bf16; w4a4 runs
// v_mfma_scale_f32_16x16x128_f8f6f4 on e2m1 codes with the E8M0 bytes as operand
// scales; FP8 runs the same instruction on e4m3 codes at unit scale, and the fp32
// block scales (a_scale[row, chunk] * w_scale[col block, chunk]) are applied to each
// chunk's partial product, per-channel scales in the epilogue.
// Workgroup ids are remapped so that each XCD walks a contiguous range of
// (block, column strip) pairs, blocks fastest: consecutive blocks of one expert
// share the expert's weight strip in that XCD's L2.
#include "gemm_common.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "sort_device.h"

#include <algorithm>
#include <atomic>

namespace moe {


// MFMA column tiles per wave of the small-block kernel.  bf16 activations cost as
// many bytes per row as four MXFP4 weight rows, so that path takes wider strips to
// amortise the activation reads over more weight rows.
#ifndef MOE_KSPLIT_NT_BF16
#define MOE_KSPLIT_NT_BF16 8
#endif
#ifndef MOE_DMA_A  // 64/128-row kernel, bf16 activations: A tile global -> LDS by direct loads
#define MOE_DMA_A 1
#endif
#ifndef MOE_DMA_AQ  // the same for the quantised activation formats, one chunk ahead: measured
#define MOE_DMA_AQ 0  // slower than their register rings (w4a4 -1%, FP8 block -4%, FP8 channel -17%)
#endif
#ifndef MOE_SCALE_DWORD
#define MOE_SCALE_DWORD 1
#endif
#ifndef MOE_KSPLIT_NT_Q
#define MOE_KSPLIT_NT_Q 4
#endif
#ifndef MOE_LDS_GEMM  // 128-row blocks on tiled weights: the LDS-staged kernel of gemm_lds.hip
#define MOE_LDS_GEMM 1
#endif
// Column tiles per wave of the 64-row kernel for w4a4 (4 for the other formats, except
// stage 2 of w4a16 below).  Six tiles cut the activation bytes per flop through the
// vector-memory return path, which bounds w4a4 here: prefill-w4a4 (T = 8192) 1.26 against
// 1.33 ms per step on MI355X (stage 2 -13%, stage 1 -2.5%), at ring depth 1 (depth 2
// spills at six tiles).
#ifndef MOE_NT_F4A4
#define MOE_NT_F4A4 6
#endif
// ... and for stage 2 of w4a16 (each A fragment read from LDS feeds six tiles): prefill
// (T = 8192) stage 2 596 against 617 us; stage 1 measured the same at four and six
#ifndef MOE_NT_W4A16_S2
#define MOE_NT_W4A16_S2 6
#endif
// Workgroups per CU the small-block launch is sized for (strips per workgroup grow
// until the grid is about this many workgroups per CU).
#ifndef MOE_KSPLIT_WGS_PER_CU
#define MOE_KSPLIT_WGS_PER_CU 2
#endif

template <int STAGE, int WF, int AF, int BM, int NT, int WL, int EPI>
// 64-row blocks: the register budget keeps two waves per SIMD resident (measured: up to
// 1.8x faster than one); 128-row blocks would spill under that budget.
__global__ __launch_bounds__(256, BM <= 64 ? 2 : 1) void moe_gemm_kernel(const GemmParams p) {
  using WLay = WLayout<WF, WL>;
  constexpr int ARB = (AF == kABf16) ? 256 : (AF == kAMxfp4 ? 64 : 128);  // A bytes per row per chunk
  constexpr int APC = ARB / 16;                                            // 16 B pieces per row per chunk
  constexpr int EPP = 128 / APC;                                           // elements per piece
  constexpr int LROW = ARB + 16;                                           // padded LDS row (bytes)
  constexpr int NPIECE = BM * APC;
  constexpr int AIT = (NPIECE + 255) / 256;
  constexpr int MT = BM / 16;
  constexpr int COLS_PER_WG = (STAGE == 1) ? 32 * NT : 64 * NT;
  static_assert(STAGE == 2 || NT % 2 == 0, "stage 1 pairs gate and up tiles");

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * LROW];
  __shared__ float lds_as[2][BM];
  __shared__ uint32_t lds_as4[2][BM];

  const int n_tiles = (p.N + COLS_PER_WG - 1) / COLS_PER_WG;
  const int G = p.num_blocks * n_tiles;
  const int lid = xcd_remap((int)blockIdx.x, G);
  const int b = lid % p.num_blocks;
  const int nt_idx = lid / p.num_blocks;
  const int npad = p.num_padded[0];
  if (b * BM >= npad) return;
  const int e = p.block_expert[b];
  if (e < 0) return;

  const int tid = (int)threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile rows and block scales stay scalar
  const int K = p.K, nch = (K + 127) / 128;
  const int TK = p.T * p.slots_per_token;
  const size_t a_row_bytes = (AF == kABf16) ? (size_t)K * 2 : (AF == kAMxfp4 ? (size_t)K / 2 : (size_t)K);

  // ---- A rows this thread stages into LDS ----
  // kDmaA (one-chunk-ahead loop): direct global -> LDS loads into an unpadded tile (ARB-byte
  // rows); position pv of row r holds the row's 16-byte unit pv ^ aswz(r), so the 16 rows
  // of a fragment read fall in 16 different bank groups.  The data never passes through
  // registers, which takes it off the vector-memory return path.
  constexpr bool kDmaA = (AF == kABf16) ? (MOE_DMA_A != 0) : (MOE_DMA_AQ != 0);
  constexpr int RPB = 256 / ARB;  // tile rows per 256 bytes
  auto aswz = [](int r) { return (r / RPB) & (APC - 1); };
  const uint8_t* a_src[AIT];
  bool a_ok[AIT];
  int a_lds[AIT], a_k0[AIT];
#pragma unroll
  for (int it = 0; it < AIT; ++it) {
    const int piece = tid + 256 * it;
    const int r = piece / APC, pc = piece % APC;
    bool ok = piece < NPIECE;
    int arow = 0;
    if (ok) {
      if (STAGE == 1) {
        const int slot = p.sorted_slots[b * BM + r];
        ok = slot < TK;
        arow = ok ? slot / p.slots_per_token : 0;
      } else {
        arow = b * BM + r;
      }
    }
    const int pu = kDmaA ? (pc ^ aswz(r)) : pc;  // the row's unit this thread moves
    a_src[it] = (const uint8_t*)p.a + (size_t)arow * a_row_bytes + pu * 16;
    a_ok[it] = ok;
    a_lds[it] = (piece < NPIECE ? r : 0) * LROW + pc * 16;
    a_k0[it] = pu * EPP;
  }
  // ---- activation scale row owned by thread tid < BM ----
  int s_row = 0;
  bool s_ok = false;
  if (AF != kABf16 && tid < BM) {
    if (STAGE == 1) {
      const int slot = p.sorted_slots[b * BM + tid];
      s_ok = slot < TK;
      s_row = s_ok ? slot / p.slots_per_token : 0;
    } else {
      s_row = b * BM + tid;
      s_ok = true;
    }
  }

  // ---- weight rows of this wave's tiles (lane li = column inside the tile) ----
  const int nbn = (p.Nw + 127) / 128, nbk = nch;
  const uint8_t* w_src[NT];
  const uint8_t* ws_src[NT];
  const float* wsb_src[NT];
  float wsc[NT];
  int col[NT], wrow[NT];
  bool col_ok[NT];
  const int cb_u = nt_idx * COLS_PER_WG + w * (NT / 2) * 16;  // stage 1: the wave's first output column
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int c, trow;
    if (STAGE == 1) {
      // the wave's output columns [cb, cb + 8 NT): separated rows pair gate tile t with
      // up tile t + NT/2; interleaved rows are tiles [2 cb + 16 t, +16), gate and up of
      // columns cb + 8 t + (0..7) in alternate lanes
      const int cb = nt_idx * COLS_PER_WG + w * (NT / 2) * 16;
      if ((EPI && p.interleaved)) {
        c = cb + 8 * t + (li >> 1);
        col_ok[t] = 2 * cb + 16 * t < p.Nw;
        trow = col_ok[t] ? 2 * cb + 16 * t : 0;
      } else {
        const int tt = t % (NT / 2);
        c = cb + tt * 16 + li;
        col_ok[t] = c < p.N;
        trow = col_ok[t] ? (t < NT / 2 ? c - li : p.N + c - li) : 0;
      }
    } else {
      c = nt_idx * COLS_PER_WG + w * NT * 16 + t * 16 + li;
      col_ok[t] = c < p.N;
      trow = col_ok[t] ? c - li : 0;
    }
    col[t] = c;
    wrow[t] = trow + li;
    w_src[t] = WLay::data(p, e, trow, li, g, lane, K);
    ws_src[t] = (WF == kWMxfp4) ? WLay::scale(p, e, trow, li, g, lane, K) : nullptr;
    if constexpr (WF == kWFp8Block) {
      // the tile's first weight row, from wave-uniform values only (trow is 0 in the lanes
      // past N), so the block scale is one scalar load per chunk, not a vector load
      const int c0 = (STAGE == 1) ? cb_u + (t % (NT / 2)) * 16 : nt_idx * COLS_PER_WG + w * NT * 16 + t * 16;
      const int r0 = c0 < p.N ? ((STAGE == 1 && t >= NT / 2) ? p.N + c0 : c0) : 0;
      wsb_src[t] = (const float*)p.w_scale + ((size_t)e * nbn + r0 / 128) * nbk;
    } else {
      wsb_src[t] = nullptr;
    }
    wsc[t] = (WF == kWFp8Channel) ? ((const float*)p.w_scale)[wsc_index(p, e, trow + li)] : 1.0f;
  }
  // Tiled MXFP4 with MXFP4 activations: a lane's E8M0 byte for tile t is byte `lane` of
  // the 64-byte scale part of tile t's block.  One dword load per lane fetches the scales
  // of four tiles of a chunk (group q: lane l reads bytes [4 (l % 16), +4) of tile
  // 4 q + l / 16) in place of a byte load per tile; each lane then takes its byte of tile
  // t from lane 16 (t % 4) + l / 4 of group t / 4 with ds_bpermute.  On large w4a4
  // batches the vector-memory return path (TD), not HBM or MFMA, bounds this kernel, and
  // a byte load costs it about half a 16-byte one (counters on MI355X); the step gained
  // 6%.  w4a16, whose LDS pipe carries four times the A reads, lost 9% with it and keeps
  // the byte loads.
  constexpr bool kScaleDword = (WF == kWMxfp4) && (AF == kAMxfp4) && (WL != 0) && (MOE_SCALE_DWORD != 0);
  constexpr int NG = (NT + 3) / 4;  // scale dwords per lane and chunk
  static_assert(!kScaleDword || NT <= 4 * kScaleGroups, "WeightRegs holds the scale dwords of this many tiles");
  const uint8_t* ws4_src[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    ws4_src[q] = nullptr;
    if constexpr (kScaleDword) {
      // lanes whose tile 4 q + l / 16 does not exist read the last tile's bytes (unused)
      const int tt = min(4 * q + (lane >> 4), NT - 1);
      const uint8_t* b = ws_src[0];
#pragma unroll
      for (int t = 1; t < NT; ++t) b = (tt == t) ? ws_src[t] : b;
      ws4_src[q] = b - lane + 4 * (lane & 15);
    }
  }

  auto load_a = [&](int c, i32x4 (&reg)[AIT]) {
#pragma unroll
    for (int it = 0; it < AIT; ++it)
      reg[it] = ld16(a_src[it], (size_t)c * ARB, a_ok[it] && (c * 128 + a_k0[it] < K));
  };
  // (chunks past the end, which the ring loop prefetches, read the zero page)
  auto load_as = [&](int c, float& fs, uint32_t& qs) {
    if constexpr (AF == kAFp8G128) {
      fs = ldf((const float*)p.a_scale, (size_t)s_row * nch + (c < nch ? c : 0), s_ok && c < nch);
    } else if constexpr (AF == kAMxfp4) {
      const uint8_t* sp = (const uint8_t*)p.a_scale + (size_t)s_row * (K / 32) + (c < nch ? c : 0) * 4;
      uint32_t v = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) v |= ld8(sp, q, s_ok && c * 128 + 32 * q < K) << (8 * q);
      qs = v;
    }
  };
  auto store_a = [&](int buf, const i32x4 (&reg)[AIT], float fs, uint32_t qs) {
#pragma unroll
    for (int it = 0; it < AIT; ++it)
      if (tid + 256 * it < NPIECE) *(i32x4*)(&lds_a[buf][a_lds[it]]) = reg[it];
    if (tid < BM) {
      if constexpr (AF == kAFp8G128) lds_as[buf][tid] = fs;
      if constexpr (AF == kAMxfp4) lds_as4[buf][tid] = qs;
    }
  };
  auto load_w = [&](int c, WeightRegs<WF, NT>& r) {
    const bool kok = c * 128 + 32 * g < K;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (WF == kWBf16) {  // the lane's 32 bf16 values, one 16 B piece per K-step of 8
#pragma unroll
        for (int q = 0; q < 4; ++q) r.w[t][q] = ld16(w_src[t], (size_t)c * WLay::kDataStride + 16 * q, kok);
      } else if constexpr (WF == kWMxfp4) {
        r.w[t][0] = ld16(w_src[t], (size_t)c * WLay::kDataStride, kok);
        if constexpr (!kScaleDword) r.s[t] = ld8(ws_src[t], (size_t)c * WLay::kScaleStride, kok);
      } else {
        r.w[t][0] = ld16(w_src[t], (size_t)c * WLay::kDataStride, kok);
        r.w[t][WF == kWMxfp4 ? 0 : 1] = ld16(w_src[t], (size_t)c * WLay::kDataStride + WLay::kHiOff, kok);
        if constexpr (WF == kWFp8Block) r.sb[t] = ld_uniform_f32(wsb_src[t] + (c < nch ? c : 0));
      }
    }
    // (the tail chunk's block holds zero scale bytes past K; chunks past the end read the zero page)
    if constexpr (kScaleDword) {
#pragma unroll
      for (int q = 0; q < NG; ++q) r.s4[q] = ld_global<uint32_t>(ws4_src[q], (size_t)c * WLay::kScaleStride, c < nch);
    }
  };
  // the E8M0 byte of tile t for this lane
  auto wscale = [&](const WeightRegs<WF, NT>& wr, int t) -> uint32_t {
    if constexpr (kScaleDword) {
      const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * (t % 4) + (lane >> 2)) << 2, (int)wr.s4[t / 4]);
      return (v >> (8 * (lane & 3))) & 0xFFu;
    } else {
      return wr.s[t];
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (AF == kAFp8Token) if (tid < BM) lds_as[0][tid] = s_ok ? ((const float*)p.a_scale)[(size_t)s_row * p.asc_rs] : 0.0f;

  // MFMAs of one chunk: A from LDS buffer buf, weights wr
  auto compute = [&](int buf, const WeightRegs<WF, NT>& wr) {
    const uint8_t* la = lds_a[buf];
    uint32_t wsb[NT] = {};
    if constexpr (WF == kWMxfp4) {
#pragma unroll
      for (int t = 0; t < NT; ++t) wsb[t] = wscale(wr, t);
    }
    if constexpr (AF == kABf16) {
      // w4a16: fp4 -> bf16 in registers, 4 K-steps of 8 per chunk
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 af[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
          af[m] = kDmaA ? *(const bf16x8*)(la + (m * 16 + li) * ARB + 16 * ((4 * g + st) ^ aswz(m * 16 + li)))
                        : *(const bf16x8*)(la + (m * 16 + li) * LROW + 64 * g + 16 * st);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          bf16x8 bfr;
          if constexpr (WF == kWBf16) {  // unquantised: the loaded bf16 values as they are
            bfr = __builtin_bit_cast(bf16x8, wr.w[t][st]);
          } else {
            const float sc = e8m0_to_f32(wsb[t]);
            const uint32_t dw = (uint32_t)wr.w[t][0][st];
            const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 0);
            const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 1);
            const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 2);
            const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 3);
            bfr = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          }
#pragma unroll
          for (int m = 0; m < MT; ++m)
            acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bfr, acc[m][t], 0, 0, 0);
        }
      }
    } else if constexpr (AF == kAMxfp4) {
      // w4a4: scaled FP4 MFMA, E8M0 bytes as operand scales
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const i32x4 a4 = kDmaA ? *(const i32x4*)(la + (m * 16 + li) * ARB + 16 * (g ^ aswz(m * 16 + li)))
                               : *(const i32x4*)(la + (m * 16 + li) * LROW + 16 * g);
        const i32x8 a8 = {a4[0], a4[1], a4[2], a4[3], 0, 0, 0, 0};
        const int sa = (int)((lds_as4[buf][m * 16 + li] >> (8 * g)) & 0xFFu);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const i32x8 b8 = {wr.w[t][0][0], wr.w[t][0][1], wr.w[t][0][2], wr.w[t][0][3], 0, 0, 0, 0};
          acc[m][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[m][t], 4, 4, 0, sa, 0,
                                                                        (int)wsb[t]);
        }
      }
    } else {
      // FP8 e4m3 x e4m3 at unit operand scale
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int R = m * 16 + li;
        const i32x4 lo = kDmaA ? *(const i32x4*)(la + R * ARB + 16 * ((2 * g) ^ aswz(R)))
                               : *(const i32x4*)(la + R * LROW + 32 * g);
        const i32x4 hi = kDmaA ? *(const i32x4*)(la + R * ARB + 16 * ((2 * g + 1) ^ aswz(R)))
                               : *(const i32x4*)(la + R * LROW + 32 * g + 16);
        const i32x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        // FP8 block scales: the products (row scale x weight block scale) of this chunk.  A
        // wave's tiles lie in one 128-row weight block, except that stage 1 with separated
        // gate and up rows has one block for its gate tiles [0, NT/2) and one for its up
        // tiles (16-row tiles in runs of 32 rows from a multiple of 32 never straddle a
        // block), so 4 or 8 products serve the m-tile's NT tiles.
        float sg[4], su[4];
        if constexpr (WF == kWFp8Block) {
          const bool two = STAGE == 1 && !(EPI && p.interleaved);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float asr = lds_as[buf][m * 16 + 4 * g + rr];
            sg[rr] = asr * wr.sb[0];
            su[rr] = two ? asr * wr.sb[NT / 2] : sg[rr];
          }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const i32x8 b8 = {wr.w[t][0][0], wr.w[t][0][1], wr.w[t][0][2], wr.w[t][0][3],
                            wr.w[t][WF == kWMxfp4 ? 0 : 1][0], wr.w[t][WF == kWMxfp4 ? 0 : 1][1],
                            wr.w[t][WF == kWMxfp4 ? 0 : 1][2], wr.w[t][WF == kWMxfp4 ? 0 : 1][3]};
          if constexpr (WF == kWFp8Block) {
            const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a8, b8, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[m][t][rr] += part[rr] * (t < NT / 2 ? sg[rr] : su[rr]);
          } else {
            acc[m][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[m][t], 0, 0, 0, 127, 0, 127);
          }
        }
      }
    }
  };

  // Two loop shapes, chosen per format by measurement on MI355X.  kPF == 0: chunk c + 1
  // is loaded at the top of iteration c (w4a16).  kPF >= 1: a ring where the loads of
  // chunks c + 1 .. c + kPF are in flight during chunk c's MFMAs, A staged in registers
  // (slot j % kPF for chunk j) and weights in ring slot j % (kPF + 1); the loop is
  // unrolled over the ring period so every slot index is a compile-time constant (a
  // register copy would wait for its load).  The per-chunk barrier orders the LDS A
  // buffers only (lds_barrier): a __syncthreads would also wait for every global load in
  // flight, i.e. drain the ring each chunk.
  // Ring depths measured on MI355X (prefill-sized batches): w4a16 0 (depth 1 is 40% slower,
  // 2 within 1%), w4a4 1 at six tiles per wave (2 spills there; at four tiles 2 was 6%
  // faster than 1, and six tiles at depth 1 beat both), FP8 block 1 and FP8 channel 2 (one more
  // spills and runs ~3x slower).
#ifndef MOE_PF_BF16
#define MOE_PF_BF16 0
#endif
#ifndef MOE_PF_F4A4
#define MOE_PF_F4A4 1  // w4a4 at more than four tiles per wave (four tiles: 2)
#endif
#ifndef MOE_PF_F8B
#define MOE_PF_F8B 1
#endif
#ifndef MOE_PF_F8C
#define MOE_PF_F8C 2
#endif
  constexpr int kPF = (AF == kABf16) ? MOE_PF_BF16
                                     : (AF == kAMxfp4 ? (NT > 4 ? MOE_PF_F4A4 : 2)
                                                      : (WF == kWFp8Channel ? MOE_PF_F8C : MOE_PF_F8B));
  auto chunk_barrier = [] { lds_barrier(); };
  // kDmaA: chunk c's A tile straight into LDS buffer buf (each wave's 64 pieces of a round
  // are 1 KB contiguous); rows past the batch and K past the end read the zero page
  auto dma_a = [&](int c, int buf) {
#pragma unroll
    for (int it = 0; it < AIT; ++it) {
      const bool ok = a_ok[it] && (c * 128 + a_k0[it] < K);
      const MOE_GLOBAL uint8_t* src =
          ok ? (const MOE_GLOBAL uint8_t*)a_src[it] + (size_t)c * ARB : (const MOE_GLOBAL uint8_t*)kZeroPage;
      dma16((const void*)src, &lds_a[buf][(size_t)(64 * w + 256 * it) * 16]);
    }
  };
  auto store_as = [&](int buf, float fs, uint32_t qs) {
    if (tid < BM) {
      if constexpr (AF == kAFp8G128) lds_as[buf][tid] = fs;
      if constexpr (AF == kAMxfp4) lds_as4[buf][tid] = qs;
    }
  };
  if constexpr (kDmaA) {
    // one chunk ahead: every load of a chunk (its A tile, the next chunk's activation scales
    // and weights) is waited for at the chunk's end, before the barrier that hands the
    // tile to the other waves
    WeightRegs<WF, NT> wr, wn;
    float fs = 0.f;
    uint32_t qs = 0;
    dma_a(0, 0);
    load_as(0, fs, qs);
    load_w(0, wr);
    store_as(0, fs, qs);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    chunk_barrier();
    for (int c = 0; c < nch; ++c) {
      const int buf = c & 1;
      const bool more = c + 1 < nch;
      if (more) {
        dma_a(c + 1, buf ^ 1);
        load_as(c + 1, fs, qs);
        load_w(c + 1, wn);
      }
      compute(buf, wr);
      if (more) {
        store_as(buf ^ 1, fs, qs);
        wr = wn;
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      chunk_barrier();
    }
  } else if constexpr (kPF == 0) {
    i32x4 areg[AIT];
    float fs = 0.f;
    uint32_t qs = 0;
    WeightRegs<WF, NT> wr, wn;
    load_a(0, areg);
    load_as(0, fs, qs);
    load_w(0, wr);
    store_a(0, areg, fs, qs);
    chunk_barrier();
    for (int c = 0; c < nch; ++c) {
      const int buf = c & 1;
      const bool more = c + 1 < nch;
      if (more) {
        load_a(c + 1, areg);
        load_as(c + 1, fs, qs);
        load_w(c + 1, wn);
      }
      compute(buf, wr);
      if (more) {
        store_a(buf ^ 1, areg, fs, qs);
        wr = wn;
      }
      chunk_barrier();
    }
  } else {
    constexpr int NA = kPF, NW = kPF + 1, U = NA * NW;  // lcm: NA and NA + 1 are coprime
    i32x4 areg[NA][AIT];
    float fsq[NA];
    uint32_t qsq[NA];
    WeightRegs<WF, NT> wq[NW];
    {
      i32x4 a0[AIT];
      float f0 = 0.f;
      uint32_t q0 = 0;
      load_a(0, a0);
      load_as(0, f0, q0);
      load_w(0, wq[0]);
#pragma unroll
      for (int j = 1; j <= kPF; ++j) {
        fsq[j % NA] = 0.f;
        qsq[j % NA] = 0;
        load_a(j, areg[j % NA]);
        load_as(j, fsq[j % NA], qsq[j % NA]);
        load_w(j, wq[j % NW]);
      }
      store_a(0, a0, f0, q0);
    }
    chunk_barrier();
    for (int c0 = 0; c0 < nch; c0 += U)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u;
      if (c >= nch) break;
      // chunk c + kPF goes into the slots chunk c (A, now in LDS) and c - 1 (weights) left
      fsq[(u + kPF) % NA] = 0.f;
      qsq[(u + kPF) % NA] = 0;
      load_a(c + kPF, areg[(u + kPF) % NA]);
      load_as(c + kPF, fsq[(u + kPF) % NA], qsq[(u + kPF) % NA]);
      load_w(c + kPF, wq[(u + kPF) % NW]);
      compute(c & 1, wq[u % NW]);
      if (c + 1 < nch) store_a((c + 1) & 1, areg[(u + 1) % NA], fsq[(u + 1) % NA], qsq[(u + 1) % NA]);
      chunk_barrier();
    }
  }


  // ---- epilogue ----
  if constexpr (STAGE == 1) {
    float bsv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) bsv[t] = (EPI && p.bias && col_ok[t]) ? bias_of(p, e, wrow[t]) : 0.0f;
    // pad rows: h is written as 0 (without a bias their projections are 0 and so is h; with
    // one, act(bias) must not reach the a2 quantiser, whose per-tensor scale covers all rows)
    bool padr[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) padr[m][rr] = EPI && p.bias && p.sorted_slots[b * BM + m * 16 + 4 * g + rr] >= TK;
    if ((EPI && p.interleaved)) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (!col_ok[t]) continue;  // wave-uniform: tiles never straddle the edge
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int row = m * 16 + 4 * g + rr;
            float v = acc[m][t][rr];
            if (WF == kWFp8Channel) v = v * lds_as[0][row] * wsc[t];
            if (EPI && p.weight_on_input) v *= fc1_weight(p, p.sorted_slots[b * BM + row]);
            v += bsv[t];
            const float up = __shfl_xor(v, 1, kWave);  // odd lane: the up row of the same column
            if (!(li & 1))
              p.h[(size_t)(b * BM + row) * p.N + col[t]] = padr[m][rr] ? 0 : (uint16_t)f32_to_bf16(glu<EPI>(p, v, up));
          }
        }
    } else {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT / 2; ++t) {
          if (!col_ok[t]) continue;
          const int tu = t + NT / 2;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int row = m * 16 + 4 * g + rr;
            float gv = acc[m][t][rr], uv = acc[m][tu][rr];
            if (WF == kWFp8Channel) {
              const float as = lds_as[0][row];
              gv = gv * as * wsc[t];
              uv = uv * as * wsc[tu];
            }
            if (EPI && p.weight_on_input) {
              const float fw = fc1_weight(p, p.sorted_slots[b * BM + row]);
              gv *= fw;
              uv *= fw;
            }
            gv += bsv[t];
            uv += bsv[tu];
            p.h[(size_t)(b * BM + row) * p.N + col[t]] = padr[m][rr] ? 0 : (uint16_t)f32_to_bf16(glu<EPI>(p, gv, uv));
          }
        }
    }
  } else {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = m * 16 + 4 * g + rr;
        const int slot = p.sorted_slots[b * BM + row];
        if (slot >= TK) continue;
        const float as = (WF == kWFp8Channel) ? lds_as[0][row] : 1.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (!col_ok[t]) continue;
          float v = acc[m][t][rr];
          if (WF == kWFp8Channel) v = v * as * wsc[t];
          if (EPI && p.bias) v += bias_of(p, e, col[t]);
          p.ybuf[(size_t)slot * p.N + col[t]] = v;
        }
      }
  }
}

// ---------------------------------------------------------------------------------
// Small-block kernel (BM <= 32 rows, the decode shape).  With few rows per expert
// the GEMM is a weight stream: every weight byte is used by at most BM rows, so the
// kernel must keep HBM reads in flight all the time.  The four waves of a workgroup
// share the output tiles of a column strip and split K between them (wave w takes
// chunks w, w+4, w+8, ...); each wave loads its A fragments (L2-resident
// activations) and weights straight into registers in MFMA operand layout, one
// chunk ahead of the MFMAs, with no LDS staging and no barrier in the K loop.  One
// workgroup walks `strips_per_wg` consecutive column strips of the same row block as
// a single stream, so the prefetch runs across strip boundaries and the start-up
// latency (block owner -> sorted slots -> rows) is paid once.  At the end of each
// strip the four partial sums are added through LDS in fixed wave order
// (deterministic; double-buffered, one barrier per strip) and wave 0 runs the
// epilogue while the other waves stream on.
template <int AF, int MT>
struct ARegs {
  i32x4 a[MT][AF == kABf16 ? 4 : (AF == kAMxfp4 ? 1 : 2)];  // 64 B / 16 B / 32 B per m-tile
  uint32_t sa[MT];                                          // MXFP4: E8M0 byte of the lane's row/group
  float as[MT][4];                                          // FP8 block: scales of the 4 output rows
};

template <int STAGE, int WF, int AF, int BM, int NT, int WL, int EPI>
__global__ __launch_bounds__(256) void moe_gemm_ksplit_kernel(const GemmParams p) {
  using WLay = WLayout<WF, WL>;
  constexpr int MT = BM / 16;
  constexpr int COLS_PER_STRIP = (STAGE == 1) ? 8 * NT : 16 * NT;
  constexpr int NACC = MT * NT * 4;
  constexpr int NA = (AF == kABf16) ? 4 : (AF == kAMxfp4 ? 1 : 2);
  static_assert(STAGE == 2 || NT % 2 == 0, "stage 1 pairs gate and up tiles");
  __shared__ float red[2][3][NACC][64];

  const int n_strips = (p.N + COLS_PER_STRIP - 1) / COLS_PER_STRIP;
  const int S = p.strips_per_wg;
  const int n_groups = (n_strips + S - 1) / S;
  const int G = p.num_blocks * n_groups;
  const int lid = xcd_remap((int)blockIdx.x, G);
  const int b = lid % p.num_blocks;
  const int grp = lid / p.num_blocks;
  const int e = p.block_expert[b];  // block_expert has num_blocks entries, -1 past the end
  if (e < 0 || b * BM >= p.num_padded[0]) return;
  const int s0 = grp * S;
  const int n_str = min(S, n_strips - s0);

  const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
  const int K = p.K, nch = (K + 127) / 128;
  const int n_my = (nch + 3) / 4;  // chunk slots per wave and strip (the same for every wave)
  const int TK = p.T * p.slots_per_token;
  const size_t a_row_bytes = (AF == kABf16) ? (size_t)K * 2 : (AF == kAMxfp4 ? (size_t)K / 2 : (size_t)K);
  const int nbn = (p.Nw + 127) / 128, nbk = nch;

  // Output column of this lane for tile t of strip s (stage 1 interleaved rows: the
  // columns of a tile are cb + 8 t + li / 2, gate in even lanes, up in odd ones), and
  // the first weight row of the lane's tile (0 for tiles past the edge).
  auto tile_col = [&](int s, int t) {
    const int cb = (s0 + s) * COLS_PER_STRIP;
    if (STAGE == 1 && (EPI && p.interleaved)) return cb + 8 * t + (li >> 1);
    return (STAGE == 1) ? cb + (t % (NT / 2)) * 16 + li : cb + t * 16 + li;
  };
  auto tile_ok = [&](int s, int t) {  // wave-uniform
    const int cb = (s0 + s) * COLS_PER_STRIP;
    if (STAGE == 1 && (EPI && p.interleaved)) return 2 * cb + 16 * t < p.Nw;
    return tile_col(s, t) - li < p.N;
  };
  auto tile_row = [&](int s, int t) {
    if (!tile_ok(s, t)) return 0;
    const int cb = (s0 + s) * COLS_PER_STRIP;
    if (STAGE == 1 && (EPI && p.interleaved)) return 2 * cb + 16 * t;
    const int c = tile_col(s, t) - li;
    return (STAGE == 1 && t >= NT / 2) ? p.N + c : c;
  };

  // A row of this lane in each m-tile, and the A rows of its 4 output rows
  const uint8_t* a_src[MT];
  bool a_ok[MT];
  int a_idx[MT];
  int o_idx[MT][4];
  bool o_ok[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    int arow = b * BM + m * 16 + li;
    bool ok = true;
    if (STAGE == 1) {
      const int slot = p.sorted_slots[arow];
      ok = slot < TK;
      arow = ok ? slot / p.slots_per_token : 0;
    }
    a_src[m] = (const uint8_t*)p.a + (size_t)arow * a_row_bytes;
    a_ok[m] = ok;
    a_idx[m] = arow;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      int orow = b * BM + m * 16 + 4 * g + rr;
      bool ook = true;
      if (STAGE == 1) {
        const int slot = p.sorted_slots[orow];
        ook = slot < TK;
        orow = ook ? slot / p.slots_per_token : 0;
      }
      o_idx[m][rr] = orow;
      o_ok[m][rr] = ook;
    }
  }

  // Loads stream item i = (strip i / n_my, chunk slot i % n_my); past the end the
  // last item is re-read with zero data.  Invalid elements read the zero page.
  const int n_items = n_str * n_my;
  auto load = [&](int i, WeightRegs<WF, NT>& wr, ARegs<AF, MT>& ar) {
    const bool in = i < n_items;
    const int ii = in ? i : n_items - 1;
    const int s = ii / n_my, c = w + 4 * (ii % n_my);
    const bool live = in && c < nch;
    const bool kok = live && (c * 128 + 32 * g < K);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int trow = tile_row(s, t);
      const uint8_t* wd = WLay::data(p, e, trow, li, g, lane, K);
      if constexpr (WF == kWMxfp4) {
        wr.w[t][0] = ld16(wd, (size_t)c * WLay::kDataStride, kok);
        wr.s[t] = ld8(WLay::scale(p, e, trow, li, g, lane, K), (size_t)c * WLay::kScaleStride, kok);
      } else {
        wr.w[t][0] = ld16(wd, (size_t)c * WLay::kDataStride, kok);
        wr.w[t][WF == kWMxfp4 ? 0 : 1] = ld16(wd, (size_t)c * WLay::kDataStride + WLay::kHiOff, kok);
        if constexpr (WF == kWFp8Block)
          wr.sb[t] = ldf((const float*)p.w_scale, ((size_t)e * nbn + trow / 128) * nbk + c, live);
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const bool ok = kok && a_ok[m];
      const size_t off = (size_t)c * (NA == 4 ? 256 : (NA == 1 ? 64 : 128)) + g * (NA * 16);
#pragma unroll
      for (int q = 0; q < NA; ++q) ar.a[m][q] = ld16(a_src[m], off + 16 * q, ok);
      if constexpr (AF == kAMxfp4)
        ar.sa[m] = ld8((const uint8_t*)p.a_scale, (size_t)a_idx[m] * (K / 32) + c * 4 + g, ok);
      if constexpr (AF == kAFp8G128) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          ar.as[m][rr] = ldf((const float*)p.a_scale, (size_t)o_idx[m][rr] * nch + c, live && o_ok[m][rr]);
      }
    }
  };

  f32x4 acc[MT][NT];
  auto clear = [&]() {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  auto compute = [&](const WeightRegs<WF, NT>& wr, const ARegs<AF, MT>& ar) {
    if constexpr (AF == kABf16) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float sc = e8m0_to_f32(wr.s[t]);
          const uint32_t dw = (uint32_t)wr.w[t][0][st];
          const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 0);
          const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 1);
          const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 2);
          const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 3);
          const bf16x8 bfr = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
          for (int m = 0; m < MT; ++m)
            acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ar.a[m][st]), bfr,
                                                                 acc[m][t], 0, 0, 0);
        }
      }
    } else if constexpr (AF == kAMxfp4) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const i32x8 a8 = {ar.a[m][0][0], ar.a[m][0][1], ar.a[m][0][2], ar.a[m][0][3], 0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const i32x8 b8 = {wr.w[t][0][0], wr.w[t][0][1], wr.w[t][0][2], wr.w[t][0][3], 0, 0, 0, 0};
          acc[m][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[m][t], 4, 4, 0, (int)ar.sa[m], 0,
                                                                        (int)wr.s[t]);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const i32x4 lo = ar.a[m][0], hi = ar.a[m][NA - 1];
        const i32x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const i32x4 wl = wr.w[t][0], wh = wr.w[t][WF == kWMxfp4 ? 0 : 1];
          const i32x8 b8 = {wl[0], wl[1], wl[2], wl[3], wh[0], wh[1], wh[2], wh[3]};
          if constexpr (WF == kWFp8Block) {
            const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a8, b8, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[m][t][rr] += part[rr] * (ar.as[m][rr] * wr.sb[t]);
          } else {
            acc[m][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[m][t], 0, 0, 0, 127, 0, 127);
          }
        }
      }
    }
  };

  // End of strip s: partial sums of waves 1..3 go through LDS (buffer s & 1), wave 0
  // adds them in wave order and writes the strip's outputs; accumulators restart.
  auto finish_strip = [&](int s) {
    const int buf = s & 1;
    if (w > 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) red[buf][w - 1][(m * NT + t) * 4 + rr][lane] = acc[m][t][rr];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int i = (m * NT + t) * 4 + rr;
            acc[m][t][rr] = ((acc[m][t][rr] + red[buf][0][i][lane]) + red[buf][1][i][lane]) + red[buf][2][i][lane];
          }
      if constexpr (STAGE == 1) {
        if ((EPI && p.interleaved)) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (!tile_ok(s, t)) continue;
            const int col = tile_col(s, t), wr = tile_row(s, t) + li;
            const float ws = (WF == kWFp8Channel) ? ((const float*)p.w_scale)[wsc_index(p, e, wr)] : 1.0f;
            const float bs = (EPI && p.bias) ? bias_of(p, e, wr) : 0.0f;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const int row = m * 16 + 4 * g + rr;
                float v = acc[m][t][rr];
                if constexpr (WF == kWFp8Channel)
                  v = v * (o_ok[m][rr] ? ((const float*)p.a_scale)[(size_t)o_idx[m][rr] * p.asc_rs] : 0.0f) * ws;
                if (EPI && p.weight_on_input) v *= fc1_weight(p, p.sorted_slots[b * BM + row]);
                v += bs;
                const float up = __shfl_xor(v, 1, kWave);
                const bool pad = EPI && p.bias && !o_ok[m][rr];  // pad rows: h = 0
                if (!(li & 1)) p.h[(size_t)(b * BM + row) * p.N + col] = pad ? 0 : (uint16_t)f32_to_bf16(glu<EPI>(p, v, up));
              }
          }
        } else {
#pragma unroll
          for (int t = 0; t < NT / 2; ++t) {
            const int col = tile_col(s, t);
            if (col >= p.N) continue;
            const int tu = t + NT / 2;
            const float wg = (WF == kWFp8Channel) ? ((const float*)p.w_scale)[wsc_index(p, e, col)] : 1.0f;
            const float wu = (WF == kWFp8Channel) ? ((const float*)p.w_scale)[wsc_index(p, e, p.N + col)] : 1.0f;
            const float bg = (EPI && p.bias) ? bias_of(p, e, col) : 0.0f, bu = (EPI && p.bias) ? bias_of(p, e, p.N + col) : 0.0f;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const int row = m * 16 + 4 * g + rr;
                float gv = acc[m][t][rr], uv = acc[m][tu][rr];
                if constexpr (WF == kWFp8Channel) {
                  const float as = o_ok[m][rr] ? ((const float*)p.a_scale)[(size_t)o_idx[m][rr] * p.asc_rs] : 0.0f;
                  gv = gv * as * wg;
                  uv = uv * as * wu;
                }
                if (EPI && p.weight_on_input) {
                  const float fw = fc1_weight(p, p.sorted_slots[b * BM + row]);
                  gv *= fw;
                  uv *= fw;
                }
                gv += bg;
                uv += bu;
                const bool pad = EPI && p.bias && !o_ok[m][rr];  // pad rows: h = 0
                p.h[(size_t)(b * BM + row) * p.N + col] = pad ? 0 : (uint16_t)f32_to_bf16(glu<EPI>(p, gv, uv));
              }
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int row = m * 16 + 4 * g + rr;
            const int slot = p.sorted_slots[b * BM + row];
            if (slot >= TK) continue;
            const float as = (WF == kWFp8Channel) ? ((const float*)p.a_scale)[(size_t)(b * BM + row) * p.asc_rs] : 1.0f;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const int col = tile_col(s, t);
              if (col >= p.N) continue;
              float v = acc[m][t][rr];
              if constexpr (WF == kWFp8Channel) v = v * as * ((const float*)p.w_scale)[wsc_index(p, e, col)];
              if (EPI && p.bias) v += bias_of(p, e, col);
              p.ybuf[(size_t)slot * p.N + col] = v;
            }
          }
      }
    }
    clear();
  };

  clear();
  WeightRegs<WF, NT> w0, w1;
  ARegs<AF, MT> a0, a1;
  if (n_str == 1) {
    // One strip (the usual case for one to a few tokens): the same stream with the strip's
    // epilogue after the loop.  With the epilogue inside the loop, as below, the compiler
    // drains every load in flight where the epilogue's branch rejoins the stream.
    load(0, w0, a0);
    for (int i = 0; i < n_items; i += 2) {
      __builtin_amdgcn_sched_barrier(0);
      load(i + 1, w1, a1);
      __builtin_amdgcn_sched_barrier(0);
      compute(w0, a0);
      __builtin_amdgcn_sched_barrier(0);
      load(i + 2, w0, a0);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < n_items) compute(w1, a1);
    }
    finish_strip(0);
    return;
  }
  // Several strips: one item in flight ahead of the MFMAs.  Each half-iteration issues the
  // next item's loads, then computes the previous one; sched_barrier keeps the scheduler
  // from sinking a prefetch below the MFMAs that follow it.
  load(0, w0, a0);
  for (int i = 0; i < n_items; i += 2) {
    __builtin_amdgcn_sched_barrier(0);
    load(i + 1, w1, a1);
    __builtin_amdgcn_sched_barrier(0);
    compute(w0, a0);
    if ((i + 1) % n_my == 0) finish_strip(i / n_my);
    __builtin_amdgcn_sched_barrier(0);
    load(i + 2, w0, a0);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 < n_items) {
      compute(w1, a1);
      if ((i + 2) % n_my == 0) finish_strip((i + 1) / n_my);
    }
  }
}

template <int AF>
constexpr int a_bytes_x2() { return AF == kABf16 ? 4 : (AF == kAMxfp4 ? 1 : 2); }  // 2 x bytes per element

// 16-byte units of one activation row per 128-K chunk.
__host__ __device__ constexpr int a_units_per_chunk(int afmt) {
  return afmt == kABf16 ? 16 : (afmt == kAMxfp4 ? 4 : 8);
}

// LDS bytes of a 16-row activation tile (rows padded to whole 128-K chunks), its row
// tables (row, slot, top-k weight) and its scales, rounded to 256 (direct loads of
// the fp32 scales write whole 64-lane dword runs).
__host__ __device__ inline size_t tile16_lds_bytes(int afmt, int K) {
  const int nch = (K + 127) / 128;
  const size_t tile = (size_t)16 * nch * a_units_per_chunk(afmt) * 16;
  size_t sc = 0;
  if (afmt == kAFp8G128) sc = 16 * (size_t)nch * 4;
  if (afmt == kAMxfp4) sc = 16 * (size_t)nch * 4;
  if (afmt == kAFp8Token) sc = 16 * 4;
  return (tile + 192 + sc + 255) / 256 * 256;
}

// ---------------------------------------------------------------------------------
// Persistent 16-row kernel (the decode shape, activation tile in LDS).  The grid is
// one resident workgroup per slot of the chip.  The work of a launch is the list of
// (block, column unit) pairs, a unit being two 16-column weight tiles (gate and up of
// 16 output columns in stage 1, 32 adjacent output columns in stage 2), and each
// workgroup takes an equal contiguous range of that list.  Inside the range, one phase
// per block: the block's activation tile is staged in LDS once, and the phase's
// (unit, 128-K chunk) steps are split into equal contiguous runs, one per wave.  A wave
// streams its run through a D-deep register ring without a break at unit boundaries
// and writes each unit it covers whole; a unit shared by consecutive waves is summed
// by the wave that holds its first chunk, adding the later waves' partials from LDS in
// wave order (a fixed order, so results do not depend on timing).  Compared with one
// workgroup per column strip, the HBM stream of a CU never drains between strips, and
// the load is balanced to within one unit per workgroup.
//
// Phase start, in issue order: the row table (sorted slots) -> the activation tile by
// direct global -> LDS loads -> the first D weight steps of the ring.  Loads complete
// in issue order, so one wait for "at most D steps' loads outstanding" means the tile
// has landed while the weights keep streaming; the MFMAs start as soon as the first
// ring step arrives.  (A plain __syncthreads here would wait for the whole ring.)  The
// tile is XOR-swizzled: 16-byte unit u of row r sits at unit u ^ (r mod units per
// chunk), so the fragment reads of the 16 rows spread over the LDS banks although each
// direct load writes 1 KB contiguously.
//
// RS = 1 (stage 1 only): the router and the align-sort run inside the kernel.  Every
// workgroup routes and sorts the whole batch in LDS (route_sort_block, its scratch
// overlapping the tile region) before its first phase, keeps the sorted rows, block
// owners and padded total in an LDS region of their own, and takes its tables from
// there; workgroup 0 also writes ids, weights, counts, offsets and the tables to global
// memory for stage 2 and the combine.  The tables are the same integers the separate
// router + sort kernels produce, so the result does not change.
template <int STAGE, int WF, int AF, int D, int WAVES, int WL, int EPI, int RS>
__global__ __launch_bounds__(64 * WAVES) void moe_gemm_persist_kernel(const GemmParams p) {
  using WLay = WLayout<WF, WL>;
  constexpr int BM = 16, NT = 2;
  constexpr int SEG = a_units_per_chunk(AF);
  // vector-memory instructions of one ring step (load_next): per tile, the 16 B code
  // piece(s) and the E8M0 byte (MXFP4) or the fp32 block / channel scale (FP8), or the
  // four 16 B pieces of 32 bf16 values (bf16 weights)
  constexpr int kStepLoads = NT * (WF == kWMxfp4 ? 2 : (WF == kWBf16 ? 4 : 3));
  static_assert(WF != kWBf16 || (AF == kABf16 && WL == 0), "bf16 weights: bf16 activations, canonical layout");
  constexpr int kRingLoads = D * kStepLoads;
  static_assert(kRingLoads <= 63, "vmcnt range");
  constexpr int kThreads = 64 * WAVES;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = (int)threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps run bookkeeping scalar
  const int K = p.K, nch = (K + 127) / 128;
  const int U = (STAGE == 1) ? (p.N + 15) / 16 : (p.N + 31) / 32;  // units per block
  int npad;
  int32_t *rs_sorted = nullptr, *rs_owner = nullptr;  // RS: the tables in LDS
  if constexpr (RS) {
    static_assert(STAGE == 1 && 64 * WAVES == kSortThreads, "the fused route + sort runs in stage 1 with 1024 threads");
    rs_sorted = (int32_t*)(smem + p.route_keep_off);
    rs_owner = rs_sorted + p.route_cap;
    int32_t* rs_total = rs_owner + p.route_cap / BM;
    const bool first = blockIdx.x == 0;
    const RouteSortOut o{first ? p.out_ids : nullptr, first ? p.out_weights : nullptr,
                         first ? p.out_counts : nullptr, first ? p.out_offsets : nullptr, rs_sorted, rs_owner, rs_total};
    route_sort_block(p.logits, p.T, p.route_E, p.route_topk, p.route_score, p.route_renorm, p.route_n_shared,
                     p.route_shared_w, BM, p.route_cap, smem, o);
    lds_barrier();
    npad = *rs_total;
    if (first) {
      for (int i = (int)threadIdx.x; i < p.route_cap; i += kThreads) p.out_sorted[i] = rs_sorted[i];
      for (int i = (int)threadIdx.x; i < p.route_cap / BM; i += kThreads) p.out_block_expert[i] = rs_owner[i];
      if (threadIdx.x == 0) p.out_num_padded[0] = npad;
    }
  } else {
    npad = p.num_padded[0];
  }
  const int nb = min(npad / BM, p.num_blocks);  // blocks in use
  const long L = (long)nb * U;
  const int P = (int)gridDim.x;
  const int wg = xcd_remap((int)blockIdx.x, P);  // neighbouring ranges (same block) share an XCD
  long u_next = L * wg / P;
  const long r_end = L * (wg + 1) / P;

  const int TK = p.T * p.slots_per_token;
  const int row_bytes = K * a_bytes_x2<AF>() / 2;
  const int upr = nch * SEG;   // 16-byte units per tile row
  const int n_dma = upr / 4;   // 64-lane direct loads per tile (16 rows x upr units)
  const int ngp = nch * 4;
  uint8_t* lds_a = smem;
  int* lds_row = (int*)(smem + (size_t)16 * upr * 16);  // activation row of each tile row (-1: pad)
  int* lds_slot = lds_row + 16;                          // sorted slot of each tile row
  float* lds_fw = (float*)(lds_slot + 16);               // router weight of each tile row (weight on input)
  uint8_t* lds_sc = (uint8_t*)(lds_slot + 32);
  // biases of the phase's units, bf16, [unit - ua][tile][16 columns]: staged in the
  // prologue so that no bias load is waited for in the stream (a load issued at a unit's
  // end would wait for every ring load in flight)
  uint16_t* lds_bias = (uint16_t*)(smem + p.bias_lds_off);
  float* lds_part = (float*)(smem + tile16_lds_bytes(AF, K));  // [WAVES][NT*4][64]
  const MOE_GLOBAL uint8_t* zp = (const MOE_GLOBAL uint8_t*)kZeroPage;

  const size_t nbn = (size_t)(p.Nw + 127) / 128;

  while (u_next < r_end) {
    const int b = (int)(u_next / U);
    const int ua = (int)(u_next - (long)b * U);
    const int ub = (int)min((long)U, r_end - (long)b * U);
    u_next = (long)b * U + ub;
    const int e = RS ? rs_owner[b] : p.block_expert[b];
    if (e < 0) continue;  // workgroup-uniform

    const int S = (ub - ua) * nch;  // steps of the phase
    const int s0 = (int)((long)S * wv / WAVES), s1 = (int)((long)S * (wv + 1) / WAVES);
    const int n = s1 - s0;          // this wave's steps (may be 0)

    // weight tile t of unit u (relative to ua): first weight row, and whether it exists.
    // Stage 1 separated rows: gate tile 16 u and up tile N + 16 u; interleaved rows: the
    // consecutive tiles 32 u and 32 u + 16 (gate and up of columns 16 u .. 16 u + 15 in
    // alternate lanes).
    auto trow_of = [&](int u, int t) {
      if (STAGE == 1) return (EPI && p.interleaved) ? 32 * (ua + u) + 16 * t : (t == 0 ? 16 * (ua + u) : p.N + 16 * (ua + u));
      return 32 * (ua + u) + 16 * t;
    };
    auto tok_of = [&](int u, int t) { return STAGE == 1 ? true : 32 * (ua + u) + 16 * t < p.N; };

    // load cursor (unit, chunk) of the next step to fetch
    int lu = s0 / nch, lc = s0 % nch, lj = 0;
    auto load_next = [&](WeightRegs<WF, NT>& r) {
      const bool live = lj < n;
      const bool kok = live && (lc * 128 + 32 * g < K);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bool tok = live && tok_of(lu, t);
        const bool ok = kok && tok;
        const int trow = tok ? trow_of(lu, t) : 0;  // the K-tail check is per lane; the block scale is not
        const uint8_t* src = WLay::data(p, e, trow, li, g, lane, K);
        r.w[t][0] = ld16(src, (size_t)lc * WLay::kDataStride, ok);
        if constexpr (WF == kWBf16) {
#pragma unroll
          for (int q = 1; q < 4; ++q) r.w[t][q] = ld16(src, (size_t)lc * WLay::kDataStride + 16 * q, ok);
        } else if constexpr (WF == kWMxfp4) {
          r.s[t] = ld8(WLay::scale(p, e, trow, li, g, lane, K), (size_t)lc * WLay::kScaleStride, ok);
        } else {
          r.w[t][1] = ld16(src, (size_t)lc * WLay::kDataStride + WLay::kHiOff, ok);
          if constexpr (WF == kWFp8Block)
            r.sb[t] = ldf((const float*)p.w_scale, ((size_t)e * nbn + trow / 128) * nch + lc, tok);
          else  // channel scale of the lane's output column, carried with the step
            r.sb[t] = ldf((const float*)p.w_scale, wsc_index(p, e, trow + li), tok);
        }
      }
      if (live) {
        ++lj;
        if (++lc == nch) { lc = 0; ++lu; }
      }
    };

    // ---- row table; every wave is done with the previous phase's LDS ----
    lds_barrier();
    int slot_v = 0;
    if (tid < BM) {
      slot_v = RS ? rs_sorted[b * BM + tid] : p.sorted_slots[b * BM + tid];
      if (STAGE == 1) lds_row[tid] = slot_v < TK ? slot_v / p.slots_per_token : -1;
    }
    if (STAGE == 1) lds_barrier();
    float fw_v = 0.0f;  // weight on input: the row's router weight (0 for pad rows), staged with the slot
    if (EPI && STAGE == 1 && p.weight_on_input && tid < BM)
      fw_v = ldf(p.topk_weights, (size_t)(slot_v < TK ? slot_v : 0), slot_v < TK);
    // bias slice: direct global -> LDS loads of bias pairs, issued with the tile below

    // activation scales (quantised formats) go through registers, issued before the tile
    constexpr int kScPer = (AF == kAMxfp4) ? 8 : 1;  // per thread: 16 x 4 x nch bytes <= 8 x kThreads
    float sc_f = 0.0f;
    uint32_t sc_b[kScPer];
    if constexpr (AF == kAFp8G128) {
      if (tid < BM * nch) {
        const int r = tid / nch, c = tid % nch;
        const int arow = STAGE == 1 ? lds_row[r] : b * BM + r;
        sc_f = ldf((const float*)p.a_scale, (size_t)(arow < 0 ? 0 : arow) * nch + c, arow >= 0);
      }
    } else if constexpr (AF == kAMxfp4) {
      const int ng = K / 32;
#pragma unroll
      for (int i = 0; i < kScPer; ++i) {
        const int q = tid + kThreads * i;
        sc_b[i] = 0;
        if (q < BM * ngp) {
          const int r = q / ngp, c = q % ngp;
          const int arow = STAGE == 1 ? lds_row[r] : b * BM + r;
          sc_b[i] = ld8((const uint8_t*)p.a_scale, (size_t)(arow < 0 ? 0 : arow) * ng + c, arow >= 0 && c < ng);
        }
      }
    } else if constexpr (AF == kAFp8Token) {
      if (tid < BM) {
        const int arow = STAGE == 1 ? lds_row[tid] : b * BM + tid;
        sc_f = ldf((const float*)p.a_scale, (size_t)(arow < 0 ? 0 : arow) * p.asc_rs, arow >= 0);
      }
    }

    // ---- bias slice and activation tile -> LDS (direct loads), then the ring ----
    if constexpr (EPI) {
      // lane l of direct load i moves the bias pair of slice entries 2 (64 i + l), +1: unit
      // u, tile t, columns c, c + 1 (c even, so the pair is 4-byte aligned and never
      // crosses a 16-column tile); past the phase, or past N in stage 2, the zero page
      const int ndw = p.bias ? (ub - ua) * 16 : 0;
      for (int i = wv; i * 64 < ndw; i += WAVES) {
        const int d = i * 64 + lane, q = 2 * d;
        const int col = trow_of(q >> 5, (q >> 4) & 1) + (q & 15);
        const bool ok = d < ndw && (STAGE == 1 || col < p.N);
        const MOE_GLOBAL uint8_t* src =
            ok ? (const MOE_GLOBAL uint8_t*)p.bias + ((size_t)e * p.Nw + col) * 2 : zp;
        dma4((const void*)src, (uint8_t*)lds_bias + (size_t)i * 256);
      }
    }
    for (int i = wv; i < n_dma; i += WAVES) {
      const int v = i * 64 + lane;
      const int r = v / upr, pv = v - r * upr;
      const int pu = pv ^ (r & (SEG - 1));  // the unit stored at position pv of row r
      const int arow = STAGE == 1 ? lds_row[r] : b * BM + r;
      const bool ok = arow >= 0 && 16 * pu < row_bytes;
      const MOE_GLOBAL uint8_t* src =
          ok ? (const MOE_GLOBAL uint8_t*)p.a + (size_t)arow * row_bytes + 16 * pu : zp;
      dma16((const void*)src, lds_a + (size_t)i * 1024);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    WeightRegs<WF, NT> ring[D];
#pragma unroll
    for (int d = 0; d < D; ++d) load_next(ring[d]);
    __builtin_amdgcn_sched_barrier(0);
    // at most the ring's loads outstanding: this wave's tile loads and scales have landed
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kRingLoads));
    if (tid < BM) {
      lds_slot[tid] = slot_v;
      if (EPI && STAGE == 1) lds_fw[tid] = fw_v;
    }

    if constexpr (AF == kAFp8G128) {
      if (tid < BM * nch) ((float*)lds_sc)[tid] = sc_f;
    } else if constexpr (AF == kAMxfp4) {
#pragma unroll
      for (int i = 0; i < kScPer; ++i)
        if (tid + kThreads * i < BM * ngp) lds_sc[tid + kThreads * i] = (uint8_t)sc_b[i];
    } else if constexpr (AF == kAFp8Token) {
      if (tid < BM) ((float*)lds_sc)[tid] = sc_f;
    }
    lds_barrier();

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float csc[NT] = {1.0f, 1.0f};  // FP8 channel: the current unit's column scales

    const int swz = li & (SEG - 1);
    auto compute = [&](int c, const WeightRegs<WF, NT>& wr) {
      const uint8_t* arow = lds_a + (size_t)li * upr * 16 + (size_t)c * SEG * 16;
      if constexpr (AF == kABf16) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16x8 af = *(const bf16x8*)(arow + 16 * ((4 * g + st) ^ swz));
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            bf16x8 bfr;
            if constexpr (WF == kWBf16) {  // unquantised: the loaded bf16 values as they are
              bfr = __builtin_bit_cast(bf16x8, wr.w[t][st]);
            } else {
              const float sc = e8m0_to_f32(wr.s[t]);
              const uint32_t dw = (uint32_t)wr.w[t][0][st];
              const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 0);
              const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 1);
              const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 2);
              const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 3);
              bfr = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
            }
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, acc[t], 0, 0, 0);
          }
        }
      } else if constexpr (AF == kAMxfp4) {
        const i32x4 a4 = *(const i32x4*)(arow + 16 * (g ^ swz));
        const i32x8 a8 = {a4[0], a4[1], a4[2], a4[3], 0, 0, 0, 0};
        const int sa = (int)lds_sc[li * ngp + 4 * c + g];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const i32x8 b8 = {wr.w[t][0][0], wr.w[t][0][1], wr.w[t][0][2], wr.w[t][0][3], 0, 0, 0, 0};
          acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[t], 4, 4, 0, sa, 0, (int)wr.s[t]);
        }
      } else {
        const i32x4 lo = *(const i32x4*)(arow + 16 * ((2 * g) ^ swz));
        const i32x4 hi = *(const i32x4*)(arow + 16 * ((2 * g + 1) ^ swz));
        const i32x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        float asr[4];
        if constexpr (WF == kWFp8Block) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) asr[rr] = ((const float*)lds_sc)[(4 * g + rr) * nch + c];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const i32x4 wl = wr.w[t][0], wh = wr.w[t][WF == kWMxfp4 ? 0 : 1];
          const i32x8 b8 = {wl[0], wl[1], wl[2], wl[3], wh[0], wh[1], wh[2], wh[3]};
          if constexpr (WF == kWFp8Block) {
            const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                                                0, 0, 127, 0, 127);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[t][rr] += part[rr] * (asr[rr] * wr.sb[t]);
          } else {
            acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[t], 0, 0, 0, 127, 0, 127);
          }
        }
      }
    };

    // Writes unit u's outputs from a complete sum.
    auto emit = [&](int u) {
      if constexpr (STAGE == 1) {
        // (bias loads and their uses stay inside `if (EPI && p.bias)`: a load whose wait could be
        // hoisted here would drain the weight ring of the no-bias path)
        if ((EPI && p.interleaved)) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int col = 16 * (ua + u) + 8 * t + (li >> 1);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int row = 4 * g + rr;
              float v = acc[t][rr];
              if constexpr (WF == kWFp8Channel) v = v * ((const float*)lds_sc)[row] * csc[t];
              if (EPI && p.weight_on_input) v *= lds_fw[row];
              if (EPI && p.bias) v += __uint_as_float((uint32_t)lds_bias[u * 32 + t * 16 + li] << 16);
              const float up = __shfl_xor(v, 1, kWave);  // odd lane: the up row of the same column
              const bool pad = EPI && p.bias && lds_row[row] < 0;  // pad rows: h = 0
              if (!(li & 1)) p.h[(size_t)(b * BM + row) * p.N + col] = pad ? 0 : (uint16_t)f32_to_bf16(glu<EPI>(p, v, up));
            }
          }
        } else {
          const int col = 16 * (ua + u) + li;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int row = 4 * g + rr;
            float gv = acc[0][rr], uv = acc[1][rr];
            if constexpr (WF == kWFp8Channel) {
              const float as = ((const float*)lds_sc)[row];
              gv = gv * as * csc[0];
              uv = uv * as * csc[1];
            }
            if (EPI && p.weight_on_input) {
              const float fw = lds_fw[row];
              gv *= fw;
              uv *= fw;
            }
            if (EPI && p.bias) {
              gv += __uint_as_float((uint32_t)lds_bias[u * 32 + li] << 16);
              uv += __uint_as_float((uint32_t)lds_bias[u * 32 + 16 + li] << 16);
            }
            const bool pad = EPI && p.bias && lds_row[row] < 0;  // pad rows: h = 0
            p.h[(size_t)(b * BM + row) * p.N + col] = pad ? 0 : (uint16_t)f32_to_bf16(glu<EPI>(p, gv, uv));
          }
        }
      } else {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = 4 * g + rr;
          const int slot = lds_slot[row];
          if (slot >= TK) continue;
          const float as = (WF == kWFp8Channel) ? ((const float*)lds_sc)[row] : 1.0f;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int col = 32 * (ua + u) + 16 * t + li;
            if (col >= p.N) continue;
            float v = acc[t][rr];
            if constexpr (WF == kWFp8Channel) v = v * as * csc[t];
            if (EPI && p.bias) v += __uint_as_float((uint32_t)lds_bias[u * 32 + t * 16 + li] << 16);
            p.ybuf[(size_t)slot * p.N + col] = v;
          }
        }
      }
    };

    // compute cursor; a run that starts inside a unit hands that unit's sum to LDS,
    // a run that ends inside a unit it started keeps the sum for the reduction below
    int cu = s0 / nch, cc = s0 % nch;
    const int head_unit = (s0 % nch != 0) ? cu : -1;
    bool tail_open = false;
    for (int j0 = 0; j0 < n; j0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int j = j0 + d;
        __builtin_amdgcn_sched_barrier(0);
        compute(cc, ring[d]);  // past the run the weights are zero: adds exact zeros
        if constexpr (WF == kWFp8Channel) {
          if (j < n) {
#pragma unroll
            for (int t = 0; t < NT; ++t) csc[t] = ring[d].sb[t];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_next(ring[d]);
        if (j < n) {
          const bool unit_end = cc == nch - 1;
          if (unit_end || j == n - 1) {
            if (cu == head_unit) {
              float* dst = lds_part + (size_t)wv * NT * 4 * 64;
#pragma unroll
              for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) dst[(t * 4 + rr) * 64 + lane] = acc[t][rr];
            } else if (unit_end) {
              emit(cu);
            } else {
              tail_open = true;
            }
            if (!tail_open) {
#pragma unroll
              for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
          if (j + 1 < n) {
            if (++cc == nch) { cc = 0; ++cu; }
          }
        }
      }
    }
    lds_barrier();  // partials of shared units are in LDS
    if (tail_open) {
      const int u_end = (cu + 1) * nch;  // first step past the open unit
      for (int q = wv + 1; q < WAVES; ++q) {
        const int q0 = (int)((long)S * q / WAVES), q1 = (int)((long)S * (q + 1) / WAVES);
        if (q0 >= u_end) break;
        if (q1 > q0) {
          const float* src = lds_part + (size_t)q * NT * 4 * 64;
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[t][rr] += src[(t * 4 + rr) * 64 + lane];
        }
      }
      emit(cu);
    }
  }
}

// out[t, :] = bf16( sum_{j ascending} w[t, j] * ybuf[t*K + j, :] ), slots with invalid
// ids skipped; w = 1 when wts is NULL (router weight applied on the input).  Each product is rounded to fp32 before it is added (no fused
// multiply-add), the same arithmetic as weighting each row first and summing after.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ybuf, const int32_t* __restrict__ ids,
                                                      const float* __restrict__ wts, int T, int K, int H, int E,
                                                      uint16_t* __restrict__ out) {
#pragma clang fp contract(off)
  const int per_row = H / 4;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)T * per_row) return;
  const int t = (int)(idx / per_row), c = (int)(idx % per_row) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // four slots at a time: their ids and weights, then their rows, are loaded together
  // (indices clamped to the token's last slot; a row of a skipped slot is read, not used)
  constexpr int kGroup = 4;
  for (int j0 = 0; j0 < K; j0 += kGroup) {
    int e[kGroup];
    float w[kGroup];
    f32x4 y[kGroup];
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      const int j = min(j0 + q, K - 1);
      e[q] = ids[(size_t)t * K + j];
      w[q] = wts ? wts[(size_t)t * K + j] : 1.0f;
    }
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      const int j = min(j0 + q, K - 1);
      y[q] = *(const f32x4*)(ybuf + ((size_t)t * K + j) * H + c);
    }
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      if (j0 + q >= K || e[q] < 0 || e[q] >= E) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float prod = y[q][i] * w[q];
        acc[i] = acc[i] + prod;
      }
    }
  }
  const uint32_t lo = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
  const uint32_t hi = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
  *(uint2*)(out + (size_t)t * H + c) = make_uint2(lo, hi);
}

// Dynamic LDS of the persistent kernel: up to kPersistLdsMax it serves 16-row blocks
// (larger activation tiles go to the K-split kernel); with the route + sort fused in it
// may take up to a CU's whole LDS, kPersistLdsFusedMax.
constexpr size_t kPersistLdsMax = 128 * 1024;
constexpr size_t kPersistLdsFusedMax = 160 * 1024;
#ifndef MOE_PERSIST_WAVES
#define MOE_PERSIST_WAVES 16
#endif
#ifndef MOE_PERSIST_WAVES_S2  // waves of a stage-2 persistent workgroup: each wave gets twice the
#define MOE_PERSIST_WAVES_S2 8  // ring steps; measured 1-4% faster on stage 2 than 16 (decode shapes)
#endif
#ifndef MOE_PERSIST_DEPTH_BF16  // bf16 weights: 128 B per lane and step already; depth 1 measured
#define MOE_PERSIST_DEPTH_BF16 1   // best on the decode shape (2 -5%, 3 -18%, 4 -37%)
#endif
#ifndef MOE_PERSIST_DEPTH_F4
#define MOE_PERSIST_DEPTH_F4 6
#endif
#ifndef MOE_PERSIST_DEPTH_F4A4  // MXFP4 weights with MXFP4 activations: the A operand needs more registers
#define MOE_PERSIST_DEPTH_F4A4 4
#endif
#ifndef MOE_PERSIST_DEPTH_F8
#define MOE_PERSIST_DEPTH_F8 2
#endif
#ifndef MOE_PERSIST_DEPTH_F8B
#define MOE_PERSIST_DEPTH_F8B 2
#endif

// Per-device caches below: atomics, since host threads may launch on several devices at once
// (two threads filling one entry store the same value).
static int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// LDS bytes of the persistent kernel: activation tile + one partial-sum slot per wave.
static size_t persist_lds_bytes(int afmt, int K, int waves) {
  return tile16_lds_bytes(afmt, K) + (size_t)waves * 2 * 4 * 64 * 4;
}

// Dynamic LDS a persistent workgroup may take on the current device: kPersistLdsFusedMax,
// or less where the device's per-workgroup limit is lower.
static size_t persist_lds_limit() {
  static std::atomic<int> lim[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64 * 1024;
  int n = lim[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || n <= 0)
      n = 64 * 1024;
    lim[dev].store(n, std::memory_order_relaxed);
  }
  return std::min((size_t)n, kPersistLdsFusedMax);
}

// Bytes of the persistent kernel's bias slice: one phase covers at most the U units of a
// block, 32 bf16 biases each (stage 1: N = I columns in gate/up pairs; stage 2: N = H),
// written by direct loads of 256 bytes.
static size_t bias_slice_bytes(int stage, int N) {
  const size_t units = stage == 1 ? (size_t)(N + 15) / 16 : (size_t)(N + 31) / 32;
  return (units * 32 * 2 + 255) / 256 * 256;
}

// LDS of the persistent stage-1 kernel with the route + sort fused in: the route
// scratch overlaps the tile, partial-sum and bias region; the kept tables (sorted rows
// [cap], block owners [cap / 16], padded total) follow all of them.  False when the batch
// is too large for the one-workgroup route + sort or the LDS does not fit.
static bool route_stage1_lds(int afmt, int K_dim, int N, bool bias, int T, int E, int topk, int n_shared,
                             size_t* keep_off, size_t* total) {
  if (64 * MOE_PERSIST_WAVES != kSortThreads || !route_sort_fusable(T, E, topk + n_shared)) return false;
  const long cap = (long)T * (topk + n_shared) + (long)(E + n_shared) * 15;
  const size_t base = persist_lds_bytes(afmt, K_dim, MOE_PERSIST_WAVES) + (bias ? bias_slice_bytes(1, N) : 0);
  const size_t scratch = route_sort_lds_bytes(T, E, topk, n_shared, (T + kWave - 1) / kWave);
  const size_t off = (std::max(base, scratch) + 15) / 16 * 16;
  const size_t all = off + (size_t)(cap + cap / 16 + 1) * 4;
  *keep_off = off;
  *total = all;
  return all <= persist_lds_limit();
}

bool persist_launch_fits(int afmt, int stage, int K_dim, int N, bool bias) {
  const size_t tile = persist_lds_bytes(afmt, K_dim, MOE_PERSIST_WAVES);
  return tile <= kPersistLdsMax && tile + (bias ? bias_slice_bytes(stage, N) : 0) <= persist_lds_limit();
}

bool route_stage1_fusable(int afmt, int K_dim, int N, int T, int E, int topk, int n_shared, bool bias) {
  size_t off = 0, all = 0;
  return T > 0 && persist_lds_bytes(afmt, K_dim, MOE_PERSIST_WAVES) <= kPersistLdsMax &&
         route_stage1_lds(afmt, K_dim, N, bias, T, E, topk, n_shared, &off, &all);
}

template <int STAGE, int WF, int AF, int WL, int EPI, int RS>
static hipError_t launch_persist(const GemmParams& p, size_t lds, hipStream_t stream) {
  constexpr int WAVES = (STAGE == 2) ? MOE_PERSIST_WAVES_S2 : MOE_PERSIST_WAVES;
  constexpr int D = (WF == kWMxfp4) ? (AF == kAMxfp4 ? MOE_PERSIST_DEPTH_F4A4 : MOE_PERSIST_DEPTH_F4)
                                    : (WF == kWBf16 ? MOE_PERSIST_DEPTH_BF16
                                                    : (WF == kWFp8Block ? MOE_PERSIST_DEPTH_F8B : MOE_PERSIST_DEPTH_F8));
  if (p.num_blocks == 0) return hipSuccess;
  auto kern = moe_gemm_persist_kernel<STAGE, WF, AF, D, WAVES, WL, EPI, RS>;
  // the dynamic-LDS limit is raised once per kernel and device (setting it twice is harmless)
  static std::atomic<bool> attr_set[64];
  int dev = 0;
  const bool cached = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64;
  if (!cached || !attr_set[dev].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)persist_lds_limit());
    if (e != hipSuccess) return e;
    if (cached) attr_set[dev].store(true, std::memory_order_release);
  }
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, 64 * WAVES, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  // no more workgroups than units of work: (blocks x units) bounds what can be split
  const long units = (long)p.num_blocks * ((STAGE == 1) ? (p.N + 15) / 16 : (p.N + 31) / 32);
  const long grid = std::max(1L, std::min((long)device_cus() * per_cu, units));
  kern<<<(unsigned)grid, 64 * WAVES, lds, stream>>>(p);
  return hipGetLastError();
}

// Small-block launch: strips per workgroup so that the grid is about
// MOE_KSPLIT_WGS_PER_CU workgroups for each of the 256 CUs, at least one strip each.
template <int STAGE, int WF, int AF, int BM, int NT, int WL, int EPI>
static hipError_t launch_ksplit(const GemmParams& p_in, hipStream_t stream) {
  constexpr int COLS_PER_STRIP = (STAGE == 1) ? 8 * NT : 16 * NT;
  GemmParams p = p_in;
  const long n_tiles = (p.N + COLS_PER_STRIP - 1) / COLS_PER_STRIP;
  const long items = (long)p.num_blocks * n_tiles;
  const long target = 256L * MOE_KSPLIT_WGS_PER_CU;
  p.strips_per_wg = (int)std::max(1L, std::min(n_tiles, items / target));
  const long G = (long)p.num_blocks * ((n_tiles + p.strips_per_wg - 1) / p.strips_per_wg);
  if (G == 0) return hipSuccess;
  if (G > 0x7FFFFFFFL) return hipErrorInvalidConfiguration;
  moe_gemm_ksplit_kernel<STAGE, WF, AF, BM, NT, WL, EPI><<<(unsigned)G, 256, 0, stream>>>(p);
  return hipGetLastError();
}

template <int STAGE, int WF, int AF, int BM, int WL, int EPI>
static hipError_t launch_one_impl(const GemmParams& p_in, hipStream_t stream) {
  if constexpr (BM == 16) {
    const size_t tile_lds = persist_lds_bytes(AF, p_in.K, MOE_PERSIST_WAVES);
    const bool bias = EPI && p_in.bias;
    GemmParams p = p_in;
    p.bias_lds_off = (int)tile_lds;  // the bias slice follows the tile and partial sums
    if constexpr (STAGE == 1 && 64 * MOE_PERSIST_WAVES == kSortThreads) {
      if (p_in.route) {
        size_t keep_off = 0, lds = 0;
        if (tile_lds > kPersistLdsMax ||
            !route_stage1_lds(AF, p.K, p.N, bias, p.T, p.route_E, p.route_topk, p.route_n_shared, &keep_off, &lds))
          return hipErrorInvalidValue;
        p.route_keep_off = (int)keep_off;
        return launch_persist<STAGE, WF, AF, WL, EPI, 1>(p, lds, stream);
      }
    }
    // 16-row blocks whose activation tile fits run here (larger tiles: the K-split kernel)
    const size_t lds = tile_lds + (bias ? bias_slice_bytes(STAGE, p_in.N) : 0);
    if (tile_lds <= kPersistLdsMax && lds <= persist_lds_limit())
      return launch_persist<STAGE, WF, AF, WL, EPI, 0>(p, lds, stream);
  }
  if (p_in.route) return hipErrorInvalidValue;  // the fused route + sort runs in the persistent kernel only
  if constexpr (BM == 128 && WL == 1 && WF != kWBf16 && MOE_LDS_GEMM != 0)
    return launch_gemm_lds(STAGE, WF, AF, EPI, p_in, stream);  // both operands staged in LDS
  constexpr bool kSplit = BM <= 32;  // small blocks: K split over waves, no LDS staging
  if constexpr (WF == kWBf16 && kSplit) {
    return hipErrorInvalidValue;  // bf16 weights: the persistent kernel or 64/128-row blocks only
  } else {
  // (bf16 weights: two tiles per wave, their 64 B per lane and chunk fill the registers)
  constexpr int NT = kSplit ? (AF == kABf16 ? MOE_KSPLIT_NT_BF16 : MOE_KSPLIT_NT_Q)
                            : (WF == kWBf16 ? 2
                                            : (BM != 64 ? 4
                                                        : (AF == kAMxfp4 ? MOE_NT_F4A4
                                                                         : (AF == kABf16 && STAGE == 2 ? MOE_NT_W4A16_S2 : 4))));
  if constexpr (kSplit) {
    // (one or two tokens leave CUs idle here, e.g. 128 workgroups for stage 2 of a 4096-wide
    // layer; strips of 2 or 1 tiles per wave that fill the chip measured 1-3% slower)
    return launch_ksplit<STAGE, WF, AF, BM, NT, WL, EPI>(p_in, stream);
  } else {
  constexpr int COLS_PER_WG = (STAGE == 1) ? 32 * NT : 64 * NT;
  const long G = (long)p_in.num_blocks * ((p_in.N + COLS_PER_WG - 1) / COLS_PER_WG);
  if (G == 0) return hipSuccess;
  if (G > 0x7FFFFFFFL) return hipErrorInvalidConfiguration;
  moe_gemm_kernel<STAGE, WF, AF, BM, NT, WL, EPI><<<(unsigned)G, 256, 0, stream>>>(p_in);
  return hipGetLastError();
  }
  }
}

template <int STAGE, int WF, int AF, int BM, int WL, int EPI>
static hipError_t launch_one(const GemmParams& p_in, hipStream_t stream) {
  // bf16 weights: canonical layout; 16-row blocks on the persistent kernel (activation
  // tile in LDS) or 64/128-row blocks (the ABI enforces all three)
  if constexpr (WF == kWBf16 && (BM == 32 || WL != 0)) {
    return hipErrorInvalidValue;
  } else {
    return launch_one_impl<STAGE, WF, AF, BM, WL, EPI>(p_in, stream);
  }
}

template <int STAGE, int WF, int AF, int WL, int EPI>
static hipError_t launch_bm_wl(int bm, const GemmParams& p, hipStream_t stream) {
  switch (bm) {
    case 16: return launch_one<STAGE, WF, AF, 16, WL, EPI>(p, stream);
    case 32: return launch_one<STAGE, WF, AF, 32, WL, EPI>(p, stream);
    case 64: return launch_one<STAGE, WF, AF, 64, WL, EPI>(p, stream);
    case 128: return launch_one<STAGE, WF, AF, 128, WL, EPI>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int STAGE, int WF, int AF>
static hipError_t launch_bm(int bm, const GemmParams& p, hipStream_t stream) {
  const bool general = p.bias || (STAGE == 1 && (p.act != kActSilu || p.interleaved || p.weight_on_input));
  if (general)
    return p.weight_layout ? launch_bm_wl<STAGE, WF, AF, 1, 1>(bm, p, stream)
                           : launch_bm_wl<STAGE, WF, AF, 0, 1>(bm, p, stream);
  return p.weight_layout ? launch_bm_wl<STAGE, WF, AF, 1, 0>(bm, p, stream)
                         : launch_bm_wl<STAGE, WF, AF, 0, 0>(bm, p, stream);
}

template <int STAGE>
static hipError_t launch_stage(int wfmt, int afmt, int bm, const GemmParams& p, hipStream_t stream) {
  if (wfmt == kWMxfp4 && afmt == kABf16) return launch_bm<STAGE, kWMxfp4, kABf16>(bm, p, stream);
  if (wfmt == kWMxfp4 && afmt == kAMxfp4) return launch_bm<STAGE, kWMxfp4, kAMxfp4>(bm, p, stream);
  if (wfmt == kWFp8Block && afmt == kAFp8G128) return launch_bm<STAGE, kWFp8Block, kAFp8G128>(bm, p, stream);
  if (wfmt == kWFp8Channel && afmt == kAFp8Token) return launch_bm<STAGE, kWFp8Channel, kAFp8Token>(bm, p, stream);
  // per tensor: the per-channel kernels with scale strides 0 (GemmParams::wsc_rs, asc_rs)
  if (wfmt == kWFp8Tensor && afmt == kAFp8Tensor) return launch_bm<STAGE, kWFp8Channel, kAFp8Token>(bm, p, stream);
  if (wfmt == kWBf16 && afmt == kABf16) return launch_bm<STAGE, kWBf16, kABf16>(bm, p, stream);
  return hipErrorInvalidValue;
}

// One-time permutation into the tiled weight layout (see moe_tile_weights).  One
// wavefront per block: lane l = 16g + r copies row r's 16 B (MXFP4) or 2 x 16 B (FP8)
// of K elements [128c + 32g, +32) and, for MXFP4, the E8M0 byte of that 32-group.
template <int WF>
__global__ __launch_bounds__(256) void tile_weights_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
                                                           uint8_t* __restrict__ out, long n_blocks, int N, int K) {
  const long blk = (long)blockIdx.x * 4 + threadIdx.x / 64;
  if (blk >= n_blocks) return;
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  const int nch = (K + 127) / 128;
  const int c = (int)(blk % nch);
  const long tile = blk / nch;                       // e * (N/16) + n16
  const long row = tile * 16 + r;                    // e * N + n
  const bool ok = c * 128 + 32 * g < K;
  if constexpr (WF == kWMxfp4) {
    uint8_t* o = out + blk * 1088;
    *(i32x4*)(o + 16 * lane) = ld16(w, row * (size_t)(K / 2) + 64 * c + 16 * g, ok);
    o[1024 + lane] = (uint8_t)ld8(ws, row * (size_t)(K / 32) + 4 * c + g, ok);
  } else {
    uint8_t* o = out + blk * 2048;
    *(i32x4*)(o + 16 * lane) = ld16(w, row * (size_t)K + 128 * c + 32 * g, ok);
    *(i32x4*)(o + 1024 + 16 * lane) = ld16(w, row * (size_t)K + 128 * c + 32 * g + 16, ok);
  }
}

hipError_t launch_tile_weights(int wfmt, int E, int N, int K, const uint8_t* w, const void* ws, uint8_t* out,
                               hipStream_t stream) {
  const long n_blocks = (long)E * (N / 16) * ((K + 127) / 128);
  if (n_blocks == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n_blocks + 3) / 4);
  if (wfmt == kWMxfp4)
    tile_weights_kernel<kWMxfp4><<<grid, 256, 0, stream>>>(w, (const uint8_t*)ws, out, n_blocks, N, K);
  else
    tile_weights_kernel<kWFp8Block><<<grid, 256, 0, stream>>>(w, nullptr, out, n_blocks, N, K);
  return hipGetLastError();
}

hipError_t launch_gemm(int stage, int wfmt, int afmt, int block_m, const GemmParams& p, hipStream_t stream) {
  return stage == 1 ? launch_stage<1>(wfmt, afmt, block_m, p, stream) : launch_stage<2>(wfmt, afmt, block_m, p, stream);
}

hipError_t launch_combine(const float* ybuf, const int32_t* topk_ids, const float* topk_weights, int T, int K,
                          int H, int E_total, uint16_t* out, hipStream_t stream) {
  const long n = (long)T * (H / 4);
  if (n == 0) return hipSuccess;
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(ybuf, topk_ids, topk_weights, T, K, H, E_total,
                                                                   out);
  return hipGetLastError();
}

}  // namespace moe
