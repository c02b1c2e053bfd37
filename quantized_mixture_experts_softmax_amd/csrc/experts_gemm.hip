// Grouped expert GEMMs on MFMA for gfx950, and the ordered top-k combine.
//
// Stage 1: per padded block of BM sorted rows of expert e, C = A . w1[e]^T over the
// gate rows and the matching up rows, with h = bf16(silu(gate) * up) in the
// epilogue (pages: "rocm_aiter_moe", AiterExperts -- SiLU, act-and-mul -- and
// rocm_aiter_fused_experts; w13 stacks gate rows over up rows).
// Stage 2: y = A . w2[e]^T, multiplied by the slot's top-k weight and written as
// fp32 to a per-slot row; the combine kernel then sums each token's slots in
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
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_remap(int L, int G) {
  const int per = G / kXcds, rem = G % kXcds;
  const int x = L % kXcds, i = L / kXcds;
  return x * per + (x < rem ? x : rem) + i;
}

template <int WF, int NT>
struct WeightRegs {
  i32x4 w[NT][WF == kWMxfp4 ? 1 : 2];  // 16 B (MXFP4) or 32 B (FP8) per tile
  uint32_t s[NT];                      // MXFP4: E8M0 byte
  float sb[NT];                        // FP8 block: w_scale of this chunk
};

template <int STAGE, int WF, int AF, int BM, int NT>
__global__ __launch_bounds__(256) void moe_gemm_kernel(const GemmParams p) {
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

  const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
  const int K = p.K, nch = (K + 127) / 128;
  const int TK = p.T * p.slots_per_token;
  const size_t a_row_bytes = (AF == kABf16) ? (size_t)K * 2 : (AF == kAMxfp4 ? (size_t)K / 2 : (size_t)K);

  // ---- A rows this thread stages into LDS ----
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
    a_src[it] = (const uint8_t*)p.a + (size_t)arow * a_row_bytes + pc * 16;
    a_ok[it] = ok;
    a_lds[it] = (piece < NPIECE ? r : 0) * LROW + pc * 16;
    a_k0[it] = pc * EPP;
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
  const size_t w_row_bytes = (WF == kWMxfp4) ? (size_t)K / 2 : (size_t)K;
  const int nbn = (p.Nw + 127) / 128, nbk = nch;
  const uint8_t* w_src[NT];
  const uint8_t* ws_src[NT];
  const float* wsb_src[NT];
  float wsc[NT];
  int col[NT];
  bool col_ok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int c, wrow;
    if (STAGE == 1) {
      const int tt = t % (NT / 2);
      c = nt_idx * COLS_PER_WG + w * (NT / 2) * 16 + tt * 16 + li;
      col_ok[t] = c < p.N;
      wrow = col_ok[t] ? (t < NT / 2 ? c : p.N + c) : 0;
    } else {
      c = nt_idx * COLS_PER_WG + w * NT * 16 + t * 16 + li;
      col_ok[t] = c < p.N;
      wrow = col_ok[t] ? c : 0;
    }
    col[t] = c;
    const size_t rowi = (size_t)e * p.Nw + wrow;
    w_src[t] = p.w + rowi * w_row_bytes + (WF == kWMxfp4 ? 16 * g : 32 * g);
    ws_src[t] = (const uint8_t*)p.w_scale + rowi * (size_t)(K / 32) + g;
    wsb_src[t] = (const float*)p.w_scale + ((size_t)e * nbn + wrow / 128) * nbk;
    wsc[t] = (WF == kWFp8Channel) ? ((const float*)p.w_scale)[rowi] : 1.0f;
  }

  auto load_a = [&](int c, i32x4 (&reg)[AIT]) {
#pragma unroll
    for (int it = 0; it < AIT; ++it) {
      const bool ok = a_ok[it] && (c * 128 + a_k0[it] < K);
      reg[it] = ok ? *(const i32x4*)(a_src[it] + (size_t)c * ARB) : i32x4{0, 0, 0, 0};
    }
  };
  auto load_as = [&](int c, float& fs, uint32_t& qs) {
    if constexpr (AF == kAFp8G128) {
      fs = s_ok ? ((const float*)p.a_scale)[(size_t)s_row * nch + c] : 0.0f;
    } else if constexpr (AF == kAMxfp4) {
      const uint8_t* sp = (const uint8_t*)p.a_scale + (size_t)s_row * (K / 32) + c * 4;
      uint32_t v = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (s_ok && c * 128 + 32 * q < K) v |= (uint32_t)sp[q] << (8 * q);
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
      if constexpr (WF == kWMxfp4) {
        r.w[t][0] = kok ? *(const i32x4*)(w_src[t] + (size_t)c * 64) : i32x4{0, 0, 0, 0};
        r.s[t] = kok ? (uint32_t)ws_src[t][c * 4] : 127u;
      } else {
        r.w[t][0] = kok ? *(const i32x4*)(w_src[t] + (size_t)c * 128) : i32x4{0, 0, 0, 0};
        r.w[t][WF == kWMxfp4 ? 0 : 1] = kok ? *(const i32x4*)(w_src[t] + (size_t)c * 128 + 16) : i32x4{0, 0, 0, 0};
        if constexpr (WF == kWFp8Block) r.sb[t] = wsb_src[t][c];
      }
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (AF == kAFp8Token) if (tid < BM) lds_as[0][tid] = s_ok ? ((const float*)p.a_scale)[s_row] : 0.0f;

  i32x4 areg[AIT];
  float fs = 0.f;
  uint32_t qs = 0;
  WeightRegs<WF, NT> wr, wn;
  load_a(0, areg);
  load_as(0, fs, qs);
  load_w(0, wr);
  store_a(0, areg, fs, qs);
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nch;
    if (more) {
      load_a(c + 1, areg);
      load_as(c + 1, fs, qs);
      load_w(c + 1, wn);
    }
    const uint8_t* la = lds_a[buf];
    if constexpr (AF == kABf16) {
      // w4a16: fp4 -> bf16 in registers, 4 K-steps of 8 per chunk
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 af[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) af[m] = *(const bf16x8*)(la + (m * 16 + li) * LROW + 64 * g + 16 * st);
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
            acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bfr, acc[m][t], 0, 0, 0);
        }
      }
    } else if constexpr (AF == kAMxfp4) {
      // w4a4: scaled FP4 MFMA, E8M0 bytes as operand scales
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const i32x4 a4 = *(const i32x4*)(la + (m * 16 + li) * LROW + 16 * g);
        const i32x8 a8 = {a4[0], a4[1], a4[2], a4[3], 0, 0, 0, 0};
        const int sa = (int)((lds_as4[buf][m * 16 + li] >> (8 * g)) & 0xFFu);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const i32x8 b8 = {wr.w[t][0][0], wr.w[t][0][1], wr.w[t][0][2], wr.w[t][0][3], 0, 0, 0, 0};
          acc[m][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[m][t], 4, 4, 0, sa, 0,
                                                                        (int)wr.s[t]);
        }
      }
    } else {
      // FP8 e4m3 x e4m3 at unit operand scale
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const i32x4 lo = *(const i32x4*)(la + (m * 16 + li) * LROW + 32 * g);
        const i32x4 hi = *(const i32x4*)(la + (m * 16 + li) * LROW + 32 * g + 16);
        const i32x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        float asr[4];
        if constexpr (WF == kWFp8Block) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) asr[rr] = lds_as[buf][m * 16 + 4 * g + rr];
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
            for (int rr = 0; rr < 4; ++rr) acc[m][t][rr] += part[rr] * (asr[rr] * wr.sb[t]);
          } else {
            acc[m][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[m][t], 0, 0, 0, 127, 0, 127);
          }
        }
      }
    }
    if (more) {
      store_a(buf ^ 1, areg, fs, qs);
      wr = wn;
    }
    __syncthreads();
  }

  // ---- epilogue ----
  if constexpr (STAGE == 1) {
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
          const float hv = gv / (1.0f + __expf(-gv)) * uv;
          p.h[(size_t)(b * BM + row) * p.N + col[t]] = (uint16_t)f32_to_bf16(hv);
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
        const float tw = p.topk_weights[slot];
        const float as = (WF == kWFp8Channel) ? lds_as[0][row] : 1.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (!col_ok[t]) continue;
          float v = acc[m][t][rr];
          if (WF == kWFp8Channel) v = v * as * wsc[t];
          p.ybuf[(size_t)slot * p.N + col[t]] = v * tw;
        }
      }
  }
}

// out[t, :] = bf16( sum_{j ascending} ybuf[t*K + j, :] ), slots with invalid ids skipped.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ybuf, const int32_t* __restrict__ ids,
                                                      int T, int K, int H, int E, uint16_t* __restrict__ out) {
  const int per_row = H / 4;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)T * per_row) return;
  const int t = (int)(idx / per_row), c = (int)(idx % per_row) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < K; ++j) {
    const int e = ids[(size_t)t * K + j];
    if (e < 0 || e >= E) continue;
    const f32x4 y = *(const f32x4*)(ybuf + ((size_t)t * K + j) * H + c);
    acc += y;
  }
  const uint32_t lo = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
  const uint32_t hi = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
  *(uint2*)(out + (size_t)t * H + c) = make_uint2(lo, hi);
}

template <int STAGE, int WF, int AF, int BM>
static hipError_t launch_one(const GemmParams& p, hipStream_t stream) {
  constexpr int NT = BM <= 32 ? 2 : 4;
  constexpr int COLS_PER_WG = (STAGE == 1) ? 32 * NT : 64 * NT;
  const long n_tiles = (p.N + COLS_PER_WG - 1) / COLS_PER_WG;
  const long G = (long)p.num_blocks * n_tiles;
  if (G == 0) return hipSuccess;
  if (G > 0x7FFFFFFFL) return hipErrorInvalidConfiguration;
  moe_gemm_kernel<STAGE, WF, AF, BM, NT><<<(unsigned)G, 256, 0, stream>>>(p);
  return hipGetLastError();
}

template <int STAGE, int WF, int AF>
static hipError_t launch_bm(int bm, const GemmParams& p, hipStream_t stream) {
  switch (bm) {
    case 16: return launch_one<STAGE, WF, AF, 16>(p, stream);
    case 32: return launch_one<STAGE, WF, AF, 32>(p, stream);
    case 64: return launch_one<STAGE, WF, AF, 64>(p, stream);
    case 128: return launch_one<STAGE, WF, AF, 128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int STAGE>
static hipError_t launch_stage(int wfmt, int afmt, int bm, const GemmParams& p, hipStream_t stream) {
  if (wfmt == kWMxfp4 && afmt == kABf16) return launch_bm<STAGE, kWMxfp4, kABf16>(bm, p, stream);
  if (wfmt == kWMxfp4 && afmt == kAMxfp4) return launch_bm<STAGE, kWMxfp4, kAMxfp4>(bm, p, stream);
  if (wfmt == kWFp8Block && afmt == kAFp8G128) return launch_bm<STAGE, kWFp8Block, kAFp8G128>(bm, p, stream);
  if (wfmt == kWFp8Channel && afmt == kAFp8Token) return launch_bm<STAGE, kWFp8Channel, kAFp8Token>(bm, p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int stage, int wfmt, int afmt, int block_m, const GemmParams& p, hipStream_t stream) {
  return stage == 1 ? launch_stage<1>(wfmt, afmt, block_m, p, stream) : launch_stage<2>(wfmt, afmt, block_m, p, stream);
}

hipError_t launch_combine(const float* ybuf, const int32_t* topk_ids, int T, int K, int H, int E_total,
                          uint16_t* out, hipStream_t stream) {
  const long n = (long)T * (H / 4);
  if (n == 0) return hipSuccess;
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(ybuf, topk_ids, T, K, H, E_total, out);
  return hipGetLastError();
}

}  // namespace moe
