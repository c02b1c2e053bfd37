// Grouped expert GEMM for 128-row blocks with both operands staged in LDS (gfx950).
//
// The 64-row kernel (experts_gemm.hip) loads each wave's weights straight into registers,
// so every weight byte that passes the vector-memory return path feeds 64 rows, and on
// large batches that path, not HBM or the MFMA pipes, sets the pace.  Here a workgroup of
// eight waves covers 128 rows (two row groups of 64) and 16 weight tiles of 16 rows (four
// column groups of four tiles): per 128-K chunk the activation tile (128 rows) and the
// workgroup's weight tiles land in LDS by direct global -> LDS loads, and every weight
// byte is read from LDS by both row groups, every activation byte by all four column
// groups.  Bytes through the return path per flop fall by 1.6x (FP8) to 2x (FP4).
//
// The weights must be in the tiled layout (moe_tile_weights): a 16-row x 128-K block of
// one chunk is 1 KB (MXFP4 codes; + 64 E8M0 bytes) or 2 x 1 KB (FP8) in MFMA lane order,
// so one 64-lane direct load moves it unchanged and the MFMA operand read from LDS is
// lane-contiguous.  The activation tile is unpadded and XOR-swizzled in 16-byte units
// (unit u of row r at position u ^ ((r / rows-per-256-B) mod units-per-row)), so the 16
// rows of a fragment read fall in different bank groups.
//
// Pipeline: a ring of S chunk buffers.  At chunk c a wave waits until its own loads of
// chunk c have landed (a counted vmcnt: the loads of the later chunks stay in flight),
// then one barrier makes every wave's loads of chunk c visible and frees the buffer of
// chunk c - 1, into which the loads of chunk c + S - 1 are issued before the MFMAs of
// chunk c.  The compiler does not order direct LDS loads against LDS reads, so these
// waits and barriers are the only ordering.
//
// MFMA per format as in the 64-row kernel: w4a16 dequantises the E2M1 codes to bf16 with
// v_cvt_scalef32_pk_bf16_fp4 and runs v_mfma_f32_16x16x32_bf16; w4a4 and FP8 run
// v_mfma_scale_f32_16x16x128_f8f6f4 (E8M0 operand scales, or unit scales with the FP8
// block / channel scales applied to the chunk's partial product or in the epilogue).
// Epilogues: stage 1 h = bf16(act(gate, up)) in sorted-row order; stage 2 the unweighted
// fp32 row of each routed slot (pages: "rocm_aiter_moe", AiterExperts, rocm_aiter_fused_experts).
#include "gemm_common.h"

#include <algorithm>
#include <atomic>

namespace moe {

namespace {

constexpr int kBM = 128;     // rows per block
constexpr int kNT = 4;       // 16-column weight tiles per wave

#ifndef MOE_LDS_WN      // column groups per workgroup (waves = 2 x column groups)
#define MOE_LDS_WN 4
#endif
#ifndef MOE_LDS_STAGES  // chunk buffers in the ring
#define MOE_LDS_STAGES 3
#endif

template <int AF, int kWaves>
struct ATile {
  static constexpr int ARB = AF == kABf16 ? 256 : (AF == kAMxfp4 ? 64 : 128);  // bytes per row and chunk
  static constexpr int APC = ARB / 16;                                           // 16-byte units per row
  static constexpr int EPP = 128 / APC;                                          // elements per unit
  static constexpr int RPB = 256 / ARB;                                          // rows per 256 bytes
  static constexpr int kBytes = kBM * ARB;
  static constexpr int kDma = kBytes / 1024;          // 64-lane x 16-byte direct loads per chunk
  static constexpr int kDmaPerWave = kDma / kWaves;
  // per-chunk activation scales in LDS: fp32 per row (FP8 128-groups) or 4 E8M0 bytes per row
  static constexpr int kScaleBytes = (AF == kAFp8G128 || AF == kAMxfp4) ? kBM * 4 : 0;
  __device__ static int swz(int r) { return (r / RPB) & (APC - 1); }
};

template <int WF, int kTiles>
struct BTile {
  static constexpr int kBlock = WF == kWMxfp4 ? 1088 : 2048;
  // MXFP4: the tiles' codes, then their 64-byte scale parts in one 1 KB run
  static constexpr int kBytes = WF == kWMxfp4 ? kTiles * 1024 + 1024 : kTiles * kBlock;
};

template <int WF, int AF, int WN, int S>
struct LdsStage {
  static constexpr int kA = 0;
  static constexpr int kAs = ATile<AF, 2 * WN>::kBytes;
  static constexpr int kB = kAs + ATile<AF, 2 * WN>::kScaleBytes;
  static constexpr int kBytes = kB + BTile<WF, 4 * WN>::kBytes;
  // after the ring: the per-row FP8 token scales (loaded once)
  static constexpr int kRing = S * kBytes;
  static constexpr int kTotal = kRing + (AF == kAFp8Token ? kBM * 4 : 0);
};

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 15]
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(vmcnt_imm(7)); break;
    case 8: __builtin_amdgcn_s_waitcnt(vmcnt_imm(8)); break;
    case 9: __builtin_amdgcn_s_waitcnt(vmcnt_imm(9)); break;
    case 10: __builtin_amdgcn_s_waitcnt(vmcnt_imm(10)); break;
    case 11: __builtin_amdgcn_s_waitcnt(vmcnt_imm(11)); break;
    case 12: __builtin_amdgcn_s_waitcnt(vmcnt_imm(12)); break;
    case 13: __builtin_amdgcn_s_waitcnt(vmcnt_imm(13)); break;
    case 14: __builtin_amdgcn_s_waitcnt(vmcnt_imm(14)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(15)); break;
  }
}

}  // namespace

template <int STAGE, int WF, int AF, int EPI, int WN, int kStages>
__global__ __launch_bounds__(128 * WN, 1) void moe_gemm_lds_kernel(const GemmParams p) {
  constexpr int kWaves = 2 * WN, kTiles = 4 * WN;  // 2 row groups x WN column groups; 4 tiles per column group
  using AT = ATile<AF, kWaves>;
  using BT = BTile<WF, kTiles>;
  using LS = LdsStage<WF, AF, WN, kStages>;
  constexpr int COLS_PER_WG = (STAGE == 1) ? 8 * kNT * WN : 16 * kNT * WN;  // gate/up pairs, or output columns
  constexpr int ARB = AT::ARB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int n_tiles = (p.N + COLS_PER_WG - 1) / COLS_PER_WG;
  const int G = p.num_blocks * n_tiles;
  const int lid = xcd_remap((int)blockIdx.x, G);
  const int b = lid % p.num_blocks;  // blocks fastest: one expert's blocks share its weight strip in L2
  const int nt_idx = lid / p.num_blocks;
  const int npad = p.num_padded[0];
  if (b * kBM >= npad) return;
  const int e = p.block_expert[b];
  if (e < 0) return;

  const int tid = (int)threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 1, wn = w >> 1;  // row group (64 rows), column group (4 tiles)
  static_assert(kTiles == 2 * kWaves, "each wave moves two weight tiles");
  const int K = p.K, nch = (K + 127) / 128;
  const int TK = p.T * p.slots_per_token;
  const size_t a_row_bytes = (AF == kABf16) ? (size_t)K * 2 : (AF == kAMxfp4 ? (size_t)K / 2 : (size_t)K);
  const MOE_GLOBAL uint8_t* zp = (const MOE_GLOBAL uint8_t*)kZeroPage;

  // ---- weight tiles: tile j = 4 wn + t of the workgroup -> its first weight row ----
  // stage 1, separated rows: tiles t < 2 are gate rows cb + 16 t, tiles t >= 2 the matching
  // up rows N + cb + 16 (t - 2), cb = the column group's first output column; interleaved
  // rows: tiles 2 cb + 16 t (gate and up of columns cb + 8 t + li / 2 in alternate lanes)
  auto tile_row = [&](int j, bool& ok) -> int {
    const int jn = j >> 2, t = j & 3;
    if (STAGE == 1) {
      const int cb = nt_idx * COLS_PER_WG + jn * 32;
      if (EPI && p.interleaved) {
        const int r = 2 * cb + 16 * t;
        ok = r < p.Nw;
        return ok ? r : 0;
      }
      const int c = cb + (t & 1) * 16;
      ok = c < p.N;
      return ok ? (t < 2 ? c : p.N + c) : 0;
    }
    const int c = nt_idx * COLS_PER_WG + jn * 64 + 16 * t;
    ok = c < p.N;
    return ok ? c : 0;
  };
  // this wave loads tiles 2w, 2w + 1 (all of their bytes)
  const uint8_t* b_src[2];
  bool b_ok[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    bool ok;
    const int trow = tile_row(2 * w + q, ok);
    b_ok[q] = ok;
    b_src[q] = p.w + ((size_t)e * p.Nw + trow) / 16 * (size_t)nch * BT::kBlock;
  }
  // MXFP4: wave 0 moves the tiles' 64-byte scale parts with one 16-byte-per-lane load
  // (lane l: tile l / 4, bytes [16 (l % 4), +16); lanes past the last tile read zeros)
  const uint8_t* bs_src = nullptr;
  bool bs_ok = false;
  if constexpr (WF == kWMxfp4) {
    bool ok;
    const int trow = tile_row((lane >> 2) < kTiles ? lane >> 2 : 0, ok);
    bs_ok = ok && (lane >> 2) < kTiles;
    bs_src = p.w + ((size_t)e * p.Nw + trow) / 16 * (size_t)nch * BT::kBlock + 1024 + 16 * (lane & 3);
  }

  // ---- activation rows this wave moves: unit v = (w * kDmaPerWave + i) * 64 + lane ----
  constexpr int NAD = AT::kDmaPerWave;
  const uint8_t* a_src[NAD];
  bool a_ok[NAD];
  int a_k0[NAD];
#pragma unroll
  for (int i = 0; i < NAD; ++i) {
    const int v = (w * NAD + i) * 64 + lane;
    const int r = v / AT::APC, pv = v % AT::APC;
    int arow = b * kBM + r;
    bool ok = true;
    if (STAGE == 1) {
      const int slot = p.sorted_slots[b * kBM + r];
      ok = slot < TK;
      arow = ok ? slot / p.slots_per_token : 0;
    }
    const int pu = pv ^ AT::swz(r);
    a_src[i] = (const uint8_t*)p.a + (size_t)arow * a_row_bytes + pu * 16;
    a_ok[i] = ok;
    a_k0[i] = pu * AT::EPP;
  }
  // ---- activation scale row of thread tid < 128 (quantised formats) ----
  int s_row = 0;
  bool s_ok = false;
  if (tid < kBM) {
    if (STAGE == 1) {
      const int slot = p.sorted_slots[b * kBM + tid];
      s_ok = slot < TK;
      s_row = s_ok ? slot / p.slots_per_token : 0;
    } else {
      s_row = b * kBM + tid;
      s_ok = true;
    }
  }
  if constexpr (AF == kAFp8Token) {
    if (tid < kBM)
      ((float*)(smem + LS::kRing))[tid] = s_ok ? ((const float*)p.a_scale)[(size_t)s_row * p.asc_rs] : 0.0f;
  }

  // direct loads a wave issues per chunk (the counted waits below): its activation units,
  // its two weight tiles, and for waves 0 and 1 the FP8 128-group scales of 64 rows, for
  // wave 0 the MXFP4 weight scales
  const int ops = NAD + 2 * (WF == kWMxfp4 ? 1 : 2) + (AF == kAFp8G128 && w < 2 ? 1 : 0) +
                  (WF == kWMxfp4 && w == 0 ? 1 : 0);
  // MXFP4 activations: the E8M0 bytes of chunk c + 1 are loaded into registers at chunk c,
  // before chunk c + 2's direct loads, so the wait for chunk c + 1 covers them (three buffers)
  static_assert(AF != kAMxfp4 || kStages <= 3, "the activation scale bytes run one chunk ahead");

  // Issues the direct loads of chunk c into ring buffer c % kStages (chunks past the end
  // read the zero page, so every chunk costs the same operations).
  auto issue = [&](int c) {
    uint8_t* st = smem + (c % kStages) * LS::kBytes;
    const bool live = c < nch;
#pragma unroll
    for (int i = 0; i < NAD; ++i) {
      const bool ok = live && a_ok[i] && (c * 128 + a_k0[i] < K);
      const MOE_GLOBAL uint8_t* src = ok ? (const MOE_GLOBAL uint8_t*)a_src[i] + (size_t)c * ARB : zp;
      dma16((const void*)src, st + LS::kA + (size_t)(w * NAD + i) * 1024);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const bool ok = live && b_ok[q];
      const MOE_GLOBAL uint8_t* src =
          ok ? (const MOE_GLOBAL uint8_t*)b_src[q] + (size_t)c * BT::kBlock + 16 * lane : zp;
      // FP8: tile j's 2 KB at 2048 j; MXFP4: its 1 KB of codes at 1024 j (scales after all 16)
      uint8_t* dst = st + LS::kB + (size_t)(2 * w + q) * (WF == kWMxfp4 ? 1024 : 2048);
      dma16((const void*)src, dst);
      if constexpr (WF != kWMxfp4) {
        const MOE_GLOBAL uint8_t* src2 =
            ok ? (const MOE_GLOBAL uint8_t*)b_src[q] + (size_t)c * BT::kBlock + 1024 + 16 * lane : zp;
        dma16((const void*)src2, dst + 1024);
      }
    }
    if constexpr (WF == kWMxfp4) {
      if (w == 0) {
        const bool ok = live && bs_ok;
        const MOE_GLOBAL uint8_t* src = ok ? (const MOE_GLOBAL uint8_t*)bs_src + (size_t)c * BT::kBlock : zp;
        dma16((const void*)src, st + LS::kB + kTiles * 1024);  // scale parts packed after the tiles' codes
      }
    }
    if constexpr (AF == kAFp8G128) {
      if (w < 2) {  // row tid = 64 w + lane: its fp32 scale lands at kAs + 4 tid
        const bool ok = live && s_ok;
        const MOE_GLOBAL uint8_t* src =
            ok ? (const MOE_GLOBAL uint8_t*)((const float*)p.a_scale + (size_t)s_row * nch + c) : zp;
        dma4((const void*)src, st + LS::kAs + (size_t)w * 256);
      }
    }
  };
  // MXFP4 activations: the four E8M0 bytes of row tid for chunk c (zero past K), loaded into
  // registers one chunk ahead and stored to the chunk's buffer before its barrier; the bytes
  // stay apart until then (combining them would wait for the loads at once)
  uint32_t as4[4] = {0, 0, 0, 0};
  auto load_as4 = [&](int c) {
    if constexpr (AF == kAMxfp4) {
      if (w < 2) {
        const uint8_t* sp = (const uint8_t*)p.a_scale + (size_t)s_row * (K / 32) + (c < nch ? c : 0) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) as4[q] = ld8(sp, q, s_ok && c < nch && c * 128 + 32 * q < K);
      }
    }
  };

  // weight scale of an FP8 128x128 block: tile j's 128-row block, chunk c (scalar load)
  const float* wsb_src[kNT];
  float wsc[kNT];
  int col[kNT], wrow[kNT];
  bool col_ok[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    bool ok;
    const int trow = tile_row(4 * wn + t, ok);
    col_ok[t] = ok;
    if (STAGE == 1) {
      const int cb = nt_idx * COLS_PER_WG + wn * 32;
      col[t] = (EPI && p.interleaved) ? cb + 8 * t + (li >> 1) : cb + (t & 1) * 16 + li;
    } else {
      col[t] = nt_idx * COLS_PER_WG + wn * 64 + 16 * t + li;
    }
    wrow[t] = trow + li;
    wsb_src[t] = (WF == kWFp8Block) ? (const float*)p.w_scale + ((size_t)e * ((p.Nw + 127) / 128) + trow / 128) * nch
                                    : nullptr;
    wsc[t] = (WF == kWFp8Channel && ok) ? ((const float*)p.w_scale)[wsc_index(p, e, trow + li)] : 1.0f;
  }

  f32x4 acc[4][kNT];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // MFMAs of chunk c from its ring buffer; sb: the tiles' FP8 block scales of chunk c
  auto compute = [&](int c, const float (&sb)[kNT]) {
    const uint8_t* st = smem + (c % kStages) * LS::kBytes;
    const uint8_t* la = st + LS::kA;
    const uint8_t* lb = st + LS::kB;
    if constexpr (AF == kABf16) {
      uint32_t sc[kNT];
      i32x4 bq[kNT];
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        bq[t] = *(const i32x4*)(lb + (size_t)(4 * wn + t) * 1024 + 16 * lane);
        sc[t] = lb[kTiles * 1024 + (4 * wn + t) * 64 + lane];
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 af[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int R = 64 * wm + 16 * m + li;
          af[m] = *(const bf16x8*)(la + R * ARB + 16 * ((4 * g + s) ^ AT::swz(R)));
        }
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
          const float scl = e8m0_to_f32(sc[t]);
          const uint32_t dw = (uint32_t)bq[t][s];
          const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scl, 0);
          const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scl, 1);
          const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scl, 2);
          const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scl, 3);
          const bf16x8 bfr = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bfr, acc[m][t], 0, 0, 0);
        }
      }
    } else if constexpr (AF == kAMxfp4) {
      i32x8 b8[kNT];
      int sb8[kNT];
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const i32x4 v = *(const i32x4*)(lb + (size_t)(4 * wn + t) * 1024 + 16 * lane);
        b8[t] = i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        sb8[t] = (int)lb[kTiles * 1024 + (4 * wn + t) * 64 + lane];
      }
      const uint32_t* las = (const uint32_t*)(st + LS::kAs);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int R = 64 * wm + 16 * m + li;
        const i32x4 a4 = *(const i32x4*)(la + R * ARB + 16 * (g ^ AT::swz(R)));
        const i32x8 a8 = {a4[0], a4[1], a4[2], a4[3], 0, 0, 0, 0};
        const int sa = (int)((las[R] >> (8 * g)) & 0xFFu);
#pragma unroll
        for (int t = 0; t < kNT; ++t)
          acc[m][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8[t], acc[m][t], 4, 4, 0, sa, 0, sb8[t]);
      }
    } else {
      i32x8 b8[kNT];
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const uint8_t* tb = lb + (size_t)(4 * wn + t) * 2048 + 16 * lane;
        const i32x4 lo = *(const i32x4*)tb, hi = *(const i32x4*)(tb + 1024);
        b8[t] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int R = 64 * wm + 16 * m + li;
        const i32x4 lo = *(const i32x4*)(la + R * ARB + 16 * ((2 * g) ^ AT::swz(R)));
        const i32x4 hi = *(const i32x4*)(la + R * ARB + 16 * ((2 * g + 1) ^ AT::swz(R)));
        const i32x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (AF == kAFp8G128) {
          // row scale x weight block scale, one product per row and block: a column
          // group's tiles lie in one 128-row weight block, except that stage 1 has one for
          // its gate tiles (t < 2) and one for its up tiles (runs of 32 rows from a
          // multiple of 32 never straddle a block)
          const float* las = (const float*)(st + LS::kAs);
          float sg[4], su[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float asr = las[64 * wm + 16 * m + 4 * g + rr];
            sg[rr] = asr * sb[0];
            su[rr] = STAGE == 1 ? asr * sb[2] : sg[rr];
          }
#pragma unroll
          for (int t = 0; t < kNT; ++t) {
            const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a8, b8[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[m][t][rr] += part[rr] * (t < 2 ? sg[rr] : su[rr]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < kNT; ++t)
            acc[m][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8[t], acc[m][t], 0, 0, 0, 127, 0, 127);
        }
      }
    }
  };

  // ---- main loop ----
  load_as4(0);
  float sb_cur[kNT], sb_nxt[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) sb_cur[t] = (WF == kWFp8Block) ? ld_uniform_f32(wsb_src[t]) : 1.0f;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) issue(s);
  for (int c = 0; c < nch; ++c) {
    // this wave's loads of chunk c (and, for MXFP4 activations, the scale bytes of chunk c
    // loaded at chunk c - 1) have landed; chunks c + 1 .. c + kStages - 2 may stay in flight
    wait_vm(ops * (kStages - 2));
    if constexpr (AF == kAMxfp4) {
      if (w < 2)
        ((uint32_t*)(smem + (c % kStages) * LS::kBytes + LS::kAs))[tid] =
            as4[0] | (as4[1] << 8) | (as4[2] << 16) | (as4[3] << 24);
    }
    lds_barrier();
    load_as4(c + 1);  // issued before chunk c + 2's loads
    issue(c + kStages - 1);
    if constexpr (WF == kWFp8Block) {
#pragma unroll
      for (int t = 0; t < kNT; ++t) sb_nxt[t] = ld_uniform_f32(wsb_src[t] + (c + 1 < nch ? c + 1 : c));
    }
    compute(c, sb_cur);
    if constexpr (WF == kWFp8Block) {
#pragma unroll
      for (int t = 0; t < kNT; ++t) sb_cur[t] = sb_nxt[t];
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the trailing zero-page loads

  // ---- epilogue ----
  const float* lds_as = (const float*)(smem + LS::kRing);  // FP8 token scales
  if constexpr (STAGE == 1) {
    float bsv[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) bsv[t] = (EPI && p.bias && col_ok[t]) ? bias_of(p, e, wrow[t]) : 0.0f;
    // pad rows: h = 0 (with a bias act(bias) must not reach the a2 quantiser)
    bool padr[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        padr[m][rr] = EPI && p.bias && p.sorted_slots[b * kBM + 64 * wm + 16 * m + 4 * g + rr] >= TK;
    if (EPI && p.interleaved) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
          if (!col_ok[t]) continue;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int row = 64 * wm + 16 * m + 4 * g + rr;
            float v = acc[m][t][rr];
            if (WF == kWFp8Channel) v = v * lds_as[row] * wsc[t];
            if (EPI && p.weight_on_input) v *= fc1_weight(p, p.sorted_slots[b * kBM + row]);
            v += bsv[t];
            const float up = __shfl_xor(v, 1, kWave);
            if (!(li & 1))
              p.h[(size_t)(b * kBM + row) * p.N + col[t]] = padr[m][rr] ? 0 : (uint16_t)f32_to_bf16(glu<EPI>(p, v, up));
          }
        }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (!col_ok[t]) continue;
          const int tu = t + 2;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int row = 64 * wm + 16 * m + 4 * g + rr;
            float gv = acc[m][t][rr], uv = acc[m][tu][rr];
            if (WF == kWFp8Channel) {
              const float as = lds_as[row];
              gv = gv * as * wsc[t];
              uv = uv * as * wsc[tu];
            }
            if (EPI && p.weight_on_input) {
              const float fw = fc1_weight(p, p.sorted_slots[b * kBM + row]);
              gv *= fw;
              uv *= fw;
            }
            gv += bsv[t];
            uv += bsv[tu];
            p.h[(size_t)(b * kBM + row) * p.N + col[t]] = padr[m][rr] ? 0 : (uint16_t)f32_to_bf16(glu<EPI>(p, gv, uv));
          }
        }
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = 64 * wm + 16 * m + 4 * g + rr;
        const int slot = p.sorted_slots[b * kBM + row];
        if (slot >= TK) continue;
        const float as = (WF == kWFp8Channel) ? lds_as[row] : 1.0f;
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
          if (!col_ok[t]) continue;
          float v = acc[m][t][rr];
          if (WF == kWFp8Channel) v = v * as * wsc[t];
          if (EPI && p.bias) v += bias_of(p, e, col[t]);
          p.ybuf[(size_t)slot * p.N + col[t]] = v;
        }
      }
  }
}

template <int STAGE, int WF, int AF, int EPI>
static hipError_t launch_lds_impl(const GemmParams& p, hipStream_t stream) {
  constexpr int WN = MOE_LDS_WN, S = MOE_LDS_STAGES;
  using LS = LdsStage<WF, AF, WN, S>;
  constexpr int COLS_PER_WG = (STAGE == 1) ? 8 * kNT * WN : 16 * kNT * WN;
  auto kern = moe_gemm_lds_kernel<STAGE, WF, AF, EPI, WN, S>;
  static std::atomic<bool> attr_set[64];
  int dev = 0;
  const bool cached = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64;
  if (!cached || !attr_set[dev].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LS::kTotal);
    if (e != hipSuccess) return e;
    if (cached) attr_set[dev].store(true, std::memory_order_release);
  }
  const long n_tiles = (p.N + COLS_PER_WG - 1) / COLS_PER_WG;
  const long G = (long)p.num_blocks * n_tiles;
  if (G == 0) return hipSuccess;
  if (G > 0x7FFFFFFFL) return hipErrorInvalidConfiguration;
  kern<<<(unsigned)G, 128 * WN, LS::kTotal, stream>>>(p);
  return hipGetLastError();
}

// 128-row blocks, tiled weights: the LDS-staged kernel (w4a16, w4a4, FP8 block, FP8
// channel / tensor).  EPI as for the other kernels.
hipError_t launch_gemm_lds(int stage, int wfmt, int afmt, int epi, const GemmParams& p, hipStream_t stream) {
#define MOE_LDS_CASE(WF, AF)                                                                         \
  if (wfmt == WF && afmt == AF) {                                                                    \
    if (stage == 1) return epi ? launch_lds_impl<1, WF, AF, 1>(p, stream) : launch_lds_impl<1, WF, AF, 0>(p, stream); \
    return epi ? launch_lds_impl<2, WF, AF, 1>(p, stream) : launch_lds_impl<2, WF, AF, 0>(p, stream);                 \
  }
  MOE_LDS_CASE(kWMxfp4, kABf16)
  MOE_LDS_CASE(kWMxfp4, kAMxfp4)
  MOE_LDS_CASE(kWFp8Block, kAFp8G128)
  MOE_LDS_CASE(kWFp8Channel, kAFp8Token)
#undef MOE_LDS_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
