// Device helpers of the grouped-GEMM kernels (gfx950, wave64): predicated global loads,
// direct global -> LDS loads, the weight layouts and the gated activation.
#pragma once
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_remap(int L, int G) {
  const int per = G / kXcds, rem = G % kXcds;
  const int x = L % kXcds, i = L / kXcds;
  return x * per + (x < rem ? x : rem) + i;
}

// Branch-free predicated loads: when the predicate is false the load reads this
// all-zero array instead, so the compiler emits straight-line loads and never has to
// wait for a load before the value is consumed (a guarded load becomes an exec-masked
// branch that waits for every load in flight; a select on the loaded value waits for
// that load).  Zero data contributes nothing to any MFMA product; a zero E8M0 scale
// byte is the finite 2^-127.
// Both candidate addresses are global memory; saying so keeps the loads global_load
// (a generic pointer would make them flat loads, which the compiler must wait for
// conservatively).  Nothing ever writes kZeroPage.
static __device__ __attribute__((aligned(64))) uint8_t kZeroPage[64];

#define MOE_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ T ld_global(const void* base, size_t off_bytes, bool ok) {
  const MOE_GLOBAL uint8_t* zp = (const MOE_GLOBAL uint8_t*)kZeroPage;
  const MOE_GLOBAL uint8_t* b = (const MOE_GLOBAL uint8_t*)base;
  return *(const MOE_GLOBAL T*)(ok ? b + off_bytes : zp);
}
__device__ __forceinline__ i32x4 ld16(const uint8_t* base, size_t off, bool ok) {
  return ld_global<i32x4>(base, off, ok);
}
__device__ __forceinline__ uint32_t ld8(const uint8_t* base, size_t off, bool ok) {
  return ld_global<uint8_t>(base, off, ok);
}
__device__ __forceinline__ float ldf(const float* base, size_t off, bool ok) {
  return ld_global<float>(base, off * sizeof(float), ok);
}
// s_waitcnt immediate for "at most n vector-memory operations outstanding" (gfx9
// encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt at their maxima, i.e.
// not waited for).
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return ((n > 63 ? 63 : n) & 0xF) | (((n > 63 ? 63 : n) >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}


// Direct global -> LDS load of 16 bytes per lane: the wave's 64 x 16 bytes land
// contiguously at dst (wave-uniform).  Counted by vmcnt like any other load.
__device__ __forceinline__ void dma16(const void* src, uint8_t* dst) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_global_load_lds((const MOE_GLOBAL void*)src, (lds_void*)dst, 16, 0, 0);
}
// The same with 4 bytes per lane: 256 contiguous bytes at dst.
__device__ __forceinline__ void dma4(const void* src, uint8_t* dst) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_global_load_lds((const MOE_GLOBAL void*)src, (lds_void*)dst, 4, 0, 0);
}

// A read-only fp32 at a wave-uniform address through the scalar data cache (a load from
// the constant address space; the cache is invalidated at each dispatch and nothing in the
// kernel writes the data).
__device__ __forceinline__ float ld_uniform_f32(const float* ptr) {
  return *(const __attribute__((address_space(4))) float*)ptr;
}

constexpr int kScaleGroups = 2;  // scale dwords of WeightRegs: up to 8 tiles
template <int WF, int NT>
struct WeightRegs {
  i32x4 w[NT][WF == kWMxfp4 ? 1 : (WF == kWBf16 ? 4 : 2)];  // 16 B (MXFP4), 32 B (FP8), 64 B (bf16) per tile
  uint32_t s[NT];                      // MXFP4: E8M0 byte
  uint32_t s4[kScaleGroups];           // tiled MXFP4 (64/128-row kernel): 4 scale bytes per dword, see kScaleDword
  float sb[NT];                        // FP8 block: w_scale of this chunk
};

// Where a lane's weight bytes live.  WL = 0: canonical row-major [E][Nw][K*] codes and
// [E][Nw][K/32] E8M0 scales; WL = 1: the tiled layout of moe_tile_weights, blocks of 16
// rows x 128 K in MFMA lane order, [E][Nw/16][nch] blocks, MXFP4 scales inside the block.
// `trow` is the first row of the lane's 16-row tile (tiles never straddle 16-row
// boundaries: Nw, I and H are multiples of 16), li the lane's row inside it.
template <int WF, int WL>
struct WLayout {
  static constexpr size_t kBlock = (WF == kWMxfp4) ? 1088 : 2048;
  static constexpr size_t kDataStride = WL ? kBlock : ((WF == kWMxfp4) ? 64 : (WF == kWBf16 ? 256 : 128));  // per 128-K chunk
  static constexpr size_t kScaleStride = WL ? kBlock : 4;
  static constexpr size_t kHiOff = WL ? 1024 : 16;  // FP8: second 16 B piece of the lane
  __device__ static const uint8_t* data(const GemmParams& p, int e, int trow, int li, int g, int lane, int K) {
    if constexpr (WL) {
      const size_t blk = ((size_t)e * p.Nw + trow) / 16 * (size_t)((K + 127) / 128);
      return p.w + blk * kBlock + 16 * lane;
    } else {
      // bytes per row and per lane's 32 K elements: MXFP4 K/2 and 16, FP8 K and 32, bf16 2K and 64
      const size_t rowb = (WF == kWMxfp4) ? (size_t)K / 2 : (WF == kWBf16 ? (size_t)K * 2 : (size_t)K);
      return p.w + ((size_t)e * p.Nw + trow + li) * rowb + (WF == kWMxfp4 ? 16 * g : (WF == kWBf16 ? 64 * g : 32 * g));
    }
  }
  __device__ static const uint8_t* scale(const GemmParams& p, int e, int trow, int li, int g, int lane, int K) {
    if constexpr (WL) {
      const size_t blk = ((size_t)e * p.Nw + trow) / 16 * (size_t)((K + 127) / 128);
      return p.w + blk * kBlock + 1024 + lane;
    } else {
      return (const uint8_t*)p.w_scale + ((size_t)e * p.Nw + trow + li) * (size_t)(K / 32) + g;
    }
  }
};

// EPI (all GEMM kernels): 0 = SiLU-and-mul, separated gate/up rows, no bias, compiled
// without the branches of the general epilogue (its registers and code size matter on
// the hot path); 1 = activation, row order and biases as GemmParams says.
template <int EPI>
__device__ __forceinline__ float glu(const GemmParams& p, float g, float u) {
  // SiLU as g * rcp(1 + e^-g): the hardware reciprocal (within an ulp) in place of the
  // correctly rounded division; h is rounded to bf16 next, so this moves h by at most one
  // bf16 ulp in the rare values that sit on a rounding boundary (g -> -inf: rcp(inf) = 0)
  if constexpr (EPI == 0) return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
  else return glu_act(p, g, u);
}

}  // namespace moe
