// Dynamic activation quantisation: FP8 e4m3fn per 128-group, per row or per tensor, and MXFP4
// (e2m1 + E8M0) per 32-group (pages: "rocm_aiter_moe", AiterFp8BlockExperts,
// AiterFp8ChannelExperts, AiterMxfp4Experts; packing two FP4 codes per byte as in
// "quark_moe", QuarkOCP_MX_MoEMethod.get_packed_dim).
//
// The encoders take their decisions in IEEE fp32 exactly as documented for
// moe_quant_act: amax is exact, s = amax / 448 and x / s are correctly rounded fp32
// divisions (s by hipcc's division, which stays correctly rounded unless fast-math is
// asked for; x / s by a one-FMA correction of x * (1/s), see div_rn), and the element
// rounding is done in integer-exact steps, so the codes are bit-identical to the oracle's
// given the same bf16 input.
#include "moe_device.h"
#include "moe_internal.h"

#include <algorithm>

namespace moe {

// Eight bf16 values (16 bytes, 16-byte aligned) as fp32; zeros when !ok.
__device__ __forceinline__ void load8_bf16(const uint16_t* p, bool ok, float (&f)[8]) {
  const uint4 v = ok ? *(const uint4*)p : make_uint4(0u, 0u, 0u, 0u);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}
__device__ __forceinline__ float amax8(const float (&f)[8]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  return m;
}
// x / s, correctly rounded, by Markstein's method (P. Markstein, IBM J. Res. Dev. 34(1),
// 1990): with r = RN(1/s), q = RN(x r) lies within an ulp of x / s, the remainder
// x - s q is exact in one FMA, and RN(q + (x - s q) r) is the correctly rounded quotient
// unless the remainder underflows.  For bf16 x with |x| <= 448 s and s >= 2^-80 (smaller
// scales take the plain division) an exhaustive host check over every such pair finds the
// result equal to the correctly rounded division wherever the quotient is at least 2^-11;
// smaller quotients, where underflow can cost the last bit, all encode to a zero code.
// (The result takes the sign of x: for x = -0 the FMAs would return +0, while -0 / s is -0
// and encodes to the code 0x80.)
__device__ __forceinline__ float div_rn(float x, float s, float r) {
  const float q = x * r;
  return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q, s, x), r, q), x);
}
constexpr float kMinFastScale = 0x1.0p-80f;  // smaller scales take the plain division

// Four e4m3 codes of v[0..3] packed little-endian, by the hardware conversion
// (v_cvt_pk_fp8_f32: round to nearest even, OCP e4m3fn).  Checked on MI355X against
// e4m3_encode over every finite fp32 value: identical for |v| < 448, and v in [448, 500]
// also gives 0x7E; the quotients here are at most RN(448 (1 + 2^-24)).
__device__ __forceinline__ uint32_t e4m3_hw4(float v0, float v1, float v2, float v3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, lo, true);
}

// e4m3 codes of f[i] / s, packed little-endian into 8 bytes
__device__ __forceinline__ uint2 e4m3_pack8(const float (&f)[8], float s) {
  uint32_t lo = 0, hi = 0;
  if (s >= kMinFastScale) {
    const float r = 1.0f / s;
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = div_rn(f[i], s, r);
    lo = e4m3_hw4(q[0], q[1], q[2], q[3]);
    hi = e4m3_hw4(q[4], q[5], q[6], q[7]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= e4m3_encode(f[i] / s) << (8 * i);
      hi |= e4m3_encode(f[4 + i] / s) << (8 * i);
    }
  }
  return make_uint2(lo, hi);
}

// FP8, 128-column groups: 16 lanes per (row, group), eight columns (16 bytes) per lane;
// a workgroup takes U runs of 16 consecutive groups and issues all U loads of a lane
// before the first reduction, so U loads per lane are in flight.  Every lane takes part
// in the group reductions (no early return before the shuffles).
template <int U>
__global__ __launch_bounds__(256) void quant_fp8_g128_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                             const int32_t* __restrict__ rows_dev,
                                                             uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int ng = (cols + 127) / 128;
  const int sub = (int)(threadIdx.x & 15);
  const int n_rows = rows_dev ? min(rows, rows_dev[0]) : rows;
  float f[U][8];
  int r[U], c[U], gi[U];
  bool live[U], ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long gid = ((long)blockIdx.x * U + u) * 16 + (threadIdx.x >> 4);
    const bool in = gid < (long)rows * ng;
    r[u] = in ? (int)(gid / ng) : 0;
    gi[u] = in ? (int)(gid % ng) : 0;
    live[u] = in && r[u] < n_rows;
    c[u] = gi[u] * 128 + 8 * sub;
    ok[u] = live[u] && c[u] < cols;  // cols % 32 == 0: eight columns are all in or all out
    load8_bf16(x + (size_t)r[u] * cols + c[u], ok[u], f[u]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float m = amax8(f[u]);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    const float s = m > 0.0f ? m / 448.0f : 1.0f;
    if (ok[u]) *(uint2*)(codes + (size_t)r[u] * cols + c[u]) = e4m3_pack8(f[u], s);
    if (live[u] && sub == 0) scales[(size_t)r[u] * ng + gi[u]] = s;
  }
}

// FP8, one scale per row: one workgroup of NT threads per row; a thread keeps its up to
// 8 * CH values in registers between the row maximum and the encoding (cols <= 8 * CH * NT).
template <int NT, int CH>
__global__ __launch_bounds__(NT) void quant_fp8_token_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                             const int32_t* __restrict__ rows_dev,
                                                             uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int r = blockIdx.x;
  if (rows_dev && r >= rows_dev[0]) return;
  __shared__ float red[NT / kWave];
  const uint16_t* xr = x + (size_t)r * cols;
  float f[CH][8];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {  // cols % 32 == 0: eight columns are all in or all out
    const int c = 8 * ((int)threadIdx.x + NT * i);
    load8_bf16(xr + c, c < cols, f[i]);
    m = fmaxf(m, amax8(f[i]));
  }
  m = wave_max(m);
  if (lane_id() == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  float amax = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) amax = fmaxf(amax, red[i]);
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = 8 * ((int)threadIdx.x + NT * i);
    if (c < cols) *(uint2*)(codes + (size_t)r * cols + c) = e4m3_pack8(f[i], s);
  }
  if (threadIdx.x == 0) scales[r] = s;
}

// MXFP4, 32-column groups: 4 lanes per group, eight columns (16 bytes in, 4 code bytes
// out) per lane; a workgroup takes U runs of 256 lanes' columns, all U loads issued first.
template <int U>
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                          const int32_t* __restrict__ rows_dev,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const long per_row = cols / 8;
  const int n_rows = rows_dev ? min(rows, rows_dev[0]) : rows;
  float f[U][8];
  int r[U], c[U];
  bool live[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long q = ((long)blockIdx.x * U + u) * 256 + threadIdx.x;  // index of 8 consecutive columns
    const bool in = q < (long)rows * per_row;
    r[u] = in ? (int)(q / per_row) : 0;
    c[u] = in ? (int)(q % per_row) * 8 : 0;
    live[u] = in && r[u] < n_rows;
    load8_bf16(x + (size_t)r[u] * cols + c[u], live[u], f[u]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float m = amax8(f[u]);
    // groups are 4 consecutive lanes (cols % 32 == 0 keeps groups inside one row)
    m = fmaxf(m, __shfl_xor(m, 2, kWave));
    m = fmaxf(m, __shfl_xor(m, 1, kWave));
    const int es = mx_shared_exp(m);
    const float inv = exp2i(-es);
    if (live[u]) {
      // e2m1 codes of x 2^-es (an exact product) by the hardware conversion at unit scale
      // (v_cvt_scalef32_pk_fp4_f32: round to nearest even, saturating at 6), checked on
      // MI355X against e2m1_encode over every finite fp32 value: identical; byte i holds
      // elements 2i (low nibble) and 2i + 1
      const float(&g)[8] = f[u];
      uint32_t packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, g[0] * inv, g[1] * inv, 1.0f, 0);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, g[2] * inv, g[3] * inv, 1.0f, 1);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, g[4] * inv, g[5] * inv, 1.0f, 2);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, g[6] * inv, g[7] * inv, 1.0f, 3);
      *(uint32_t*)(codes + (size_t)r[u] * (cols / 2) + c[u] / 2) = packed;
      if ((c[u] & 31) == 0) scales[(size_t)r[u] * (cols / 32) + c[u] / 32] = (uint8_t)(es + 127);
    }
  }
}

// FP8, one scale for the whole tensor (rows [0, *rows_dev) when rows_dev is given).
// Four launches that need no scratch memory: the scale slot first holds the amax as
// float bits (values are >= 0, so their uint order is their float order and an integer
// atomic max is exact and order-independent), then the scale.
__global__ void tensor_amax_zero_kernel(uint32_t* acc) { acc[0] = 0u; }

__global__ __launch_bounds__(256) void tensor_amax_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                          const int32_t* __restrict__ rows_dev,
                                                          uint32_t* __restrict__ acc) {
  __shared__ float red[4];
  const int n_rows = rows_dev ? min(rows, rows_dev[0]) : rows;
  const long octs = (long)n_rows * (cols / 8);  // 8 elements (16 bytes) per step
  float m = 0.0f;
  for (long q = (long)blockIdx.x * blockDim.x + threadIdx.x; q < octs; q += (long)gridDim.x * blockDim.x) {
    float f[8];
    load8_bf16(x + 8 * q, true, f);
    m = fmaxf(m, amax8(f));
  }
  m = wave_max(m);
  if (lane_id() == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(acc, __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

__global__ __launch_bounds__(256) void quant_fp8_tensor_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                               const int32_t* __restrict__ rows_dev,
                                                               uint8_t* __restrict__ codes,
                                                               const uint32_t* __restrict__ acc) {
  const float amax = __uint_as_float(acc[0]);
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  const int n_rows = rows_dev ? min(rows, rows_dev[0]) : rows;
  const long octs = (long)n_rows * (cols / 8);
  for (long q = (long)blockIdx.x * blockDim.x + threadIdx.x; q < octs; q += (long)gridDim.x * blockDim.x) {
    float f[8];
    load8_bf16(x + 8 * q, true, f);
    *(uint2*)(codes + 8 * q) = e4m3_pack8(f, s);
  }
}

__global__ void tensor_scale_final_kernel(uint32_t* acc) {
  const float amax = __uint_as_float(acc[0]);
  ((float*)acc)[0] = amax > 0.0f ? amax / 448.0f : 1.0f;
}

hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, int fmt, const int32_t* rows_dev,
                            uint8_t* codes, void* scales, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (fmt == kAFp8Tensor) {
    const long octs = (long)rows * (cols / 8);
    const unsigned g = (unsigned)std::min<long>((octs + 255) / 256, 4096);
    uint32_t* acc = (uint32_t*)scales;
    tensor_amax_zero_kernel<<<1, 1, 0, stream>>>(acc);
    tensor_amax_kernel<<<g, 256, 0, stream>>>(x, rows, cols, rows_dev, acc);
    quant_fp8_tensor_kernel<<<g, 256, 0, stream>>>(x, rows, cols, rows_dev, codes, acc);
    tensor_scale_final_kernel<<<1, 1, 0, stream>>>(acc);
    return hipGetLastError();
  }
  constexpr int U = 4;  // loads in flight per lane in the group quantisers
  if (fmt == kAFp8G128) {
    const long groups = (long)rows * ((cols + 127) / 128);  // 16 U per 256-thread workgroup
    quant_fp8_g128_kernel<U><<<(unsigned)((groups + 16 * U - 1) / (16 * U)), 256, 0, stream>>>(x, rows, cols, rows_dev,
                                                                                              codes, (float*)scales);
  } else if (fmt == kAFp8Token) {
    // one workgroup per row; the smallest of these shapes that holds the row, so that a
    // thread has several 16-byte loads in flight: 256 threads x 1..8 octets (up to 16384
    // columns), then 512 and 1024 threads x 8 octets (up to 65536).  With few rows (up to
    // 512, e.g. a2 of one to a few tokens) the chip is mostly idle and each row's latency
    // counts: 1024 threads per wide row, so that a thread encodes fewer values in sequence.
    const int oct = cols / 8;
    float* sc = (float*)scales;
    const unsigned R = (unsigned)rows;
    if (rows <= 512 && oct > 512) {
      if (oct <= 2048) quant_fp8_token_kernel<1024, 2><<<R, 1024, 0, stream>>>(x, rows, cols, rows_dev, codes, sc);
      else if (oct <= 4096) quant_fp8_token_kernel<1024, 4><<<R, 1024, 0, stream>>>(x, rows, cols, rows_dev, codes, sc);
      else quant_fp8_token_kernel<1024, 8><<<R, 1024, 0, stream>>>(x, rows, cols, rows_dev, codes, sc);
    } else if (oct <= 256) quant_fp8_token_kernel<256, 1><<<R, 256, 0, stream>>>(x, rows, cols, rows_dev, codes, sc);
    else if (oct <= 512) quant_fp8_token_kernel<256, 2><<<R, 256, 0, stream>>>(x, rows, cols, rows_dev, codes, sc);
    else if (oct <= 1024) quant_fp8_token_kernel<256, 4><<<R, 256, 0, stream>>>(x, rows, cols, rows_dev, codes, sc);
    else if (oct <= 2048) quant_fp8_token_kernel<256, 8><<<R, 256, 0, stream>>>(x, rows, cols, rows_dev, codes, sc);
    else if (oct <= 4096) quant_fp8_token_kernel<512, 8><<<R, 512, 0, stream>>>(x, rows, cols, rows_dev, codes, sc);
    else quant_fp8_token_kernel<1024, 8><<<R, 1024, 0, stream>>>(x, rows, cols, rows_dev, codes, sc);
  } else {
    const long octs = (long)rows * (cols / 8);
    quant_mxfp4_kernel<U><<<(unsigned)((octs + 256 * U - 1) / (256 * U)), 256, 0, stream>>>(x, rows, cols, rows_dev,
                                                                                           codes, (uint8_t*)scales);
  }
  return hipGetLastError();
}

}  // namespace moe
