// Dynamic activation quantisation: FP8 e4m3fn per 128-group, per row or per tensor, and MXFP4
// (e2m1 + E8M0) per 32-group (pages: "rocm_aiter_moe", AiterFp8BlockExperts,
// AiterFp8ChannelExperts, AiterMxfp4Experts; packing two FP4 codes per byte as in
// "quark_moe", QuarkOCP_MX_MoEMethod.get_packed_dim).
//
// The encoders take their decisions in IEEE fp32 exactly as documented for
// moe_quant_act: amax is exact, s = amax / 448 and x / s are correctly rounded fp32
// divisions (hipcc keeps fp32 division correctly rounded unless fast-math is asked
// for), and the element rounding is done in integer-exact steps, so the codes are
// bit-identical to the oracle's given the same bf16 input.
#include "moe_device.h"
#include "moe_internal.h"

#include <algorithm>

namespace moe {

// FP8, 128-column groups: one wave per (row, group), two columns per lane.
__global__ __launch_bounds__(256) void quant_fp8_g128_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                             const int32_t* __restrict__ rows_dev,
                                                             uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int ng = (cols + 127) / 128;
  const long gid = (long)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (gid >= (long)rows * ng) return;
  const int r = (int)(gid / ng), g = (int)(gid % ng);
  if (rows_dev && r >= rows_dev[0]) return;
  const int lane = lane_id();
  const int c = g * 128 + 2 * lane;
  const bool ok = c < cols;
  uint32_t pair = ok ? *(const uint32_t*)(x + (size_t)r * cols + c) : 0u;
  const float v0 = bf16_to_f32(pair & 0xFFFFu), v1 = bf16_to_f32(pair >> 16);
  const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (ok) {
    const uint32_t q = e4m3_encode(v0 / s) | (e4m3_encode(v1 / s) << 8);
    *(uint16_t*)(codes + (size_t)r * cols + c) = (uint16_t)q;
  }
  if (lane == 0) scales[(size_t)r * ng + g] = s;
}

// FP8, one scale per row: one 256-thread workgroup per row.
__global__ __launch_bounds__(256) void quant_fp8_token_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                              const int32_t* __restrict__ rows_dev,
                                                              uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int r = blockIdx.x;
  if (rows_dev && r >= rows_dev[0]) return;
  __shared__ float red[4];
  const uint16_t* xr = x + (size_t)r * cols;
  float m = 0.0f;
  for (int c = 2 * (int)threadIdx.x; c < cols; c += 512) {
    const uint32_t pair = *(const uint32_t*)(xr + c);
    m = fmaxf(m, fmaxf(fabsf(bf16_to_f32(pair & 0xFFFFu)), fabsf(bf16_to_f32(pair >> 16))));
  }
  m = wave_max(m);
  if (lane_id() == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int c = 2 * (int)threadIdx.x; c < cols; c += 512) {
    const uint32_t pair = *(const uint32_t*)(xr + c);
    const uint32_t q = e4m3_encode(bf16_to_f32(pair & 0xFFFFu) / s) | (e4m3_encode(bf16_to_f32(pair >> 16) / s) << 8);
    *(uint16_t*)(codes + (size_t)r * cols + c) = (uint16_t)q;
  }
  if (threadIdx.x == 0) scales[r] = s;
}

// MXFP4, 32-column groups: 16 lanes per group, two columns (one output byte) per lane.
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                          const int32_t* __restrict__ rows_dev,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const long pairs_per_row = cols / 2;
  const long p = (long)blockIdx.x * blockDim.x + threadIdx.x;  // pair index
  const bool in = p < (long)rows * pairs_per_row;
  const int r = in ? (int)(p / pairs_per_row) : 0;
  const int c = in ? (int)(p % pairs_per_row) * 2 : 0;
  const bool live = in && !(rows_dev && r >= rows_dev[0]);
  const uint32_t pair = live ? *(const uint32_t*)(x + (size_t)r * cols + c) : 0u;
  const float v0 = bf16_to_f32(pair & 0xFFFFu), v1 = bf16_to_f32(pair >> 16);
  float m = fmaxf(fabsf(v0), fabsf(v1));
  // groups are 16 consecutive lanes (cols % 32 == 0 keeps groups inside one row)
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  const int es = mx_shared_exp(m);
  const float inv = exp2i(-es);
  if (live) {
    codes[(size_t)r * (cols / 2) + c / 2] = (uint8_t)(e2m1_encode(v0 * inv) | (e2m1_encode(v1 * inv) << 4));
    if ((c & 31) == 0) scales[(size_t)r * (cols / 32) + c / 32] = (uint8_t)(es + 127);
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
  const long pairs = (long)n_rows * (cols / 2);
  float m = 0.0f;
  for (long q = (long)blockIdx.x * blockDim.x + threadIdx.x; q < pairs; q += (long)gridDim.x * blockDim.x) {
    const uint32_t pair = *(const uint32_t*)(x + 2 * q);
    m = fmaxf(m, fmaxf(fabsf(bf16_to_f32(pair & 0xFFFFu)), fabsf(bf16_to_f32(pair >> 16))));
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
  const long pairs = (long)n_rows * (cols / 2);
  for (long q = (long)blockIdx.x * blockDim.x + threadIdx.x; q < pairs; q += (long)gridDim.x * blockDim.x) {
    const uint32_t pair = *(const uint32_t*)(x + 2 * q);
    const uint32_t c = e4m3_encode(bf16_to_f32(pair & 0xFFFFu) / s) | (e4m3_encode(bf16_to_f32(pair >> 16) / s) << 8);
    *(uint16_t*)(codes + 2 * q) = (uint16_t)c;
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
    const long pairs = (long)rows * (cols / 2);
    const unsigned g = (unsigned)std::min<long>((pairs + 255) / 256, 4096);
    uint32_t* acc = (uint32_t*)scales;
    tensor_amax_zero_kernel<<<1, 1, 0, stream>>>(acc);
    tensor_amax_kernel<<<g, 256, 0, stream>>>(x, rows, cols, rows_dev, acc);
    quant_fp8_tensor_kernel<<<g, 256, 0, stream>>>(x, rows, cols, rows_dev, codes, acc);
    tensor_scale_final_kernel<<<1, 1, 0, stream>>>(acc);
    return hipGetLastError();
  }
  if (fmt == kAFp8G128) {
    const long groups = (long)rows * ((cols + 127) / 128);
    quant_fp8_g128_kernel<<<(unsigned)((groups + 3) / 4), 256, 0, stream>>>(x, rows, cols, rows_dev, codes,
                                                                              (float*)scales);
  } else if (fmt == kAFp8Token) {
    quant_fp8_token_kernel<<<(unsigned)rows, 256, 0, stream>>>(x, rows, cols, rows_dev, codes, (float*)scales);
  } else {
    const long pairs = (long)rows * (cols / 2);
    quant_mxfp4_kernel<<<(unsigned)((pairs + 255) / 256), 256, 0, stream>>>(x, rows, cols, rows_dev, codes,
                                                                             (uint8_t*)scales);
  }
  return hipGetLastError();
}

}  // namespace moe
