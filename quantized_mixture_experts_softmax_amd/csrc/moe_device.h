// Device-side helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even (NaN -> canonical quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Nearest e4m3fn code (OCP FP8: bias 7, max 448, no inf), ties to even mantissa,
// saturating at 448; the sign bit follows the input's sign bit.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a != a) {
    code = 0x7Fu;
  } else if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    // subnormal binade, spacing 2^-9; a result of 8 is the smallest normal (code 8)
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t ab = __float_as_uint(a);
    const int E = (int)(ab >> 23) - 127;                               // -6 .. 8
    const float m8 = __uint_as_float((ab & 0x007FFFFFu) | 0x41000000u); // 1.m * 8 in [8, 16)
    const uint32_t q = (uint32_t)__builtin_rintf(m8);                  // 8 .. 16
    // q - 8 == 8 carries into the exponent field, which is the next binade's 1.0
    code = ((uint32_t)(E + 7) << 3) + (q - 8u);
  }
  return sign | code;
}

// Nearest e2m1 code (OCP MX FP4: 0, .5, 1, 1.5, 2, 3, 4, 6), ties to even
// mantissa bit, saturating at 6; sign bit copied from the input.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
  const float a = fabsf(v);
  uint32_t code;
  if (!(a < 6.0f)) code = 7u;
  else if (a < 2.0f) code = (uint32_t)__builtin_rintf(a * 2.0f);
  else if (a < 4.0f) code = 2u + (uint32_t)__builtin_rintf(a);
  else code = 4u + (uint32_t)__builtin_rintf(a * 0.5f);
  return sign | code;
}

// OCP MX shared exponent of an FP4 block: floor(log2 amax) - 2, clamped to
// [-127, 127]; -127 for an all-zero block.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127 - 2; // subnormal amax -> clamped below
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^e as fp32 for e in [-127, 127] (2^-127 is subnormal).
__device__ __forceinline__ float exp2i(int e) {
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// E8M0 byte -> fp32 scale 2^(b-127) (one v_ldexp_f32, exact down to the subnormal
// 2^-127; the byte 255, NaN in E8M0, is not produced by any path here).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) { return __builtin_ldexpf(1.0f, (int)b - 127); }

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Workgroup barrier for LDS hand-over only: waits for this wave's LDS operations, not
// for its global loads in flight (__syncthreads waits for those too, which would drain
// a weight prefetch ring).  The empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace moe
