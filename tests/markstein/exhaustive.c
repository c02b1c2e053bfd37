/* The FP8 quantisers divide x by s with one FMA correction of x * RN(1/s) (csrc/quant_act.hip,
 * div_rn).  This checks that method against the correctly rounded division for every pair of
 * bf16 values the quantisers can see: every positive bf16 amax whose scale s = RN(amax / 448)
 * is at least 2^-80 (smaller scales take the plain division), and every bf16 x in (0, amax]
 * (the method and the rounding are symmetric in the sign of nonzero x), and x = +0 and -0,
 * whose quotient must keep the sign of x (the device code applies copysign; without it the
 * FMAs turn -0 into +0, a different e4m3 code).  Quotients below 2^-11 round
 * to a zero e4m3 code whatever their last bit, so only quotients at or above it must agree.
 * Exit status 0 when every such quotient matches. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void) {
  long bad = 0, n = 0;
  for (uint32_t a = 0x0080; a < 0x7F80; ++a) {
    const float amax = from_bits(a << 16);
    const float s = amax / 448.0f;
    if (!(s >= 0x1.0p-80f)) continue;
    const float r = 1.0f / s;
    for (int neg = 0; neg < 2; ++neg) {  /* signed zeros */
      const float x = neg ? -0.0f : 0.0f;
      const float d = copysignf(fmaf(fmaf(-(x * r), s, x), r, x * r), x);
      ++n;
      if (to_bits(d) != to_bits(x / s)) ++bad;
    }
    for (uint32_t b = 1; b <= a; ++b) {
      const float x = from_bits(b << 16);
      const float q = x * r;
      const float d = copysignf(fmaf(fmaf(-q, s, x), r, q), x);
      const float ref = x / s;
      ++n;
      if (to_bits(d) != to_bits(ref) && fabsf(ref) >= 0x1.0p-11f) {
        if (bad < 5) printf("x=%a s=%a: %a, correctly rounded %a\n", x, s, d, ref);
        ++bad;
      }
    }
  }
  printf("%ld of %ld quotients differ\n", bad, n);
  return bad != 0;
}
