/* Host check of the arithmetic the GPU quantiser uses in place of IEEE
 * division (Markstein's theorem on FMA-based division):
 *  1. scale: for m in [2^-40, 2^68], q0 = RN(m*y), y = RN(1/448),
 *     s = RN(q0 + RN(m - 448*q0)*y) (two FMAs) equals RN(m/448);
 *  2. quotient: for s in [2^-49, 2^60], r = RN(1/s), q0 = RN(a*r),
 *     q = copysign(fma(fma(-q0, s, a), r, q0), a) equals RN(a/s) for
 *     |a| >= 2^-60 and a = +-0; for smaller nonzero |a| both are below
 *     2^-11 in magnitude (an e4m3 zero) with a's sign.
 * argv[1]: random cases per check.  Prints "checked mismatches". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t xr(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }

static float scale448(float m) {
  const float y = 1.0f / 448.0f;
  float q0 = m * y, e = fmaf(-q0, 448.0f, m);
  return fmaf(e, y, q0);
}
static float step_div(float a, float s) {
  float r = 1.0f / s, q0 = a * r, e = fmaf(-q0, s, a);
  return copysignf(fmaf(e, r, q0), a);
}

int main(int argc, char** argv) {
  long n = argc > 1 ? atol(argv[1]) : 1000000, checked = 0, bad = 0;
  for (long i = 0; i < n; ++i) {   /* 1: scales over the whole domain */
    float m = fb((uint32_t)(xr() & 0x7FFFFFFF));
    if (!(m >= 0x1p-40f && m <= 0x1p68f)) continue;
    ++checked;
    if (bf(scale448(m)) != bf(m / 448.0f)) ++bad;
  }
  for (long i = 0; i < n; ++i) {   /* 2: quotients */
    float a, s;
    if (i & 1) {   /* quantiser-shaped: s = amax/448, |a| <= amax, bf16 values */
      float amax = fb((uint32_t)(xr() & 0x7FFF) << 16);
      a = fb((uint32_t)(xr() & 0xFFFF) << 16);
      if (!(amax > 0) || isinf(amax) || isnan(a) || isinf(a) || fabsf(a) > amax) continue;
      s = amax / 448.0f;
    } else {       /* any finite pair, zeros of both signs included */
      s = fb((uint32_t)(xr() & 0x7FFFFFFF));
      uint32_t au = (uint32_t)xr();
      if ((i & 255) == 0) au &= 0x80000000u;
      a = fb(au);
      if (isnan(a) || isinf(a) || isnan(s) || isinf(s)) continue;
    }
    if (!(s >= 0x1p-49f && s <= 0x1p60f)) continue;
    float ref = a / s;
    if (isinf(ref)) continue;
    float q = step_div(a, s);
    ++checked;
    if (fabsf(a) >= 0x1p-60f || a == 0.0f) {
      if (bf(q) != bf(ref)) ++bad;
    } else if (!(fabsf(q) < 0x1p-11f && fabsf(ref) < 0x1p-11f && signbit(q) == signbit(a) &&
                 signbit(ref) == signbit(a))) {
      ++bad;
    }
  }
  printf("%ld %ld\n", checked, bad);
  return 0;
}
