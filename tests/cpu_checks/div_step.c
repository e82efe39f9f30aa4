/* Checks, on the host, the division step the GPU quantiser uses: for s in
 * [2^-60, 2^60] and |a| >= 2^-60 (or a = 0), with r = RN(1/s),
 * q0 = RN(a*r), e = fma(-q0, s, a), q = (e == 0 ? q0 : fma(e, r, q0))
 * equals RN(a/s) bit for bit (Markstein's theorem on FMA division).
 * argv[1]: number of random cases.  Prints the mismatch count. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t xr(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }

static int in_domain(float a, float s) {
  return s >= 0x1p-60f && s <= 0x1p60f && (fabsf(a) >= 0x1p-60f || a == 0.0f);
}
static float step_div(float a, float s) {
  float r = 1.0f / s, q0 = a * r, e = fmaf(-q0, s, a);
  return e == 0.0f ? q0 : fmaf(e, r, q0);
}

int main(int argc, char** argv) {
  long n = argc > 1 ? atol(argv[1]) : 1000000, checked = 0, bad = 0;
  for (long i = 0; i < n; ++i) {
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
      if (isnan(a) || isinf(a) || isnan(s) || isinf(s) || s == 0) continue;
    }
    if (!in_domain(a, s)) continue;
    float ref = a / s;
    if (isinf(ref)) continue;
    ++checked;
    if (bf(step_div(a, s)) != bf(ref)) ++bad;
  }
  printf("%ld %ld\n", checked, bad);
  return 0;
}
