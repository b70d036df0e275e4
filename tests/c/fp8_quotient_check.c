/* Checks the quotient route of the in-wave FP8 row encode against correctly rounded
 * fp32 division, on the host (IEEE binary32 mul / fma / div, no contraction).
 *
 * Route (for a row scale s >= 2^-64): y = 1/s rounded, q0 = x*y rounded,
 * e = fma(-s, q0, x) (the exact remainder), q = fma(e, y, q0), then x's sign bit
 * copied onto q.  Markstein's theorem (P. Markstein, IBM J. Res. Dev. 34(1), 1990;
 * also Muller et al., Handbook of Floating-Point Arithmetic, section on division
 * with an FMA) gives q = RN(x/s) when y = RN(1/s), q0 is within one ulp of x/s and
 * nothing underflows.  The encode only needs that much where the quotient can round
 * to a nonzero E4M3 value: there (|x/s| >= 2^-11) q must equal x/s correctly
 * rounded bit for bit; below, both round to an E4M3 zero, so q must stay below
 * 2^-10 in magnitude and carry x's sign.
 *
 * Prints "ok <checks>" or the first failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float route(float x, float s) {
  volatile float y = 1.0f / s;
  volatile float q0 = x * y;
  volatile float e = fmaf(-s, q0, x);
  volatile float q = fmaf(e, y, q0);
  return f_of((u_of(q) & 0x7fffffffu) | (u_of(x) & 0x80000000u));
}

static long checked = 0;

static int check(float x, float s) {
  volatile float ref = x / s;
  const float q = route(x, s);
  ++checked;
  if (fabsf(ref) >= 0x1p-11f) {
    if (u_of(q) != u_of(ref)) {
      printf("FAIL x=%a s=%a route=%a div=%a\n", x, s, q, ref);
      return 1;
    }
  } else if (!(fabsf(q) < 0x1p-10f) || (u_of(q) >> 31) != (u_of(x) >> 31)) {
    printf("FAIL small x=%a s=%a route=%a div=%a\n", x, s, q, ref);
    return 1;
  }
  return 0;
}

/* every finite x with lo <= |x| <= hi, both signs */
static int sweep(float s, float lo, float hi) {
  for (uint32_t u = u_of(lo); u < 0x7f800000u; ++u) {
    const float x = f_of(u);
    if (x > hi) break;
    if (check(x, s) || check(-x, s)) return 1;
  }
  return 0;
}

static uint64_t st = 0x9e3779b97f4a7c15ull;
static uint32_t rnd(void) {  /* splitmix64 */
  uint64_t z = (st += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}

/* Usage: fp8_quotient_check <random pairs> [full]
 * full: every x with |x| <= 448 s for each scale below (8.8e9 checks, minutes);
 * otherwise every x in the binades around the 2^-11 threshold and in the top
 * binade [256 s, 448 s]. */
int main(int argc, char** argv) {
  const long pairs = argc > 1 ? atol(argv[1]) : 20000000L;
  const int full = argc > 2 && strcmp(argv[2], "full") == 0;
  /* scales: the threshold, a generic significand, all-ones significands, 1/448 */
  const float scales[] = {0x1p-64f, 0x1.fffffep-64f, 0x1.3c5e8ap-20f, 0x1.fffffep-1f,
                          1.0f / 448.0f};
  for (unsigned i = 0; i < sizeof(scales) / sizeof(scales[0]); ++i) {
    const float s = scales[i], top = 448.0f * s * (1.0f + 0x1p-20f);
    /* signed zeros and the subnormal ends (the division's sign must survive) */
    const float tiny[] = {0.0f, 0x1p-149f, 0x1.fffffcp-127f, 0x1p-126f};
    for (unsigned t = 0; t < sizeof(tiny) / sizeof(tiny[0]); ++t)
      if (check(tiny[t], s) || check(-tiny[t], s)) return 1;
    if (full ? sweep(s, 0.0f, top)
             : (sweep(s, 0x1p-13f * s, 0x1p-9f * s) || sweep(s, 256.0f * s, top)))
      return 1;
  }
  /* random row scales s = RN(amax/448) >= 2^-64 and random |x| <= amax, as bit
   * patterns (so every magnitude down to the subnormals is drawn) */
  for (long k = 0; k < pairs; ++k) {
    const uint32_t ea = 64 + 9 + (rnd() % (254 - 73));          /* amax exponent field */
    const float amax = f_of((ea << 23) | (rnd() & 0x7fffffu));
    float s = amax / 448.0f;
    if (s < 0x1p-64f) continue;
    const uint32_t xu = rnd() % (u_of(amax) + 1u);
    const float x = f_of(xu | ((rnd() & 1u) << 31));
    if (check(x, s)) return 1;
  }
  printf("ok %ld\n", checked);
  return 0;
}
