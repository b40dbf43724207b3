/* Host check of the two fp32 identities the activation quantizer's fast
 * path relies on (built with gcc -ffp-contract=off, so every product and sum
 * below is one IEEE binary32 operation and fmaf is the fused operation):
 *
 *  1. Markstein's correction: with r = RN(1/d), q0 = RN(n*r),
 *     e = fma(-q0, d, n), q1 = fma(e, r, q0), q1 equals the correctly
 *     rounded quotient RN(n/d).  The kernel uses it only for divisors in
 *     [2^-100, 2^122) (smaller scales are lifted by 2^64 first) and quotients
 *     up to 127 in magnitude.  Checked exhaustively over every fp32 n with
 *     2^-3 <= |n/d| <= 128 for a set of divisors d (mantissa extremes, the
 *     scales of typical rows, both ends of that range), and on 2e8 random
 *     (n, d) pairs with d in [2^-100, 2^100).  Below 2^-100 the remainder
 *     fma(-q0, d, n) can fall under the subnormal grid and the identity
 *     fails (e.g. d just under 2^-100, n/d near 1/8).
 *  2. Rounding half away from zero: for every fp32 q with |q| <= 128,
 *     trunc(q + copysign(0.49999997, q)) == roundf(q).  Exhaustive.
 *
 * Prints one line per check and exits non-zero on the first mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* PLANT_* builds plant a known mistake so the test can show the checker
 * rejects it. */
static float markstein(float n, float d, float r) {
  const float q0 = n * r;
#ifdef PLANT_NO_CORRECTION
  (void)d;
  return q0;
#else
  const float e = fmaf(-q0, d, n);
  return fmaf(e, r, q0);
#endif
}

static int half_away(float q) {
#ifdef PLANT_PLAIN_HALF
  const float h = f_of((u_of(q) & 0x80000000u) | 0x3f000000u);
#else
  const float h = f_of((u_of(q) & 0x80000000u) | 0x3effffffu);
#endif
  return (int)(q + h);
}

static uint64_t splitmix(uint64_t* s) {
  uint64_t z = (*s += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

static int check_divisor(float d) {
  const float r = 1.0f / d;
  const uint32_t lo = u_of(d * 0.125f);
  const uint32_t hi = isinf(d * 128.0f) ? 0x7f7fffffu : u_of(d * 128.0f);  /* finite n only */
  long bad = 0;
  uint32_t first = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (int64_t k = lo; k <= (int64_t)hi; ++k) {
    for (int sign = 0; sign < 2; ++sign) {
      const float n = f_of((uint32_t)k | (sign ? 0x80000000u : 0u));
      if (u_of(markstein(n, d, r)) != u_of(n / d)) {
        bad += 1;
        first = (uint32_t)k;
      }
    }
  }
  printf("markstein d=%a: %u numerators x2 signs, %ld mismatches\n", d, hi - lo + 1, bad);
  if (bad) printf("  e.g. n=%a\n", f_of(first));
  return bad != 0;
}

int main(void) {
  /* 2: exhaustive rounding check */
  long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (int64_t k = 0; k <= 0x43000000ll; ++k) {
    for (int sign = 0; sign < 2; ++sign) {
      const float q = f_of((uint32_t)k | (sign ? 0x80000000u : 0u));
      if (half_away(q) != (int)roundf(q)) bad += 1;
    }
  }
  printf("half_away: every |q| <= 128, %ld mismatches\n", bad);
  if (bad) return 1;

  /* 1: exhaustive Markstein over chosen divisors */
  const float divisors[] = {
      1.0f, f_of(0x3fffffffu), f_of(0x3f800001u), f_of(0x3fc00000u), f_of(0x3faaaaabu),
      f_of(0x3f7fffffu), 1.0f / 127.0f, 3.0f / 127.0f, 0.02f * 16.0f * 4.0f / 127.0f,
      0x1p-100f, f_of(0x0d800001u), f_of(0x0dffffffu), 0x1p+100f, 0x1p+121f, f_of(0x7c7fffffu),
      7.3e-3f, 123.456f, 0.1f};
  for (size_t i = 0; i < sizeof(divisors) / sizeof(divisors[0]); ++i)
    if (check_divisor(divisors[i])) return 1;

  /* 1: random pairs, d with exponent in [2^-100, 2^100), |n/d| in [2^-3, 128] */
  const long pairs = 200000000l;
  bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (long i = 0; i < pairs; ++i) {
    uint64_t st = (uint64_t)i * 0x632be59bd9b4e019ull + 12345u;
    const uint64_t a = splitmix(&st), b = splitmix(&st);
    const float d = f_of((uint32_t)((27 + (a % 200)) << 23) | (uint32_t)(a >> 41));
    const float qt = f_of((uint32_t)((124 + (b % 10)) << 23) | (uint32_t)(b >> 41));
    float n = qt * d;
    if (b & (1ull << 40)) n = -n;
    const float r = 1.0f / d;
    if (u_of(markstein(n, d, r)) != u_of(n / d)) bad += 1;
  }
  printf("markstein random: %ld pairs, %ld mismatches\n", pairs, bad);
  return bad != 0;
}
