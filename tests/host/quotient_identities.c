/* Host check of the fp32 arithmetic the activation quantizer's fast path
 * relies on (built with gcc -ffp-contract=off, so every product and sum below
 * is one IEEE binary32 operation and fmaf is the fused operation).
 *
 * The kernel turns a rotated value v into its int8 code with one fused
 * multiply-add and a byte pick:
 *     rb   = RN(1/d) raised by two units in the last place   (once per row)
 *     bits = fma(v, rb, 1.5 * 2^23)
 *     code = the low byte of bits, as a two's-complement int8
 * and d = absmax / 127 is the row's scale.
 *
 *  1. Byte identity: for every real p with |p| < 2^22, RN(p + 1.5 * 2^23)
 *     is 1.5 * 2^23 + RNE(p) (the unit in the last place there is 1 and
 *     1.5 * 2^23 is even, so ties go to the even integer), whose low byte
 *     is RNE(p) mod 256.  Checked exhaustively over every fp32 p with
 *     |p| <= 128 (fmaf(p, 1, magic)), and on 1e8 random products v * rb
 *     (exact in fp64) whose rounding the fused operation takes once.
 *  2. Bias: rb * d > 1 strictly and rb * d - 1 <= 2^-22 + 2^-24, for every
 *     24-bit mantissa of d in one binade (scaling d by a power of two scales
 *     RN(1/d) exactly, so the binade stands for the kernel's whole range of
 *     scales, [2^-100, 2^122)).  Hence |v * rb| > |v / d|: an exact tie
 *     v / d = n + 1/2 rounds away from zero, as the definition does, and
 *     |v * rb| exceeds |v / d| by at most 2^-21 of it.
 *  3. The decision: on 2e8 random (v, d) pairs with |v / d| <= 127, and on
 *     every exact tie n + 1/2 (n = 0..126) at 20000 scales, the byte code
 *     equals round_half_away(v / d) taken exactly, except just below a
 *     rounding boundary: where the exact |v / d| lies within 2^-21 of it
 *     under n + 1/2, the code may be one further from zero.
 *
 * Prints one line per check and exits non-zero on the first failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* PLANT_* builds plant a known mistake so the test can show the checker
 * rejects it. */
#ifdef PLANT_MAGIC_2P23
static const float kMagic = 8388608.0f;         /* 2^23: negative p fall into the binade below */
#else
static const float kMagic = 12582912.0f;        /* 1.5 * 2^23 */
#endif

static float raise2(float r) {
#ifdef PLANT_NO_BUMP
  return r;                                      /* exact ties would round to even */
#else
  return f_of(u_of(r) + 2u);
#endif
}

static int byte_code(float v, float rb) { return (int)(int8_t)(u_of(fmaf(v, rb, kMagic)) & 0xffu); }

static double half_away(double t) { return round(t); }   /* C's round: half away from zero */

static uint64_t splitmix(uint64_t* s) {
  uint64_t z = (*s += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

/* 3: one (v, d) pair against the exact definition.  v / d in fp64 is the
 * correctly rounded quotient: within 2^-53 of the exact one, and exact
 * whenever the exact one is a tie (a tie has a short binary expansion). */
static int decision_ok(float v, float d) {
  const float rb = raise2(1.0f / d);
  const int got = byte_code(v, rb);
  const double t = (double)v / (double)d;
  const int want = (int)half_away(t);
  if (got == want) return 1;
  const double a = fabs(t), frac = a - floor(a);
  const int further = (t > 0 && got == want + 1) || (t < 0 && got == want - 1);
  return further && frac < 0.5 && 0.5 - frac <= 0x1p-21 * a + 0x1p-50;
}

int main(void) {
  /* 1: exhaustive byte identity over every |p| <= 128 */
  long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (int64_t k = 0; k <= 0x43000000ll; ++k) {
    for (int sign = 0; sign < 2; ++sign) {
      const float p = f_of((uint32_t)k | (sign ? 0x80000000u : 0u));
      if (byte_code(p, 1.0f) != (int)(int8_t)((int)rint((double)p) & 0xff)) bad += 1;
    }
  }
  printf("byte identity: every |p| <= 128, %ld mismatches\n", bad);
  if (bad) return 1;

  /* 1: random products v * rb, |v * rb| < 128 */
  const long prods = 100000000l;
  bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (long i = 0; i < prods; ++i) {
    uint64_t st = (uint64_t)i * 0x9e3779b97f4a7c15ull + 7u;
    const uint64_t a = splitmix(&st), b = splitmix(&st);
    const float rb = f_of((uint32_t)((100 + (a % 54)) << 23) | (uint32_t)(a >> 41));
    const float pt = f_of((uint32_t)((110 + (b % 23)) << 23) | (uint32_t)(b >> 41));  /* 2^-17 <= |p| < 128 */
    float v = pt / rb;
    if (b & (1ull << 40)) v = -v;
    const double p = (double)v * (double)rb;     /* exact: 24 + 24 bits */
    if (fabs(p) >= 128.0) continue;
    if (byte_code(v, rb) != (int)(int8_t)((int)rint(p) & 0xff)) bad += 1;
  }
  printf("byte identity random: %ld products, %ld mismatches\n", prods, bad);
  if (bad) return 1;

  /* 2: bias over every mantissa of one binade */
  bad = 0;
  double worst = 0.0, least = 1.0;
#pragma omp parallel for reduction(+ : bad) reduction(max : worst) reduction(min : least) schedule(static)
  for (uint32_t m = 0; m < (1u << 23); ++m) {
    const float d = f_of(0x3f800000u | m);       /* [1, 2) */
    const float rb = raise2(1.0f / d);
    const double e = (double)rb * (double)d - 1.0; /* exact */
    if (!(e > 0.0) || e > 0x1p-22 + 0x1p-24) bad += 1;
    if (e > worst) worst = e;
    if (e < least) least = e;
  }
  printf("bias: 2^23 scales, rb*d - 1 in [%a, %a], %ld outside (0, 2^-22 + 2^-24]\n", least, worst, bad);
  if (bad) return 1;

  /* 3: exact ties n + 1/2 at many scales: always away from zero */
  bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (int i = 0; i < 20000; ++i) {
    uint64_t st = (uint64_t)i * 0x2545f4914f6cdd1dull + 99u;
    const uint64_t a = splitmix(&st);
    /* d with few mantissa bits, so (n + 1/2) * d is exact in fp32 */
    const float d = f_of((uint32_t)((27 + (a % 200)) << 23) | (uint32_t)((a >> 20) & 0x7f0000u));
    for (int n = 0; n < 127; ++n) {
      const float v = (float)(n + 0.5) * d;
      if ((double)v != (n + 0.5) * (double)d) continue;   /* not exact: not a tie */
      if (byte_code(v, raise2(1.0f / d)) != n + 1) bad += 1;
      if (byte_code(-v, raise2(1.0f / d)) != -(n + 1)) bad += 1;
    }
  }
  printf("ties: 20000 scales x 127 half-integers x 2 signs, %ld not away from zero\n", bad);
  if (bad) return 1;

  /* 3: random pairs against the exact definition */
  const long pairs = 200000000l;
  bad = 0;
  long off = 0;
#pragma omp parallel for reduction(+ : bad, off) schedule(static)
  for (long i = 0; i < pairs; ++i) {
    uint64_t st = (uint64_t)i * 0x632be59bd9b4e019ull + 12345u;
    const uint64_t a = splitmix(&st), b = splitmix(&st);
    const float d = f_of((uint32_t)((27 + (a % 200)) << 23) | (uint32_t)(a >> 41));
    const float qt = f_of((uint32_t)((118 + (b % 15)) << 23) | (uint32_t)(b >> 41));  /* 2^-9 <= |v/d| < 128 */
    float v = qt * d;
    if (b & (1ull << 40)) v = -v;
    if (fabs((double)v / (double)d) > 127.0) continue;
    if (!decision_ok(v, d)) bad += 1;
    if (byte_code(v, raise2(1.0f / d)) != (int)half_away((double)v / (double)d)) off += 1;
  }
  printf("decision random: %ld pairs, %ld off the definition away from a boundary, %ld at a boundary\n", pairs,
         bad, off);
  return bad != 0;
}
