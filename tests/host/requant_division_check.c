/*
 * Host check of the reciprocal-and-correction quotient used by the re-tiling
 * kernel, whose numerators are arbitrary binary32 values (x_hat = fl32(s *
 * dec(q)) is not a bf16 value, so the exhaustive bf16 check does not cover it).
 * For a divisor s = fl32(amax/448) and a signed numerator x, |x| <= amax:
 *   amax >= 2^-64:  d = s,          x' = x
 *   amax <  2^-64:  d = s * 2^64,   x' = x * 2^64   (both exact)
 *   r = fl32(1/d) (0 when d == 0), q0 = x'*r, e = fma(q0, d, -x'), q = fma(-e, r, q0)
 * must give the same E4M3 code (nearest even, saturating, sign bit from the
 * sign of x, also for -0) as the IEEE binary32 quotient |x|/s (0 when s == 0)
 * with x's sign, and |q| must not exceed 464.  (This is
 * Markstein's correction: with r the correctly rounded reciprocal and q0
 * within one ulp of the quotient, q is the correctly rounded quotient; the
 * scaling keeps e and r clear of underflow and overflow.)
 * Samples, per divisor: numerators placed within +-6 ulps of every E4M3
 * rounding boundary times s (where a one-ulp quotient error would change the
 * code), the divisor's own amax, and uniformly random numerators.  Divisors:
 * amax over every binade of binary32 (normal and subnormal) with random
 * significands.  argv[1] = number of amax samples per binade.
 * Exit status 0 when every sample agrees; prints counts.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float fromb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* E4M3 (OCP "fn") code of a non-negative binary32 value: RNE, saturating */
static uint32_t e4m3(float v) {
  uint32_t u = bits(v), E = u >> 23;
  if (E == 0) return 0;
  uint64_t sig = (1u << 23) | (u & 0x7FFFFF);
  int e = (int)E - 127, qe = (e > -6 ? e : -6) - 3, sh = qe - (e - 23);
  uint64_t k;
  if (sh >= 64) k = 0;
  else {
    k = sig >> sh;
    uint64_t rem = sig & ((1ull << sh) - 1), half = 1ull << (sh - 1);
    if (rem > half || (rem == half && (k & 1))) k++;
  }
  long c = (qe == -9) ? (long)k : ((long)(e + 7) << 3) + (long)k - 8;
  return c > 0x7E ? 0x7E : (uint32_t)c;
}

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return rng; }

static long long bad = 0, total = 0;

/* signed code: the sign bit of v, then the code of |v| */
static uint32_t e4m3_signed(float v) { return ((bits(v) >> 24) & 0x80u) | e4m3(fabsf(v)); }

static void check1(float amax, float x) {
  const float s = amax / 448.0f;
  const int tiny = amax < 0x1p-64f;
  const float d = tiny ? s * 0x1p64f : s;
  const float r = d == 0.0f ? 0.0f : 1.0f / d;
  const float xp = tiny ? x * 0x1p64f : x;
  const float q0 = xp * r;
  const float e = fmaf(q0, d, -xp);
  const float q = fmaf(-e, r, q0);
  const float ref = s == 0.0f ? copysignf(0.0f, x) : copysignf(fabsf(x) / s, x);
  ++total;
  if (e4m3_signed(q) != e4m3_signed(ref) || fabsf(q) > 464.0f) {
    if (bad < 8) printf("mismatch amax=%a x=%a q=%a ieee=%a\n", amax, x, q, ref);
    ++bad;
  }
}

/* both signs of a magnitude 0 <= a <= amax */
static void check(float amax, float a) {
  check1(amax, a);
  check1(amax, -a);
}

int main(int argc, char** argv) {
  const int per_binade = argc > 1 ? atoi(argv[1]) : 64;
  /* E4M3 rounding boundaries (midpoints between consecutive finite values, and 464) */
  float bound[300];
  int nb = 0;
  float prev = 0.0f;
  for (uint32_t c = 1; c <= 0x7E; ++c) {
    const uint32_t E = c >> 3, M = c & 7;
    const float v = E == 0 ? ldexpf((float)M, -9) : ldexpf((float)(8 + M), (int)E - 10);
    bound[nb++] = 0.5f * (prev + v);
    prev = v;
  }
  bound[nb++] = 464.0f;
  for (int E = 0; E < 255; ++E) {
    for (int k = 0; k < per_binade; ++k) {
      const uint32_t mant = (k == 0) ? 0 : (k == 1 ? 0x7FFFFF : (uint32_t)(next() & 0x7FFFFF));
      const float amax = fromb(((uint32_t)E << 23) | mant);
      if (amax == 0.0f) continue;
      const float s = amax / 448.0f;
      check(amax, amax);
      check(amax, 0.0f);                           /* +0 and -0 */
      for (int i = 0; i < nb; ++i) {
        const float c = bound[i] * s;              /* near a rounding boundary of the quotient */
        if (!(c > 0.0f)) continue;
        const uint32_t cb = bits(c);
        for (int du = -6; du <= 6; ++du) {
          const float a = fromb(cb + du);
          if (a >= 0.0f && a <= amax) check(amax, a);
        }
      }
      for (int i = 0; i < 64; ++i) {
        const float a = fromb((uint32_t)(next() % (bits(amax) + 1u)));
        check(amax, a);
      }
    }
  }
  printf("samples=%lld mismatches=%lld\n", total, bad);
  return bad != 0;
}
