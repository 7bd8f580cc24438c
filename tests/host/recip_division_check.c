/*
 * Host check of the quantizer's division identity (used by the HIP kernels).
 * For every pair of non-negative bf16 values (amax, x) with x <= amax and
 * s = fl32(amax/448):
 *   amax >= threshold (2^-64 in the kernels): d = s, r = fl32(1/d), a = x;
 *   amax <  threshold (tiny tiles):           d = s * 2^64, r = fl32(1/d)
 *                                             (0 when d == 0), a = x * 2^64;
 * with rl = fl32(fma(-d, r, 1) * r), the low part of 1/d, the quotient
 *     q = fma(a, r, fl32(a * rl))
 * must give the same E4M3 code (round to nearest even, saturating) as the
 * IEEE binary32 quotient x/s, and q must not exceed 464 (the hardware
 * conversion rounds (448, 464] to 448; above that it would not saturate).
 * Negative x is covered by symmetry: the kernels quantize |x| and restore the
 * sign bit afterwards.  Exit status 0 when every pair agrees; prints counts.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bf16(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

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

static long long check_range(uint32_t lo, uint32_t hi, int tiny, long long* pairs) {
  long long bad = 0;
  for (uint32_t ab = lo; ab < hi; ++ab) {
    float amax = from_bf16(ab);
    float s = amax / 448.0f;
    float d = tiny ? s * 0x1p64f : s;
    float r = d == 0.0f ? 0.0f : 1.0f / d;
    float rl = fmaf(-d, r, 1.0f) * r;
    for (uint32_t xb = 0; xb <= ab; ++xb) {
      float x = from_bf16(xb);
      float a = tiny ? x * 0x1p64f : x;
      float t = a * rl;
      float q = fmaf(a, r, t);
      float ref = s == 0.0f ? 0.0f : x / s;
      ++*pairs;
      if (e4m3(q) != e4m3(ref) || q > 464.0f) {
        if (bad < 5) printf("mismatch amax=%a x=%a q=%a ieee=%a\n", amax, x, q, ref);
        ++bad;
      }
    }
  }
  return bad;
}

int main(int argc, char** argv) {
  uint32_t tiny_bits = argc > 1 ? (uint32_t)strtoul(argv[1], 0, 0) : 0x1F80u;
  long long pairs_tiny = 0, pairs = 0;
  long long bad_tiny = check_range(0, tiny_bits, 1, &pairs_tiny);
  long long bad = check_range(tiny_bits, 0x7F80, 0, &pairs);
  printf("tiny: pairs=%lld mismatches=%lld (amax < bf16 0x%04x, scaled by 2^64)\n", pairs_tiny, bad_tiny, tiny_bits);
  printf("pairs=%lld mismatches=%lld (amax >= bf16 0x%04x)\n", pairs, bad, tiny_bits);
  return (bad != 0 || bad_tiny != 0);
}
