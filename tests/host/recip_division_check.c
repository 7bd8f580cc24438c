/*
 * Host check of the quantizer's division identity (used by the HIP kernels):
 * for every pair of positive bf16 values (amax, x) with x <= amax and
 * amax >= 2^-64 (tiles below that use IEEE division), with s = fl32(amax/448)
 * and r = fl32(1/s), the correction step
 *     q0 = x*r;  e = fma(-q0, s, x);  q = fma(e, r, q0)
 * must give the same E4M3 code (round to nearest even, saturating at 448) as
 * the IEEE binary32 quotient x/s.  Negative x is covered by symmetry: the
 * kernels quantize |x| and restore the sign bit afterwards.
 * Exit status 0 when every pair agrees; prints the counts.
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

int main(int argc, char** argv) {
  uint32_t tiny_bits = argc > 1 ? (uint32_t)strtoul(argv[1], 0, 0) : 0x1F80u;
  long long pairs = 0, bad = 0;
  for (uint32_t ab = tiny_bits; ab < 0x7F80; ++ab) {
    float amax = from_bf16(ab);
    float s = amax / 448.0f;
    float r = 1.0f / s;
    for (uint32_t xb = 0; xb <= ab; ++xb) {
      float x = from_bf16(xb);
      float q0 = x * r;
      float e = fmaf(-q0, s, x);
      float q = fmaf(e, r, q0);
      if (q > 448.0f) q = 448.0f;
      float ref = x / s;
      ++pairs;
      if (e4m3(q) != e4m3(ref)) {
        if (bad < 5) printf("mismatch amax=%a x=%a q=%a ieee=%a\n", amax, x, q, ref);
        ++bad;
      }
    }
  }
  printf("pairs=%lld mismatches=%lld (amax >= bf16 0x%04x)\n", pairs, bad, tiny_bits);
  return bad != 0;
}
