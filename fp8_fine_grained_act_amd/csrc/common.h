// Shared device helpers for the fp8bs kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8bs.h"

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;           // scale-group length along the contraction
constexpr float kE4M3Max = 448.0f;

// Tiles whose amax (as bf16 bits, sign cleared) is below this take true IEEE
// division for x / s.  Above it, x / s is evaluated as q0 = x*r, e = fma(-q0, s, x),
// q = fma(e, r, q0) with r = 1/s correctly rounded (Markstein's correction step);
// an exhaustive host check over every pair of bf16 values (amax, |x| <= amax)
// shows that this gives the same E4M3 code as the IEEE quotient whenever
// amax >= 2^-104.  0x1F80 is 2^-64, far inside that range.
constexpr uint32_t kTinyAmaxBits = 0x1F80u;

// ---- cross-lane max inside a row of 16 lanes (DPP, no LDS traffic) ----------
// dpp controls: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_shuffle(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// max over aligned groups of 8 lanes
__device__ __forceinline__ uint32_t max8_u32(uint32_t v) {
  v = max(v, dpp_shuffle<0xB1>(v));
  v = max(v, dpp_shuffle<0x4E>(v));
  v = max(v, dpp_shuffle<0x141>(v));
  return v;
}

// max over the whole wavefront (64 lanes), result in every lane
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max8_u32(v);
  v = max(v, dpp_shuffle<0x140>(v));          // rows of 16
  v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

// max of the two bf16 magnitudes held in one dword (sign bits cleared)
__device__ __forceinline__ uint32_t absmax_pair(uint32_t x) {
  uint32_t a = x & 0x7FFF7FFFu;
  return max(a & 0xFFFFu, a >> 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// Per-group quantization constants derived from the group's amax (bf16 bits).
struct GroupScale {
  float s;     // dequantization scale amax / 448 (IEEE division)
  float r;     // 1 / s correctly rounded (0 when the slow path is taken)
  bool slow;   // amax tiny or zero: use IEEE division per element
};

__device__ __forceinline__ GroupScale group_scale(uint32_t amax_bits) {
  GroupScale g;
  float amax = __uint_as_float(amax_bits << 16);
  g.s = amax / kE4M3Max;
  g.slow = amax_bits < kTinyAmaxBits;
  g.r = g.slow ? 0.0f : 1.0f / g.s;
  return g;
}

// |x| / s as the binary32 quotient, clamped to 448 (values in (448, 464) round
// to 448 under RNE anyway; the quotient never exceeds 448 by more than a few ulp).
__device__ __forceinline__ float scaled_mag(float a, const GroupScale& g) {
  float q;
  if (!g.slow) {
    float q0 = a * g.r;
    float e = __builtin_fmaf(-q0, g.s, a);
    q = __builtin_fmaf(e, g.r, q0);
  } else {
    q = (g.s == 0.0f) ? 0.0f : a / g.s;
  }
  return __builtin_fminf(q, kE4M3Max);
}

// Quantize four bf16 values (two dwords, element 0 in the low half of x01)
// into four E4M3 codes packed little-endian in one dword.
__device__ __forceinline__ uint32_t quant4(uint32_t x01, uint32_t x23, const GroupScale& g) {
  uint32_t m01 = x01 & 0x7FFF7FFFu, m23 = x23 & 0x7FFF7FFFu;
  float q0 = scaled_mag(bf16_lo(m01), g);
  float q1 = scaled_mag(bf16_hi(m01), g);
  float q2 = scaled_mag(bf16_lo(m23), g);
  float q3 = scaled_mag(bf16_hi(m23), g);
  int d = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  d = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, d, true);
  // sign bits: byte 1 and byte 3 of each bf16 pair carry them in bit 7
  uint32_t hi_bytes = __builtin_amdgcn_perm(x23, x01, 0x07050301u);
  return (uint32_t)d | (hi_bytes & 0x80808080u);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace fp8bs
