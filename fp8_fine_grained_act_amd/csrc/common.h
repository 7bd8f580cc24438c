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

// x / s is evaluated as q = fma(x, r, x * rl) with r = 1/s correctly rounded
// and rl = fl32(fma(-s, r, 1) * r) its low part: 1 - s*r is exact in binary32
// for the correctly rounded reciprocal, so r + rl carries 1/s to about 2^-48
// relative, and the fma rounds x*(r + rl) once.  That is not a correctly
// rounded quotient for every binary32 x, but x here is a bf16 value: an
// exhaustive host check over every pair of bf16 values (amax, |x| <= amax)
// shows that it gives the same E4M3 code as the IEEE quotient, and never
// exceeds 464.  Tiles whose amax (bf16 bits, sign cleared) is below
// kTinyAmaxBits (2^-64) run the same two operations on x * 2^64 and
// s * 2^64: both products are exact (s may be subnormal, s * 2^64 is normal),
// the quotient is unchanged, and 1 / (s * 2^64) is finite; the same host
// check covers every pair of that range.  A zero tile has s = r = rl = 0,
// which yields q = 0.
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

// lane-wise max of two pairs of 16-bit unsigned values (one v_pk_max_u16)
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// max of the two bf16 magnitudes held in one dword (sign bits cleared)
__device__ __forceinline__ uint32_t absmax_pair(uint32_t x) {
  uint32_t a = x & 0x7FFF7FFFu;
  return max(a & 0xFFFFu, a >> 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

constexpr float kTinyScale = 0x1p64f;

// Per-group quantization constants derived from the group's amax (bf16 bits).
struct GroupScale {
  float s;     // dequantization scale amax / 448 (IEEE division), the stored scale
  float d;     // divisor: s, or s * 2^64 for a tiny tile
  float r;     // 1 / d correctly rounded (0 for an all-zero tile)
  float rl;    // low part of 1 / d: fl32(fma(-d, r, 1) * r) (0 for an all-zero tile)
  bool slow;   // tiny tile: the values are multiplied by 2^64 first
};

__device__ __forceinline__ GroupScale group_scale(uint32_t amax_bits) {
  GroupScale g;
  const float amax = __uint_as_float(amax_bits << 16);
  g.s = amax / kE4M3Max;
  g.slow = amax_bits < kTinyAmaxBits;
  g.d = g.slow ? g.s * kTinyScale : g.s;
  g.r = g.d == 0.0f ? 0.0f : 1.0f / g.d;
  g.rl = __builtin_fmaf(-g.d, g.r, 1.0f) * g.r;
  return g;
}

// Quantize four bf16 values (two dwords, element 0 in the low half of x01)
// into four E4M3 codes packed little-endian in one dword.  SLOW: tiny tile,
// the magnitudes are scaled by 2^64 first.  No clamp is needed before the
// E4M3 conversion: |x| <= amax keeps the quotient at most 448 * (1 + 2^-7)
// even for a subnormal s (a few ulp above 448 otherwise), and
// v_cvt_pk_fp8_f32 rounds every binary32 value in (448, 464] to 448 (0x7E)
// under round-to-nearest-even (checked on gfx950 for all of them, both signs).
//
// The magnitudes come from the abs source modifier of the instructions that
// first read them (no masking of the packed words), the signs from the bf16
// sign bits; the first conversion's upper half is a placeholder (x01) that
// the second conversion overwrites.
template <bool SLOW>
__device__ __forceinline__ uint32_t quant4_path(uint32_t x01, uint32_t x23, const GroupScale& g) {
  const float a[4] = {bf16_lo(x01), bf16_hi(x01), bf16_lo(x23), bf16_hi(x23)};
  float qv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float ai = SLOW ? __builtin_fabsf(a[i]) * kTinyScale : __builtin_fabsf(a[i]);
    qv[i] = __builtin_fmaf(ai, g.r, ai * g.rl);
  }
  int d = __builtin_amdgcn_cvt_pk_fp8_f32(qv[0], qv[1], (int)x01, false);
  d = __builtin_amdgcn_cvt_pk_fp8_f32(qv[2], qv[3], d, true);
  // sign bits: byte 1 and byte 3 of each bf16 pair carry them in bit 7
  const uint32_t hi_bytes = __builtin_amdgcn_perm(x23, x01, 0x07050301u);
  return (uint32_t)d | (hi_bytes & 0x80808080u);
}

__device__ __forceinline__ uint32_t quant4(uint32_t x01, uint32_t x23, const GroupScale& g) {
  return g.slow ? quant4_path<true>(x01, x23, g) : quant4_path<false>(x01, x23, g);
}

// Codes of 2*N bf16 values held in N dwords (in order) -> N/2 code dwords.
// One branch on the group's path for the whole run.
template <int N>
__device__ __forceinline__ void quant_run(const uint32_t* in, uint32_t* out, const GroupScale& g) {
  static_assert(N % 2 == 0, "pairs of dwords");
  if (g.slow) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) out[i] = quant4_path<true>(in[2 * i], in[2 * i + 1], g);
  } else {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) out[i] = quant4_path<false>(in[2 * i], in[2 * i + 1], g);
  }
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---- streaming (non-temporal) 16-byte loads and stores ----------------------
// For data touched once per kernel (a dispatch payload written far larger than
// the caches, expert rows gathered once): the accesses carry the non-temporal
// hint, so they do not displace other lines in the caches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_nt(void* p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_nt(void* p, uint2 v) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}

// ---- buffer copies straight into LDS, and vmcnt waits ---------------------
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer access, gfx9 family

typedef __attribute__((address_space(3))) void lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t nb = bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFLL ? 0xFFFFFFFFu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nb, kRsrcWord3);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t*)lds, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t*)lds, 4, (int)voff, (int)soff, 0, 0);
}

// s_waitcnt with only a vmcnt limit (expcnt, lgkmcnt left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
// wave-uniform runtime limit: a chain of scalar compares picks the immediate
template <int N>
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if (n >= N) {
    wait_vmcnt<N>();
  } else if constexpr (N > 0) {
    wait_vmcnt_le<N - 1>(n);
  }
}
__device__ __forceinline__ void wait_vmcnt_dyn(int n) { wait_vmcnt_le<47>(n); }

}  // namespace fp8bs
