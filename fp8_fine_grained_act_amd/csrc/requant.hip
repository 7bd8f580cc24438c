// Re-tiling of a cached FP8 activation along its rows (gfx950).
//
// Activations are kept in FP8 between the forward and the backward pass
// (deepseek.csdn.net page, section 二(四) "FP8 低精度训练"; qqstock.cn page,
// FP8 section).  The cached form of x [T, C] is the forward's own 1x128 tiles
// along C; the weight gradient contracts over the tokens
// ("DeepSeek-V3 技术报告深度解读", section 3), so it needs tiles along T.
// This kernel makes them from the cache alone:
//   x_hat[t, c] = fl32(s[t, c/128] * dec(q[t, c]))        (one binary32 multiply)
//   tiles of x_hat^T: amax over 128 tokens, s' = fl32(amax / 448),
//   code = E4M3 nearest-even of fl32(|x_hat| / s') with the sign of x_hat.
// The quotient uses the reciprocal and one correction step on the signed value
// (r = fl32(1/d), q0 = x*r, e = fma(q0, d, -x), q = fma(-e, r, q0): Markstein's
// correction, which yields the correctly rounded quotient when r is the
// correctly rounded reciprocal; by the sign symmetry of rounding |q| is that
// of |x|, and the sign, also of a zero, is x's), with numerator and divisor
// scaled by 2^64 when amax < 2^-64 so that nothing underflows.  x_hat is an arbitrary binary32 value, so the
// exhaustive bf16 check of the other quantizers does not cover it; a host
// check (tests/host/requant_division_check.c) compares the E4M3 codes with
// those of the IEEE quotient for numerators within a few ulps of every E4M3
// rounding boundary, for divisors in every binade.
//
// One 256-thread workgroup per 128 x 128 square.  The square's codes (16 KB,
// read once: non-temporal loads, 19.6 -> 18.3 us on 4096 x 7168) are staged
// in LDS; lane (g, j) (g = tid / 8, j = tid % 8) then owns columns
// 4g..4g+3 and tokens 16j..16j+15: one 4-byte LDS read per token gives its
// four columns (two packed decodes), a column's amax is a max over the 8
// lanes of the group (DPP), and for each column the group's 8 lanes store its
// whole 128-byte output row, one 16-byte piece each, in one instruction.  Dword d of staged row r
// (32 dwords) sits at d ^ (4 * ((r / 16) % 8)), which keeps each 16-byte
// chunk whole and spreads the 8 rows a group reads (16 apart, so all on the
// same half of the 64 banks) over the dwords: a read instruction touches each
// bank at most twice.  (Two passes per read: the square's global traffic,
// not LDS, bounds the kernel.)

#include "common.h"
#include "launch.h"

namespace fp8bs {

__device__ __forceinline__ int req_dw(int r, int d) { return r * 32 + (d ^ (((r >> 4) & 7) << 2)); }
__device__ __forceinline__ int req_rs(int r) { return r + (r >> 6); }   // token scales, 2 banks apart per half

constexpr float kReqTinyAmax = 0x1p-64f;

typedef float v2f __attribute__((ext_vector_type(2)));

// Codes of four signed values x (tokens in order, packed little-endian).  The
// quotient x / d takes the reciprocal and one correction on the signed value:
// q0 = x r, e = fma(q0, d, -x), q = fma(-e, r, q0).  Round-to-nearest and fma
// are symmetric in sign, so |q| equals the quotient of |x| step for step, and
// this order keeps the sign of a zero x (-0 gives -0, so code 0x80);
// v_cvt_pk_fp8_f32 then codes the sign with the magnitude.  SLOW: tiny tiles,
// x scaled by up (2^64, or 1 for the other columns of the wave) first.
template <bool SLOW>
__device__ __forceinline__ uint32_t requant_code4(const float* x, float up, float d, float rcp) {
  float qv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float xv = SLOW ? x[e] * up : x[e];
    const float q0 = xv * rcp;
    const float err = __builtin_fmaf(q0, d, -xv);
    qv[e] = __builtin_fmaf(-err, rcp, q0);
  }
  int wv = __builtin_amdgcn_cvt_pk_fp8_f32(qv[0], qv[1], 0, false);
  wv = __builtin_amdgcn_cvt_pk_fp8_f32(qv[2], qv[3], wv, true);
  return (uint32_t)wv;
}

__global__ __launch_bounds__(256) void requant_t_kernel(const uint8_t* __restrict__ q, int64_t ldq,
                                                        const float* __restrict__ s, int64_t rows,
                                                        int64_t cols, uint8_t* __restrict__ qt, int64_t ldqt,
                                                        float* __restrict__ st) {
  __shared__ __align__(16) uint32_t tile[128 * 32];
  __shared__ float rs[130];
  const int64_t cblocks = cols / kGroup, tblocks = rows / kGroup;
  const int64_t tb = (int64_t)blockIdx.x / cblocks, cb = (int64_t)blockIdx.x - tb * cblocks;
  const int64_t t0 = tb * kGroup, c0 = cb * kGroup;
  const int tid = threadIdx.x;

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + 256 * j, r = i >> 3, ch = i & 7;
    const uint4 v = load_nt(q + (t0 + r) * ldq + c0 + 16 * ch);
    *reinterpret_cast<uint4*>(tile + req_dw(r, 4 * ch)) = v;
  }
  if (tid < 128) rs[req_rs(tid)] = s[(t0 + tid) * cblocks + cb];
  __syncthreads();

  const int g = tid >> 3, j = tid & 7;
  float xh[4][16];
  float am[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * j + i;
    const int w = (int)tile[req_dw(r, g)];
    const float sc = rs[req_rs(r)];
    const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    const float dv[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      xh[b][i] = dv[b] * sc;
      am[b] = fmaxf(am[b], fabsf(xh[b][i]));
    }
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    // amax over the group's 8 lanes (non-negative floats order as their bits)
    const float amax = __uint_as_float(max8_u32(__float_as_uint(am[b])));
    const float sp = amax / kE4M3Max;
    const bool tiny = amax < kReqTinyAmax;
    const float d = tiny ? sp * kTinyScale : sp;       // exact scaling of numerator and divisor
    const float rcp = d == 0.0f ? 0.0f : 1.0f / d;
    uint32_t packed[4];
    if (__ballot(tiny)) {                               // a tiny column anywhere in the wave
      const float up = tiny ? kTinyScale : 1.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) packed[k] = requant_code4<true>(&xh[b][4 * k], up, d, rcp);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) packed[k] = requant_code4<false>(&xh[b][4 * k], 1.0f, d, rcp);
    }
    const int64_t c = c0 + 4 * g + b;
    *reinterpret_cast<uint4*>(qt + c * ldqt + t0 + 16 * j) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    if (j == 0) st[c * tblocks + tb] = sp;
  }
}

}  // namespace fp8bs

using namespace fp8bs;

extern "C" int fp8bs_requantize_act_1x128_t(const uint8_t* q, const float* scales, int64_t rows, int64_t cols,
                                            int64_t ldq, uint8_t* qt, int64_t ldqt, float* scales_t,
                                            void* stream) {
  if (!q || !scales || !qt || !scales_t) return FP8BS_ERR_NULL;
  if (rows <= 0 || cols <= 0 || rows % kGroup || cols % kGroup || ldq < cols || ldqt < rows)
    return FP8BS_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(qt, 16) || !aligned(scales, 4) || !aligned(scales_t, 4) || ldq % 16 ||
      ldqt % 16)
    return FP8BS_ERR_ALIGN;
  const int64_t grid = (rows / kGroup) * (cols / kGroup);
  if (grid > kMaxGrid) return FP8BS_ERR_SHAPE;
  hipLaunchKernelGGL(requant_t_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, q, ldq, scales,
                     rows, cols, qt, ldqt, scales_t);
  return launch_status();
}
