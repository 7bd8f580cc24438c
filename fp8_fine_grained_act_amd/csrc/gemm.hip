// Block-scaled FP8 GEMMs on gfx950 MFMA, and their C-ABI entry points.
//
// The pages ("DeepSeek-V3 技术报告深度解读", section 3) run the forward, the
// activation-gradient and the weight-gradient GEMM in FP8, with activation
// scales per 1x128 tile and weight scales per 128x128 block, and promote the
// partial sums to FP32 after every 128 elements of the contraction.  On gfx950
// one v_mfma_f32_16x16x128_f8f6f4 contracts exactly one 128-long K block of a
// 16x16 output tile into fresh FP32 registers, so the promotion is the scale
// step itself:  acc += (sa * sb) * P_kb  (one FP32 FMA per output element per
// K block), with P_kb the MFMA result for that block.
//
// Tiling: 128x128 output tile per 256-thread block (4 waves, 2x2, each wave
// 64x64 = 4x4 MFMA tiles), K staged through LDS in 128-deep slabs, two slabs
// in flight (the next slab's global loads overlap this slab's MFMAs).
// Operand roles: MFMA src0 carries B rows (output columns n), src1 carries A
// rows (output rows m), so each lane ends with one output row and four
// consecutive output columns -- one 8-byte (bf16) or 16-byte (f32) store.
// LDS rows are 128 bytes (one K slab of one matrix row); 16-byte chunks are
// XOR-swizzled with the row index so fragment reads and slab writes spread
// over the banks.

#include "common.h"
#include "launch.h"

namespace fp8bs {

enum GemmMode : int { kFprop = 0, kDgrad = 1, kWgrad = 2, kGrouped = 3 };

struct GemmArgs {
  const uint8_t* qa;
  const float* sa;
  const uint8_t* qb;
  const float* sb;
  void* c;
  int64_t ldc;
  int64_t m, n, k;
  const int32_t* seg;
  int64_t num_experts;
  int64_t tiles_n;
  int accumulate;
};

constexpr int BM = 128, BN = 128, BK = 128;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

// 4x4 byte transpose: rows r0..r3 (4 bytes each) -> column dwords o0..o3,
// o_j = (r0.b_j, r1.b_j, r2.b_j, r3.b_j).
__device__ __forceinline__ void transpose4x4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                             uint32_t& o0, uint32_t& o1, uint32_t& o2, uint32_t& o3) {
  uint32_t t0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
  uint32_t t1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
  uint32_t t2 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
  uint32_t t3 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
  o0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  o1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  o2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  o3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int MODE>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, g = lane >> 4;

  const int64_t tile = blockIdx.x;
  const int64_t tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t M = p.m, N = p.n, K = p.k;
  const int nkb = (int)(K / BK);

  const uint8_t* qb = p.qb;
  const float* sb = p.sb;
  if (MODE == kGrouped) {
    // expert whose segment holds row m0: the largest e with seg[e] <= m0
    int lo = 0, hi = (int)p.num_experts;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if ((int64_t)p.seg[mid] <= m0) lo = mid; else hi = mid - 1;
    }
    lo = min(lo, (int)p.num_experts - 1);
    qb += (int64_t)lo * N * K;
    sb += (int64_t)lo * (N / BN) * nkb;
  }

  // ---- global -> register staging of one K slab ---------------------------
  const int lr = tid >> 3, lch = tid & 7;      // row (0..31, +32p) and 16-byte chunk
  uint4 ra[4], rb[4];

  auto load_slab = [&](int kb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = m0 + lr + 32 * q;
      ra[q] = make_uint4(0, 0, 0, 0);
      if (row < M) ra[q] = *reinterpret_cast<const uint4*>(p.qa + row * K + (int64_t)kb * BK + lch * 16);
    }
    if (MODE == kDgrad) {
      // B is [K, N]: rows 4*lr .. 4*lr+3 of the slab, columns n0 + 16*lch .. +16
#pragma unroll
      for (int q = 0; q < 4; ++q)
        rb[q] = *reinterpret_cast<const uint4*>(qb + ((int64_t)kb * BK + 4 * lr + q) * N + n0 + 16 * lch);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = n0 + lr + 32 * q;
        rb[q] = make_uint4(0, 0, 0, 0);
        if (row < N) rb[q] = *reinterpret_cast<const uint4*>(qb + row * K + (int64_t)kb * BK + lch * 16);
      }
    }
  };

  auto store_slab = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = lr + 32 * q;
      *reinterpret_cast<uint4*>(&As[buf][swz(r, lch)]) = ra[q];
    }
    if (MODE == kDgrad) {
      // transpose 4 (k) x 16 (n) bytes into 16 rows n holding 4 consecutive k
      const int kofs = 4 * lr;                 // k offset within the slab
      const int kchunk = kofs >> 4, kin = kofs & 15;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t o[4];
        transpose4x4(u4get(rb[0], d), u4get(rb[1], d), u4get(rb[2], d), u4get(rb[3], d), o[0], o[1],
                     o[2], o[3]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int nr = 16 * lch + 4 * d + j;
          *reinterpret_cast<uint32_t*>(&Bs[buf][swz(nr, kchunk) + kin]) = o[j];
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = lr + 32 * q;
        *reinterpret_cast<uint4*>(&Bs[buf][swz(r, lch)]) = rb[q];
      }
    }
  };

  // ---- scales of one K block ----------------------------------------------
  float wa[4];            // activation scale of this lane's output row, per m-subtile
  float wb[4][4];         // weight-gradient: scale of each of this lane's 16 output columns
  float wbs = 0.0f;       // forward / dgrad / grouped: the tile's single weight-block scale
  float na[4], nb[4][4], nbs = 0.0f;

  auto load_scales = [&](int kb, float (&a)[4], float (&b)[4][4], float& bs) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = m0 + 64 * wm + 16 * j + l16;
      a[j] = row < M ? p.sa[row * nkb + kb] : 0.0f;
    }
    if (MODE == kWgrad) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t col = n0 + 64 * wn + 16 * i + 4 * g + v;
          b[i][v] = col < N ? sb[col * nkb + kb] : 0.0f;
        }
    } else if (MODE == kDgrad) {
      bs = sb[(int64_t)kb * (N / BN) + tn];
    } else {
      bs = sb[tn * nkb + kb];
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  load_slab(0);
  load_scales(0, wa, wb, wbs);
  store_slab(0);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) {
      load_slab(kb + 1);
      load_scales(kb + 1, na, nb, nbs);
    }

    v8i af[4], bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 64 * wm + 16 * j + l16;
      uint4 lo = *reinterpret_cast<const uint4*>(&As[buf][swz(r, 2 * g)]);
      uint4 hi = *reinterpret_cast<const uint4*>(&As[buf][swz(r, 2 * g + 1)]);
      af[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 64 * wn + 16 * i + l16;
      uint4 lo = *reinterpret_cast<const uint4*>(&Bs[buf][swz(r, 2 * g)]);
      uint4 hi = *reinterpret_cast<const uint4*>(&Bs[buf][swz(r, 2 * g + 1)]);
      bf[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[i], af[j], zero, 0, 0, 0, 0, 0, 0);
        if (MODE == kWgrad) {
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(wa[j] * wb[i][v], P[v], acc[i][j][v]);
        } else {
          const float w = wa[j] * wbs;
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(w, P[v], acc[i][j][v]);
        }
      }
    }

    if (more) {
      store_slab(buf ^ 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) wa[j] = na[j];
      if (MODE == kWgrad) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) wb[i][v] = nb[i][v];
      } else {
        wbs = nbs;
      }
    }
    __syncthreads();
  }

  // ---- epilogue --------------------------------------------------------------
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t row = m0 + 64 * wm + 16 * j + l16;
    if (row >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t col = n0 + 64 * wn + 16 * i + 4 * g;
      if (MODE == kWgrad) {
        if (col >= N) continue;
        float* dst = reinterpret_cast<float*>(p.c) + row * p.ldc + col;
        float4 o = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        if (p.accumulate) {
          float4 old = *reinterpret_cast<const float4*>(dst);
          o.x += old.x; o.y += old.y; o.z += old.z; o.w += old.w;
        }
        *reinterpret_cast<float4*>(dst) = o;
      } else {
        uint16_t* dst = reinterpret_cast<uint16_t*>(p.c) + row * p.ldc + col;
        uint2 o;
        o.x = f32_to_bf16_rne(acc[i][j][0]) | (f32_to_bf16_rne(acc[i][j][1]) << 16);
        o.y = f32_to_bf16_rne(acc[i][j][2]) | (f32_to_bf16_rne(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2*>(dst) = o;
      }
    }
  }
}

template <int MODE>
static int launch_gemm(const GemmArgs& a, int64_t tiles_m, hipStream_t s) {
  const int64_t grid = tiles_m * a.tiles_n;
  if (grid > kMaxGrid) return FP8BS_ERR_SHAPE;
  hipLaunchKernelGGL(gemm_kernel<MODE>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return launch_status();
}

}  // namespace fp8bs

using namespace fp8bs;

extern "C" int fp8bs_gemm(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb,
                          int64_t m, int64_t n, int64_t k, int b_layout, uint16_t* c, int64_t ldc,
                          void* stream) {
  if (!qa || !sa || !qb || !sb || !c) return FP8BS_ERR_NULL;
  if (b_layout != 0 && b_layout != 1) return FP8BS_ERR_FLAG;
  if (m <= 0 || n <= 0 || k <= 0 || n % BN || k % BK || ldc < n) return FP8BS_ERR_SHAPE;
  if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(c, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
      ldc % 8)
    return FP8BS_ERR_ALIGN;
  GemmArgs a{qa, sa, qb, sb, c, ldc, m, n, k, nullptr, 0, n / BN, 0};
  const int64_t tiles_m = (m + BM - 1) / BM;
  if (b_layout == 0) return launch_gemm<kFprop>(a, tiles_m, (hipStream_t)stream);
  return launch_gemm<kDgrad>(a, tiles_m, (hipStream_t)stream);
}

extern "C" int fp8bs_grouped_gemm(const uint8_t* qa, const float* sa, const int32_t* seg_offsets,
                                  int64_t num_experts, int64_t total_rows, const uint8_t* qb,
                                  const float* sb, int64_t n, int64_t k, uint16_t* c, void* stream) {
  if (!qa || !sa || !seg_offsets || !qb || !sb || !c) return FP8BS_ERR_NULL;
  if (num_experts < 1 || num_experts > 65536 || total_rows <= 0 || total_rows % BM || n <= 0 ||
      k <= 0 || n % BN || k % BK)
    return FP8BS_ERR_SHAPE;
  if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(c, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
      !aligned(seg_offsets, 4))
    return FP8BS_ERR_ALIGN;
  GemmArgs a{qa, sa, qb, sb, c, n, total_rows, n, k, seg_offsets, num_experts, n / BN, 0};
  return launch_gemm<kGrouped>(a, total_rows / BM, (hipStream_t)stream);
}

extern "C" int fp8bs_gemm_wgrad(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb,
                                int64_t m, int64_t n, int64_t t, float* c, int64_t ldc, int accumulate,
                                void* stream) {
  if (!qa || !sa || !qb || !sb || !c) return FP8BS_ERR_NULL;
  if (accumulate != 0 && accumulate != 1) return FP8BS_ERR_FLAG;
  if (m <= 0 || n <= 0 || t <= 0 || t % BK || n % 4 || ldc < n) return FP8BS_ERR_SHAPE;
  if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(c, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
      ldc % 4)
    return FP8BS_ERR_ALIGN;
  GemmArgs a{qa, sa, qb, sb, c, ldc, m, n, t, nullptr, 0, (n + BN - 1) / BN, accumulate};
  return launch_gemm<kWgrad>(a, (m + BM - 1) / BM, (hipStream_t)stream);
}
