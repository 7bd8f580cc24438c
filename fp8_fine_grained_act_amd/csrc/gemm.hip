// Block-scaled FP8 GEMMs on gfx950 MFMA, and their C-ABI entry points.
//
// The pages ("DeepSeek-V3 技术报告深度解读", section 3) run the forward, the
// activation-gradient and the weight-gradient GEMM in FP8, with activation
// scales per 1x128 tile and weight scales per 128x128 block, and promote the
// partial sums to FP32 after every 128 elements of the contraction.  On gfx950
// one v_mfma_f32_16x16x128_f8f6f4 contracts exactly one 128-long K block of a
// 16x16 output tile into fresh FP32 registers, so the promotion is the scale
// step itself:  acc += (sa * sb) * P_kb  (one FP32 FMA per output element per
// K block), with P_kb the MFMA result for that block.  Inside the block the
// matrix core does its own summation of the 128 products (not exact when the
// products span many binades); the FP32 promotion bounds how far that error
// can accumulate, as on the pages' hardware.
//
// Structure of one workgroup (4 waves in a 2x2 grid, each wave a
// (BM/2) x (BN/2) patch of 16x16 MFMA tiles):
//   * K is walked in 128-deep slabs.  A slab of A (BM rows x 128 bytes), of B
//     (BN rows x 128 bytes) and of the scales that go with it is copied from
//     memory straight into LDS with buffer_load ... lds (16 bytes per lane),
//     STAGES slabs in flight, so no VGPRs hold staged data and rows past the
//     matrix edge read as zero (buffer range check).
//   * LDS rows are 128 bytes; their 16-byte chunks are XOR-swizzled with the
//     row index (applied to the global address of the copy), so the fragment
//     reads (two ds_read_b128 per 16x128 operand) hit distinct banks.
//   * MFMA src0 carries B rows (output columns n), src1 carries A rows (output
//     rows m): each lane ends with one output row and four consecutive output
//     columns -- one 8-byte (bf16) or 16-byte (f32) store.
//   * dgrad reads the forward weight as stored ([K, N], N contiguous): its
//     slab is copied as is (LDS rows = k) and the MFMA fragments, which need 32
//     consecutive k per lane, are gathered with ds_read_b64_tr_b8 (gfx950's
//     transposing LDS read).  Within a 16-lane group that instruction hands
//     lane i byte (i mod 8) of the 8-byte words read by lanes (i div 8) + 2b,
//     b = 0..7; pointing even lanes at 8 consecutive k rows of columns n..n+7
//     and odd lanes at the same rows of columns n+8..n+15 leaves lane i with 8
//     consecutive k of column n + i.

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

constexpr int BK = 128;
constexpr int kThreads = 256;
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

// swizzled byte offset of 16-byte chunk `chunk` of LDS row `row`
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

// wait until at most n vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <int BM, int BN>
struct Smem {
  uint8_t a[BM * BK];
  uint8_t b[BN * BK];
  float sa[BM];
  float sb[BN];
};

template <int MODE, int BM, int BN, int STAGES>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void gemm_kernel(GemmArgs p) {
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile");
  constexpr int WM = BM / 2, WN = BN / 2;         // wave patch
  constexpr int TM = WM / 16, TN = WN / 16;       // MFMA tiles per wave
  constexpr int A_CP = BM * BK / (kThreads * 16); // 16-byte copies per thread per A slab
  constexpr int B_CP = BN * BK / (kThreads * 16);
  static_assert(A_CP * kThreads * 16 == BM * BK && B_CP * kThreads * 16 == BN * BK, "copy split");
  static_assert(BM == 128 && BN == 128, "staging split assumes a 128 x 128 tile");
  // vector-memory operations one wave issues per slab (waited on by count)
  constexpr int kSlabOps = A_CP + B_CP + 1;

  __shared__ __attribute__((aligned(16))) Smem<BM, BN> sm[STAGES];

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
    sb += (int64_t)lo * (N / 128) * nkb;
  }

  // ---- buffer resources (ranges clip ragged edges to zeros) ------------------
  const int64_t rows_a = M - m0 < BM ? M - m0 : BM;
  const int64_t rows_b = N - n0 < BN ? N - n0 : BN;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.qa + m0 * K, rows_a * K);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.sa + m0 * nkb, rows_a * nkb * 4);
  __amdgpu_buffer_rsrc_t rb, rsb;
  if (MODE == kDgrad) {
    rb = make_rsrc(qb + n0, K * N - n0);
    rsb = make_rsrc(sb, (K / 128) * (N / 128) * 4);
  } else if (MODE == kWgrad) {
    rb = make_rsrc(qb + n0 * K, rows_b * K);
    rsb = make_rsrc(sb + n0 * nkb, rows_b * nkb * 4);
  } else {
    rb = make_rsrc(qb + n0 * K, rows_b * K);
    rsb = make_rsrc(sb, (N / 128) * nkb * 4);
  }

  // per-thread copy offsets (without the K-block term), swizzle on the global side
  uint32_t aoff[A_CP], boff[B_CP];
#pragma unroll
  for (int i = 0; i < A_CP; ++i) {
    const int c = (i * 4 + wave) * 64 + lane;   // 16-byte chunk index inside the slab
    const int row = c >> 3, pc = c & 7;
    aoff[i] = (uint32_t)(row * K + ((pc ^ (row & 7)) << 4));
  }
#pragma unroll
  for (int i = 0; i < B_CP; ++i) {
    const int c = (i * 4 + wave) * 64 + lane;
    const int row = c >> 3, pc = c & 7;
    const int64_t ld = MODE == kDgrad ? N : K;      // dgrad: slab rows are k, ld = N
    boff[i] = (uint32_t)(row * ld + ((pc ^ (row & 7)) << 4));
  }

  auto issue_slab = [&](int kb, Smem<BM, BN>& s) {
    const uint32_t ks = (uint32_t)kb * BK;
#pragma unroll
    for (int i = 0; i < A_CP; ++i) dma16(ra, s.a + (i * 4 + wave) * 1024, aoff[i], ks);
    {
      const uint32_t kso = MODE == kDgrad ? ks * (uint32_t)N : ks;   // dgrad: K-block = 128 rows of [K, N]
#pragma unroll
      for (int i = 0; i < B_CP; ++i) dma16(rb, s.b + (i * 4 + wave) * 1024, boff[i], kso);
    }
    // scales of this K block: exactly one 4-byte-per-lane copy per wave, so every
    // wave has the same number of copies in flight per slab
    if (wave < 2) {
      dma4(rsa, s.sa + wave * 64, (uint32_t)((wave * 64 + lane) * nkb) * 4u, (uint32_t)kb * 4u);
    } else if (MODE == kWgrad) {
      const int wv = wave - 2;
      dma4(rsb, s.sb + wv * 64, (uint32_t)((wv * 64 + lane) * nkb) * 4u, (uint32_t)kb * 4u);
    } else {
      // the tile's single weight-block scale, broadcast to every lane's slot
      const uint32_t nb0 = (uint32_t)(n0 / 128);
      const uint32_t idx = MODE == kDgrad ? (uint32_t)kb * (uint32_t)(N / 128) + nb0
                                          : nb0 * (uint32_t)nkb + (uint32_t)kb;
      dma4(rsb, s.sb + (wave - 2) * 64, 0u, idx * 4u);
    }
  };

  v4f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Fragments of one slab: every LDS read of the slab happens here, before the
  // next slab's copies are issued, so the copies never wait behind these reads
  // and the MFMA phase below touches registers only.
  struct Frags {
    v8i af[TM], bf[TN];
    float wa[TM];
    v4f wb[TN];
  };
  auto load_frags = [&](const Smem<BM, BN>& s, Frags& f) {
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int r = WM * wm + 16 * j + l16;
      const uint4 lo = *reinterpret_cast<const uint4*>(&s.a[swz(r, 2 * g)]);
      const uint4 hi = *reinterpret_cast<const uint4*>(&s.a[swz(r, 2 * g + 1)]);
      f.af[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      if (MODE == kDgrad) {
        // rows of s.b are k; lane (g, l16) needs k = 32g .. 32g+31 of column WN*wn + 16i + l16
        const int col16 = (WN * wn + 16 * i) >> 4;       // 16-byte chunk of the columns
        const int half = (l16 & 1) << 3;                 // odd lanes: columns +8 .. +15
        v2i part[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 32 * g + 8 * q + (l16 >> 1);
          part[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) v2i*)(&s.b[swz(row, col16) + half]));
        }
        f.bf[i] = v8i{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
      } else {
        const int r = WN * wn + 16 * i + l16;
        const uint4 lo = *reinterpret_cast<const uint4*>(&s.b[swz(r, 2 * g)]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&s.b[swz(r, 2 * g + 1)]);
        f.bf[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) f.wa[j] = s.sa[WM * wm + 16 * j + l16];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      if (MODE == kWgrad) {
        f.wb[i] = *reinterpret_cast<const v4f*>(&s.sb[WN * wn + 16 * i + 4 * g]);
      } else {
        const float v = s.sb[0];
        f.wb[i] = v4f{v, v, v, v};
      }
    }
  };

  auto mfma_phase = [&](const Frags& f) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.bf[i], f.af[j], zero, 0, 0, 0, 0, 0, 0);
        if (MODE == kWgrad) {
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(f.wa[j] * f.wb[i][v], P[v], acc[i][j][v]);
        } else {
          const float w = f.wa[j] * f.wb[i][0];
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(w, P[v], acc[i][j][v]);
        }
      }
    }
  };

  // ---- main loop: STAGES slabs in flight -------------------------------------
  // LDS hand-off: a wave waits for its own copies of the slab it is about to
  // read (vmcnt, counting only the newer slabs still allowed in flight) and for
  // its own LDS writes (lgkmcnt), then the workgroup barrier publishes every
  // wave's part.  The barrier also guarantees that the stage about to be
  // refilled is no longer being read.
  auto publish = [&](bool newer_in_flight) {
    if (newer_in_flight) wait_vmcnt<(STAGES - 2) * kSlabOps>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's ds_write done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nkb) issue_slab(s, sm[s]);

  for (int kb0 = 0; kb0 < nkb; kb0 += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      const int kb = kb0 + s;
      if (kb < nkb) {
        const int nxt = kb + STAGES - 1;
        const int ns = (s + STAGES - 1) % STAGES;
        publish(kb + STAGES - 2 < nkb);
        Frags f;
        load_frags(sm[s], f);
        if (nxt < nkb) issue_slab(nxt, sm[ns]);
        mfma_phase(f);
      }
    }
  }

  // ---- epilogue --------------------------------------------------------------
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int64_t row = m0 + WM * wm + 16 * j + l16;
    if (row >= M) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int64_t col = n0 + WN * wn + 16 * i + 4 * g;
      if (MODE == kWgrad) {
        if (col >= N) continue;
        float* dst = reinterpret_cast<float*>(p.c) + row * p.ldc + col;
        float4 o = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        if (p.accumulate) {
          const float4 old = *reinterpret_cast<const float4*>(dst);
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

template <int MODE, int BM, int BN, int STAGES>
static int launch_gemm(GemmArgs a, hipStream_t s) {
  a.tiles_n = (a.n + BN - 1) / BN;
  const int64_t tiles_m = (a.m + BM - 1) / BM;
  const int64_t grid = tiles_m * a.tiles_n;
  if (grid > kMaxGrid) return FP8BS_ERR_SHAPE;
  hipLaunchKernelGGL((gemm_kernel<MODE, BM, BN, STAGES>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return launch_status();
}

}  // namespace fp8bs

using namespace fp8bs;

// Offsets inside one operand are 32-bit (buffer addressing): a tile's rows of
// A or B, and the dgrad weight as a whole, must stay below 4 GiB.
static bool fits_u32(int64_t bytes) { return bytes < 0xFFFFFFFFLL; }

extern "C" int fp8bs_gemm(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb,
                          int64_t m, int64_t n, int64_t k, int b_layout, uint16_t* c, int64_t ldc,
                          void* stream) {
  if (!qa || !sa || !qb || !sb || !c) return FP8BS_ERR_NULL;
  if (b_layout != 0 && b_layout != 1) return FP8BS_ERR_FLAG;
  if (m <= 0 || n <= 0 || k <= 0 || n % 128 || k % BK || ldc < n) return FP8BS_ERR_SHAPE;
  if (!fits_u32(256 * k) || (b_layout == 1 && !fits_u32(k * n))) return FP8BS_ERR_SHAPE;
  if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(c, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
      ldc % 8)
    return FP8BS_ERR_ALIGN;
  GemmArgs a{qa, sa, qb, sb, c, ldc, m, n, k, nullptr, 0, 0, 0};
  if (b_layout == 0) return launch_gemm<kFprop, 128, 128, 2>(a, (hipStream_t)stream);
  return launch_gemm<kDgrad, 128, 128, 2>(a, (hipStream_t)stream);
}

extern "C" int fp8bs_grouped_gemm(const uint8_t* qa, const float* sa, const int32_t* seg_offsets,
                                  int64_t num_experts, int64_t total_rows, const uint8_t* qb,
                                  const float* sb, int64_t n, int64_t k, uint16_t* c, void* stream) {
  if (!qa || !sa || !seg_offsets || !qb || !sb || !c) return FP8BS_ERR_NULL;
  if (num_experts < 1 || num_experts > 65536 || total_rows <= 0 || total_rows % 128 || n <= 0 ||
      k <= 0 || n % 128 || k % BK)
    return FP8BS_ERR_SHAPE;
  if (!fits_u32(256 * k)) return FP8BS_ERR_SHAPE;
  if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(c, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
      !aligned(seg_offsets, 4))
    return FP8BS_ERR_ALIGN;
  GemmArgs a{qa, sa, qb, sb, c, n, total_rows, n, k, seg_offsets, num_experts, 0, 0};
  return launch_gemm<kGrouped, 128, 128, 2>(a, (hipStream_t)stream);
}

extern "C" int fp8bs_gemm_wgrad(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb,
                                int64_t m, int64_t n, int64_t t, float* c, int64_t ldc, int accumulate,
                                void* stream) {
  if (!qa || !sa || !qb || !sb || !c) return FP8BS_ERR_NULL;
  if (accumulate != 0 && accumulate != 1) return FP8BS_ERR_FLAG;
  if (m <= 0 || n <= 0 || t <= 0 || t % BK || n % 4 || ldc < n) return FP8BS_ERR_SHAPE;
  if (!fits_u32(256 * t)) return FP8BS_ERR_SHAPE;
  if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(c, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
      ldc % 4)
    return FP8BS_ERR_ALIGN;
  GemmArgs a{qa, sa, qb, sb, c, ldc, m, n, t, nullptr, 0, 0, accumulate};
  return launch_gemm<kWgrad, 128, 128, 2>(a, (hipStream_t)stream);
}
