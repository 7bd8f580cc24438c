// Fine-grained FP8 quantization kernels and their C-ABI entry points.
//
// Groups (pages: "DeepSeek-V3 技术报告深度解读", section 3; deepseek.csdn.net
// page, section 二(四)): one scale per 1x128 activation tile and per 128x128
// weight block.  Per group: s = amax / 448 (binary32), code = E4M3 RNE of x / s
// with saturation, the sign kept also for zeros.  The kernels are bound by HBM
// traffic (2 bytes read, 1 byte + 4/group bytes written per element), so every
// load and store is a full 16-byte vector access and the amax reduction stays
// in registers (DPP), apart from one LDS exchange per weight block.

#include "common.h"
#include "launch.h"

namespace fp8bs {

// ---------------------------------------------------------------------------
// 1x128 tiles along the columns: x [rows, cols] -> q [rows, cols], s [rows, cols/128]
// One tile = 128 bf16 = 256 bytes, handled by 8 lanes (16 elements = 32 bytes each).
// A 256-thread block covers 32 consecutive tiles (row-major tile order).
// ROUTED: only the rows whose row_token entry is >= 0 are read and written
// (the rows that carry a routed token in an expert-major padded layout); the
// 8 lanes of a tile share its row, and a skipped tile's lanes return at once.
// ---------------------------------------------------------------------------
template <bool ROUTED>
__global__ __launch_bounds__(256) void quant_act_rows_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ scales, int64_t tiles_per_row, int64_t total_tiles,
    const int32_t* __restrict__ row_token) {
  const int lane8 = threadIdx.x & 7;
  const int64_t tile = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int64_t t = tile < total_tiles ? tile : total_tiles - 1;   // keep the reduction converged
  const int64_t row = t / tiles_per_row;
  const int64_t tb = t - row * tiles_per_row;
  const bool valid = tile < total_tiles && (!ROUTED || row_token[row] >= 0);
  // a skipped tile's 8 lanes leave together; the amax exchange below never
  // reads a lane outside its own tile's 8
  if (ROUTED && !valid) return;

  const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx + tb * kGroup + lane8 * 16);
  uint4 v0 = src[0];
  uint4 v1 = src[1];

  constexpr uint32_t kMag = 0x7FFF7FFFu;
  const uint32_t m2 = max_u16x2(max_u16x2(max_u16x2(v0.x & kMag, v0.y & kMag), max_u16x2(v0.z & kMag, v0.w & kMag)),
                                max_u16x2(max_u16x2(v1.x & kMag, v1.y & kMag), max_u16x2(v1.z & kMag, v1.w & kMag)));
  const uint32_t m = max8_u32(max(m2 & 0xFFFFu, m2 >> 16));
  GroupScale g = group_scale(m);

  const uint32_t in[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint4 out;
  quant_run<8>(in, reinterpret_cast<uint32_t*>(&out), g);
  if (valid) {
    *reinterpret_cast<uint4*>(q + row * ldq + tb * kGroup + lane8 * 16) = out;
    if (lane8 == 0) scales[t] = g.s;
  }
}

// ---------------------------------------------------------------------------
// Tiles along the rows (transposed output), optionally fused with the tiles
// along the columns.  x [T, C] -> qt [C, T], st [C, T/128]; with ROWS also
// q [T, C], s [T, C/128] from the same read of x.
//
// A 256-thread block owns one square of 128 x 128.  The square (32 KB of
// bf16) is loaded with 8 loads of 16 bytes per thread (every row segment a
// full 256 bytes) and staged in LDS.
//
// LDS: row R of the square is 256 bytes; its 16-byte chunk q sits at chunk
// q ^ f(R), f(R) = (R & 15) ^ (((R >> 5) & 3) << 2).
//
// Transposed tiles use ds_read_b64_tr_b16 (gfx950): in a group of 16 lanes
// that each point at 4 bf16 of some row, lane i receives element (i mod 4) of
// the rows addressed by lanes (i div 4), 4 + (i div 4), 8 + (i div 4) and
// 12 + (i div 4).  Lane j of a group addresses row 32 (j mod 4) + 4t + (j div 4)
// at a fixed 4-column quad, so after t = 0..7 lane i holds column
// (quad + i mod 4) for the 32 consecutive rows 32 (i div 4) .. +31.  Those 16
// rows fall in 16 distinct swizzled chunks (no bank conflict); the four lanes
// of a column meet through two DPP row rotations for the amax, and each
// writes its 32 codes as two 16-byte stores.  Each 16-lane group codes two
// column quads.
//
// Row tiles (ROWS) take 8 lanes per row and 16 codes per lane, so their
// stores write whole rows of q (see below).
// ---------------------------------------------------------------------------
constexpr int kQB = 128;                   // rows and columns per square

__device__ __forceinline__ int qswz(int row) { return (row & 15) ^ (((row >> 5) & 3) << 2); }

typedef short v4s __attribute__((ext_vector_type(4)));

// STREAM: the input is larger than half the last-level cache, so it is read
// with the non-temporal hint (cold 16384 x 7168: 78 -> 72 us; the fused
// kernel on 4096 x 32768: 125 -> 112 us); an input that fits may still be
// cached from its producer, and the hint loses those hits (warm 16384 x 1536:
// 14.7 -> 18.5 us; the fused kernel on inputs that fit is slower with it too).
template <bool ROWS, bool STREAM = false>
__global__ __launch_bounds__(256) void quant_act_cols_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t rows, int64_t cols,
    uint8_t* __restrict__ qt, int64_t ldqt, float* __restrict__ st,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kQB * 256];

  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kQB;               // the square's first column
  const int64_t r0 = (int64_t)blockIdx.y * kQB;               // and first row (rows % 128 == 0: squares are full)

  // staging lanes: thread (chunk, rr) covers rows rr, rr+16, ... at 16-byte chunk `chunk`.
  // A chunk past the last column (cols % 8 == 0, so chunks are whole) loads a valid
  // address of the same row and is replaced by zeros.
  const int chunk = tid & 15;
  const int rr = tid >> 4;
  const bool cok = c0 + chunk * 8 < cols;
  const uint16_t* src = x + (r0 + rr) * ldx + (cok ? c0 + chunk * 8 : 0);
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t* a = src + (int64_t)(16 * i) * ldx;
    v[i] = STREAM ? load_nt(a) : *reinterpret_cast<const uint4*>(a);
  }
  if (!cok) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = make_uint4(0, 0, 0, 0);
  }

  const int lane = tid & 15;                                   // lane inside its 16-lane group
  const int grp16 = tid >> 4;                                  // 16 groups
  {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = rr + 16 * i;
      *reinterpret_cast<uint4*>(&tile[row * 256 + ((chunk ^ qswz(row)) << 4)]) = v[i];
    }
    __syncthreads();

    // ---- transposed tiles: two column quads per 16-lane group
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cq = grp16 + 16 * u;                           // column quad 0..31
      const int qc = cq >> 1, half = (cq & 1) << 3;
      uint32_t vals[16];
      uint32_t m2 = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int row = 32 * (lane & 3) + 4 * t + (lane >> 2);
        const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(&tile[row * 256 + ((qc ^ qswz(row)) << 4) + half]));
        vals[2 * t] = (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
        vals[2 * t + 1] = (uint32_t)(uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16);
        m2 = max_u16x2(m2, max_u16x2(vals[2 * t] & 0x7FFF7FFFu, vals[2 * t + 1] & 0x7FFF7FFFu));
      }
      uint32_t m = max(m2 & 0xFFFFu, m2 >> 16);
      m = max(m, dpp_shuffle<0x124>(m));                       // row_ror:4
      m = max(m, dpp_shuffle<0x128>(m));                       // row_ror:8
      const int64_t col = c0 + 4 * cq + (lane & 3);
      if (col < cols) {
        const GroupScale gs = group_scale(m);
        uint8_t* dst = qt + col * ldqt + r0 + 32 * (lane >> 2);
        uint4 o[2];
        quant_run<16>(vals, reinterpret_cast<uint32_t*>(o), gs);
        reinterpret_cast<uint4*>(dst)[0] = o[0];
        reinterpret_cast<uint4*>(dst)[1] = o[1];
        if ((lane >> 2) == 0) st[col * (rows / kGroup) + r0 / kGroup] = gs.s;
      }
    }

    // ---- row tiles (fused mode, cols % 128 == 0): 8 lanes per row, 16 codes
    // per lane, so each 16-byte store instruction writes whole 128-byte rows
    // of q (8 rows per wave).  Measured on the memory pattern alone (reads of
    // the square plus both outputs, no arithmetic): 26.2 us with half rows per
    // lane, 20.9 us with whole lines, for a 4096 x 7168 input.  The 8 lanes of
    // a row read chunks 2s, 2s + 1; within a ds_read_b128 pass (4-lane groups
    // of one index parity) the four rows' chunk positions are distinct.
    if (ROWS) {
      const int sgm = tid & 7;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = 32 * it + (tid >> 3);
        const uint4 a = *reinterpret_cast<const uint4*>(&tile[r * 256 + (((2 * sgm) ^ qswz(r)) << 4)]);
        const uint4 b = *reinterpret_cast<const uint4*>(&tile[r * 256 + (((2 * sgm + 1) ^ qswz(r)) << 4)]);
        constexpr uint32_t kMag = 0x7FFF7FFFu;
        const uint32_t m2 = max_u16x2(max_u16x2(max_u16x2(a.x & kMag, a.y & kMag), max_u16x2(a.z & kMag, a.w & kMag)),
                                      max_u16x2(max_u16x2(b.x & kMag, b.y & kMag), max_u16x2(b.z & kMag, b.w & kMag)));
        const uint32_t m = max8_u32(max(m2 & 0xFFFFu, m2 >> 16));
        const GroupScale gs = group_scale(m);
        const uint32_t in[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint4 o;
        quant_run<8>(in, reinterpret_cast<uint32_t*>(&o), gs);
        *reinterpret_cast<uint4*>(q + (r0 + r) * ldq + c0 + 16 * sgm) = o;
        if (sgm == 0) s[(r0 + r) * (cols / kGroup) + c0 / kGroup] = gs.s;
      }
    }
  }
}

// one block per 128 x 128 square: x walks the column strips, y the rows
static dim3 cols_grid(int64_t rows, int64_t cols) {
  return dim3((unsigned)((cols + kQB - 1) / kQB), (unsigned)(rows / kQB));
}
static bool cols_grid_ok(int64_t rows, int64_t cols) {
  return rows / kQB <= 65535 && (cols + kQB - 1) / kQB <= kMaxGrid;
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks: w [n, k] -> q [n, k], s [n/128, k/128].
// One 256-thread block per weight block; lane group of 16 covers one 256-byte
// row segment, each thread holds 8 rows x 8 bf16 in registers between the amax
// pass and the encode pass, so the block is read from HBM once.  STREAM (a
// weight tensor larger than half the last-level cache, such as stacked experts):
// weights and codes pass through with the non-temporal hint (32 experts of
// 4096 x 7168: 501-526 -> 486-498 us); smaller tensors keep plain accesses, so
// a weight still cached from its update is read from the cache and its codes
// stay there for the GEMM that follows.
// ---------------------------------------------------------------------------
template <bool STREAM>
__global__ __launch_bounds__(256) void quant_w_kernel(
    const uint16_t* __restrict__ w, int64_t ldw, uint8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ scales, int64_t kblocks) {
  __shared__ uint32_t part[4];
  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;
  const int64_t bn = blk / kblocks;
  const int64_t bk = blk - bn * kblocks;
  const int chunk = tid & 15;                // 16-byte chunk within the 256-byte row segment
  const int rr = tid >> 4;                   // 0..15

  const uint16_t* base = w + (bn * 128 + rr) * ldw + bk * 128 + chunk * 8;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t* a = base + (int64_t)(16 * i) * ldw;
    v[i] = STREAM ? load_nt(a) : *reinterpret_cast<const uint4*>(a);
  }

  constexpr uint32_t kMag = 0x7FFF7FFFu;
  uint32_t m2 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    m2 = max_u16x2(m2, max_u16x2(max_u16x2(v[i].x & kMag, v[i].y & kMag), max_u16x2(v[i].z & kMag, v[i].w & kMag)));
  uint32_t m = wave_max_u32(max(m2 & 0xFFFFu, m2 >> 16));
  if ((tid & 63) == 0) part[tid >> 6] = m;
  __syncthreads();
  m = max(max(part[0], part[1]), max(part[2], part[3]));
  GroupScale g = group_scale(m);

  uint8_t* dst = q + (bn * 128 + rr) * ldq + bk * 128 + chunk * 8;
  uint2 o[8];
  quant_run<32>(reinterpret_cast<const uint32_t*>(v), reinterpret_cast<uint32_t*>(o), g);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint8_t* d = dst + (int64_t)(16 * i) * ldq;
    if (STREAM) store_nt(d, o[i]);
    else *reinterpret_cast<uint2*>(d) = o[i];
  }
  if (tid == 0) scales[blk] = g.s;
}

}  // namespace fp8bs

using namespace fp8bs;

extern "C" int fp8bs_quantize_act_1x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                        int transpose, uint8_t* q, int64_t ldq, float* scales,
                                        void* stream) {
  if (!x || !q || !scales) return FP8BS_ERR_NULL;
  if (transpose != 0 && transpose != 1) return FP8BS_ERR_FLAG;
  if (rows <= 0 || cols <= 0) return FP8BS_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4) || ldx % 8 || ldq % 16)
    return FP8BS_ERR_ALIGN;
  if (ldx < cols) return FP8BS_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (transpose == 0) {
    if (cols % kGroup || ldq < cols) return FP8BS_ERR_SHAPE;
    const int64_t tpr = cols / kGroup;
    const int64_t total = rows * tpr;
    const int64_t blocks = (total + 31) / 32;
    if (blocks > kMaxGrid) return FP8BS_ERR_SHAPE;
    hipLaunchKernelGGL(quant_act_rows_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, x, ldx, q,
                       ldq, scales, tpr, total, (const int32_t*)nullptr);
  } else {
    if (rows % kGroup || cols % 8 || ldq < rows) return FP8BS_ERR_SHAPE;
    if (!cols_grid_ok(rows, cols)) return FP8BS_ERR_SHAPE;
    if (rows * cols * 2 > kStreamBytes)
      hipLaunchKernelGGL((quant_act_cols_kernel<false, true>), cols_grid(rows, cols), dim3(256), 0, s, x,
                         ldx, rows, cols, q, ldq, scales, (uint8_t*)nullptr, (int64_t)0, (float*)nullptr);
    else
      hipLaunchKernelGGL((quant_act_cols_kernel<false, false>), cols_grid(rows, cols), dim3(256), 0, s, x,
                         ldx, rows, cols, q, ldq, scales, (uint8_t*)nullptr, (int64_t)0, (float*)nullptr);
  }
  return launch_status();
}

extern "C" int fp8bs_quantize_act_1x128_routed(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                               const int32_t* row_token, uint8_t* q, int64_t ldq,
                                               float* scales, void* stream) {
  if (!x || !row_token || !q || !scales) return FP8BS_ERR_NULL;
  if (rows <= 0 || cols <= 0 || cols % kGroup || ldx < cols || ldq < cols) return FP8BS_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4) || !aligned(row_token, 4) || ldx % 8 ||
      ldq % 16)
    return FP8BS_ERR_ALIGN;
  const int64_t tpr = cols / kGroup;
  const int64_t total = rows * tpr;
  const int64_t blocks = (total + 31) / 32;
  if (blocks > kMaxGrid) return FP8BS_ERR_SHAPE;
  hipLaunchKernelGGL(quant_act_rows_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, x,
                     ldx, q, ldq, scales, tpr, total, row_token);
  return launch_status();
}

extern "C" int fp8bs_quantize_act_1x128_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                             uint8_t* q, int64_t ldq, float* scales, uint8_t* qt,
                                             int64_t ldqt, float* scales_t, void* stream) {
  if (!x || !q || !scales || !qt || !scales_t) return FP8BS_ERR_NULL;
  if (rows <= 0 || cols <= 0 || rows % kGroup || cols % kGroup) return FP8BS_ERR_SHAPE;
  if (ldx < cols || ldq < cols || ldqt < rows) return FP8BS_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(qt, 16) || !aligned(scales, 4) ||
      !aligned(scales_t, 4) || ldx % 8 || ldq % 16 || ldqt % 16)
    return FP8BS_ERR_ALIGN;
  if (!cols_grid_ok(rows, cols)) return FP8BS_ERR_SHAPE;
  if (rows * cols * 2 > kStreamBytes)
    hipLaunchKernelGGL((quant_act_cols_kernel<true, true>), cols_grid(rows, cols), dim3(256), 0,
                       (hipStream_t)stream, x, ldx, rows, cols, qt, ldqt, scales_t, q, ldq, scales);
  else
    hipLaunchKernelGGL(quant_act_cols_kernel<true>, cols_grid(rows, cols), dim3(256), 0,
                       (hipStream_t)stream, x, ldx, rows, cols, qt, ldqt, scales_t, q, ldq, scales);
  return launch_status();
}

extern "C" int fp8bs_quantize_w_128x128(const uint16_t* w, int64_t n, int64_t k, int64_t ldw,
                                        uint8_t* q, int64_t ldq, float* scales, void* stream) {
  if (!w || !q || !scales) return FP8BS_ERR_NULL;
  if (n <= 0 || k <= 0 || n % kGroup || k % kGroup) return FP8BS_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scales, 4) || ldw % 8 || ldq % 16)
    return FP8BS_ERR_ALIGN;
  if (ldw < k || ldq < k) return FP8BS_ERR_SHAPE;
  const int64_t kb = k / kGroup;
  const int64_t blocks = (n / kGroup) * kb;
  if (blocks > kMaxGrid) return FP8BS_ERR_SHAPE;
  if (n * k * 2 > kStreamBytes)
    hipLaunchKernelGGL(quant_w_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, w,
                       ldw, q, ldq, scales, kb);
  else
    hipLaunchKernelGGL(quant_w_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, w,
                       ldw, q, ldq, scales, kb);
  return launch_status();
}

extern "C" const char* fp8bs_status_string(int status) {
  switch (status) {
    case FP8BS_OK: return "ok";
    case FP8BS_ERR_NULL: return "null pointer argument";
    case FP8BS_ERR_SHAPE: return "invalid size (non-positive, not a required multiple, or too large)";
    case FP8BS_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case FP8BS_ERR_FLAG: return "unknown flag value";
    case FP8BS_ERR_LAUNCH: return "kernel launch failed";
    case FP8BS_ERR_SCRATCH: return "problem needs more than the fixed scratch array";
    default: return "unknown status";
  }
}
