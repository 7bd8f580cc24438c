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
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_act_rows_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ scales, int64_t tiles_per_row, int64_t total_tiles) {
  const int lane8 = threadIdx.x & 7;
  const int64_t tile = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const bool valid = tile < total_tiles;
  const int64_t t = valid ? tile : total_tiles - 1;   // keep the reduction converged
  const int64_t row = t / tiles_per_row;
  const int64_t tb = t - row * tiles_per_row;

  const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx + tb * kGroup + lane8 * 16);
  uint4 v0 = src[0];
  uint4 v1 = src[1];

  uint32_t m = max(max(absmax_pair(v0.x), absmax_pair(v0.y)), max(absmax_pair(v0.z), absmax_pair(v0.w)));
  m = max(m, max(max(absmax_pair(v1.x), absmax_pair(v1.y)), max(absmax_pair(v1.z), absmax_pair(v1.w))));
  m = max8_u32(m);
  GroupScale g = group_scale(m);

  uint4 out;
  out.x = quant4(v0.x, v0.y, g);
  out.y = quant4(v0.z, v0.w, g);
  out.z = quant4(v1.x, v1.y, g);
  out.w = quant4(v1.z, v1.w, g);
  if (valid) {
    *reinterpret_cast<uint4*>(q + row * ldq + tb * kGroup + lane8 * 16) = out;
    if (lane8 == 0) scales[t] = g.s;
  }
}

// ---------------------------------------------------------------------------
// Transposed 1x128 tiles (tiles along the rows of x): x [T, C] -> q [C, T],
// s [C, T/128].  One block handles 128 rows x 64 columns: the bf16 tile is
// staged through LDS, then each lane owns one column and each wave a quarter
// (32 rows) of the 128-row group; the four partial amax values meet in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_act_cols_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t cols, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scales, int64_t groups_t) {
  __shared__ uint16_t tile[128][64 + 8];     // +8 bf16 keeps 16-byte row alignment
  __shared__ uint32_t part[4][64];

  const int tid = threadIdx.x;
  const int64_t gt = blockIdx.y;             // token group (128 rows)
  const int64_t c0 = (int64_t)blockIdx.x * 64;

  // load 128 rows x 64 columns: 8 lanes x 16 bytes per row, 32 rows per pass
  {
    const int chunk = tid & 7;
    const int r0 = tid >> 3;
    const int64_t col = c0 + chunk * 8;
    const bool cok = col < cols;             // cols % 8 == 0, so a chunk is all in or all out
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = r0 + 32 * p;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (cok) v = *reinterpret_cast<const uint4*>(x + (gt * 128 + r) * ldx + col);
      *reinterpret_cast<uint4*>(&tile[r][chunk * 8]) = v;
    }
  }
  __syncthreads();

  const int lane = tid & 63;
  const int wave = tid >> 6;                 // rows 32*wave .. 32*wave+31
  uint32_t vals[16];                         // 32 bf16, packed in pairs along the rows
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t lo = tile[32 * wave + 2 * i][lane];
    uint32_t hi = tile[32 * wave + 2 * i + 1][lane];
    vals[i] = lo | (hi << 16);
    m = max(m, absmax_pair(vals[i]));
  }
  part[wave][lane] = m;
  __syncthreads();
  m = max(max(part[0][lane], part[1][lane]), max(part[2][lane], part[3][lane]));
  GroupScale g = group_scale(m);

  const int64_t col = c0 + lane;
  if (col < cols) {
    uint8_t* dst = q + col * ldq + gt * 128 + 32 * wave;
    uint4 o0, o1;
    o0.x = quant4(vals[0], vals[1], g);
    o0.y = quant4(vals[2], vals[3], g);
    o0.z = quant4(vals[4], vals[5], g);
    o0.w = quant4(vals[6], vals[7], g);
    o1.x = quant4(vals[8], vals[9], g);
    o1.y = quant4(vals[10], vals[11], g);
    o1.z = quant4(vals[12], vals[13], g);
    o1.w = quant4(vals[14], vals[15], g);
    reinterpret_cast<uint4*>(dst)[0] = o0;
    reinterpret_cast<uint4*>(dst)[1] = o1;
    if (wave == 0) scales[col * groups_t + gt] = g.s;
  }
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks: w [n, k] -> q [n, k], s [n/128, k/128].
// One 256-thread block per weight block; lane group of 16 covers one 256-byte
// row segment, each thread holds 8 rows x 8 bf16 in registers between the amax
// pass and the encode pass, so the block is read from HBM once.
// ---------------------------------------------------------------------------
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
  for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const uint4*>(base + (int64_t)(16 * i) * ldw);

  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    m = max(m, max(max(absmax_pair(v[i].x), absmax_pair(v[i].y)), max(absmax_pair(v[i].z), absmax_pair(v[i].w))));
  m = wave_max_u32(m);
  if ((tid & 63) == 0) part[tid >> 6] = m;
  __syncthreads();
  m = max(max(part[0], part[1]), max(part[2], part[3]));
  GroupScale g = group_scale(m);

  uint8_t* dst = q + (bn * 128 + rr) * ldq + bk * 128 + chunk * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint2 o;
    o.x = quant4(v[i].x, v[i].y, g);
    o.y = quant4(v[i].z, v[i].w, g);
    *reinterpret_cast<uint2*>(dst + (int64_t)(16 * i) * ldq) = o;
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
    hipLaunchKernelGGL(quant_act_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, ldx, q,
                       ldq, scales, tpr, total);
  } else {
    if (rows % kGroup || cols % 8 || ldq < rows) return FP8BS_ERR_SHAPE;
    const int64_t gt = rows / kGroup;
    const int64_t cb = (cols + 63) / 64;
    if (gt > 65535 || cb > kMaxGrid) return FP8BS_ERR_SHAPE;
    hipLaunchKernelGGL(quant_act_cols_kernel, dim3((unsigned)cb, (unsigned)gt), dim3(256), 0, s, x,
                       ldx, cols, q, ldq, scales, gt);
  }
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
  hipLaunchKernelGGL(quant_w_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, w,
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
    default: return "unknown status";
  }
}
