// MoE dispatch and combine around the grouped GEMM (gfx950).
//
// Each token is routed to k of the routed experts (deepseek.csdn.net page,
// section 一(二) "DeepSeekMoE 架构"); a layer's chunk dispatches the tokens to
// their experts before the expert MLP and combines the expert outputs after it
// (qqstock.cn page, section "DualPipe 流水線并行"); activations travel in FP8
// and the combined outputs in BF16 (deepseek.csdn.net page, section 二(四)).
// On one GPU the dispatch is a permutation into expert-major rows, each
// expert's run padded to a multiple of 128 rows so that every 128-row tile of
// the grouped GEMM belongs to one expert.
//
//   moe_route_kernel     one workgroup: a stable counting sort of the
//                        (token, slot) pairs by expert id, giving the padded
//                        segment starts and each pair's row; with
//   moe_route_rows_kernel  each row's token
//   moe_dispatch_kernel  each token row is read once, coded once in 1x128
//                        tiles and its codes and scales stored to its k rows;
//                        four workgroups per expert zero its padding rows
//   moe_combine_kernel   one wave per token: the gate-weighted FP32 sum of the
//                        token's k expert-output rows, rounded once to bf16
//
// Nothing here reads a size from the device to size a launch: the grids come
// from host sizes and the largest padded row count, so the three calls and the
// grouped GEMM between them need no host synchronization.  Every row index
// that comes from device memory is checked against the row capacity before it
// is used, so no device contents can make a kernel access memory outside the
// caller's buffers.

#include "common.h"
#include "launch.h"

namespace fp8bs {

constexpr int kRouteWaves = 16;            // one 1024-thread workgroup
constexpr int kRouteMaxExperts = 512;      // LDS: 96 KB of per-wave tables
constexpr int kMaxTopk = 64;               // a token's slots fit in one wave's lanes

// ---------------------------------------------------------------------------
// Routing: wave w owns the pairs [lo_w, hi_w) (pairs in row-major
// (token, slot) order, chunks in wave order), so "earlier pair" means an
// earlier wave, or an earlier 64-pair step of the same wave, or a lower lane.
//   1. each wave walks its chunk 64 pairs at a time: every lane ORs its lane
//      bit into its expert's 64-bit mask in LDS (an atomic OR: the order of
//      the lanes does not matter), then reads the mask back: the lanes of the
//      step that hold the same expert.  A pair's rank among them is the
//      population count of the lower lanes; its rank within the wave's chunk
//      (the wave's running count for that expert, also in LDS, plus that
//      rank) goes to slot_rows for now, and the lowest lane of the group
//      advances the running count by the group's size and clears the mask.
//      (One ballot per id bit instead: 38 us against 26 us for the whole
//      routing of 32768 pairs over 256 experts, the ballots' vector work
//      saturating the workgroup's one compute unit.)
//   2. per expert: exclusive prefix of the running counts over the waves,
//      count, padded size; an exclusive scan of the padded sizes over the
//      experts gives the segment starts; each wave's first row for expert e is
//      start + its prefix
//   3. every pair adds its wave's first row for its expert to its rank
//      (independent pairs: no chain)
//   4. padding rows and the rows past the padded total get token -1, written
//      by whole waves in runs
// The ids of 16 steps are loaded together, so each wave waits for memory once
// per 1024 pairs.  The row -> token entries of the routed pairs are scattered
// by moe_route_rows_kernel, a separate grid over the pairs: from one
// workgroup those 4-byte stores to 64 different rows per instruction would
// serialize in the workgroup's one memory pipeline.
constexpr int kRouteBatch = 16;

__global__ __launch_bounds__(1024) void moe_route_kernel(const int32_t* __restrict__ ids, int64_t pairs,
                                                         int num_e, int32_t* __restrict__ seg,
                                                         int32_t* __restrict__ slot_rows,
                                                         int32_t* __restrict__ row_token, int64_t cap) {
  __shared__ int next_row[kRouteWaves][kRouteMaxExperts];
  __shared__ int seg_s[kRouteMaxExperts + 1];
  __shared__ int cnt_s[kRouteMaxExperts];
  __shared__ int wave_sum[kRouteWaves];
  __shared__ unsigned long long match[kRouteWaves][kRouteMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  if (tid < num_e)
    for (int v = 0; v < kRouteWaves; ++v) {
      next_row[v][tid] = 0;
      match[v][tid] = 0;
    }
  __syncthreads();

  const int64_t chunk = ((pairs + kRouteWaves - 1) / kRouteWaves + 63) / 64 * 64;
  const int64_t lo = min(pairs, (int64_t)w * chunk), hi = min(pairs, lo + chunk);
  const uint64_t below = (1ull << lane) - 1ull;
  for (int64_t b0 = lo; b0 < hi; b0 += 64 * kRouteBatch) {
    int ev[kRouteBatch];
#pragma unroll
    for (int st = 0; st < kRouteBatch; ++st) {
      const int64_t i = b0 + 64 * st + lane;
      ev[st] = i < hi ? ids[i] : -1;
    }
#pragma unroll
    for (int st = 0; st < kRouteBatch; ++st) {
      if (b0 + 64 * st >= hi) break;
      const int64_t i = b0 + 64 * st + lane;
      const int e = ev[st];
      const bool ok = i < hi && e >= 0 && e < num_e;
      if (ok) atomicOr(&match[w][e], 1ull << lane);
      if (ok) {
        const uint64_t same = match[w][e];
        const int rank = __popcll(same & below);
        const int base = next_row[w][e];
        slot_rows[i] = base + rank;
        if (rank == 0) {
          next_row[w][e] = base + __popcll(same);
          match[w][e] = 0;
        }
      } else if (i < hi) {
        slot_rows[i] = -1;
      }
    }
  }
  __syncthreads();

  int padded = 0;
  if (tid < num_e) {
    int run = 0;
    for (int v = 0; v < kRouteWaves; ++v) {
      const int c = next_row[v][tid];
      next_row[v][tid] = run;
      run += c;
    }
    cnt_s[tid] = run;
    padded = (run + 127) & ~127;
  }
  int incl = padded;                                   // inclusive scan inside the wave
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_sum[w] = incl;
  __syncthreads();
  int excl = incl - padded;
  for (int v = 0; v < w; ++v) excl += wave_sum[v];
  if (tid < num_e) {
    seg_s[tid] = excl;
    seg[tid] = excl;
    for (int v = 0; v < kRouteWaves; ++v) next_row[v][tid] += excl;
    if (tid == num_e - 1) {
      seg_s[num_e] = excl + padded;
      seg[num_e] = excl + padded;
    }
  }
  __syncthreads();

  for (int64_t b0 = lo; b0 < hi; b0 += 64 * kRouteBatch) {
    int ev[kRouteBatch], rv[kRouteBatch];
#pragma unroll
    for (int st = 0; st < kRouteBatch; ++st) {
      const int64_t i = b0 + 64 * st + lane;
      ev[st] = i < hi ? ids[i] : -1;
      rv[st] = i < hi ? slot_rows[i] : -1;            // this lane's own store of step 1
    }
#pragma unroll
    for (int st = 0; st < kRouteBatch; ++st) {
      const int64_t i = b0 + 64 * st + lane;
      if (i < hi && ev[st] >= 0 && ev[st] < num_e) slot_rows[i] = next_row[w][ev[st]] + rv[st];
    }
  }

  for (int e = w; e < num_e; e += kRouteWaves)
    for (int r = seg_s[e] + cnt_s[e] + lane; r < seg_s[e + 1]; r += 64) row_token[r] = -1;
  for (int64_t r = (int64_t)seg_s[num_e] + tid; r < cap; r += 1024) row_token[r] = -1;
}

// row -> token for every routed pair (the other rows were set by moe_route_kernel)
__global__ __launch_bounds__(256) void moe_route_rows_kernel(const int32_t* __restrict__ slot_rows, int64_t pairs,
                                                             int topk, int32_t* __restrict__ row_token,
                                                             int64_t cap) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= pairs) return;
  const int r = slot_rows[i];
  if (r >= 0 && r < cap) row_token[r] = (int)(i / topk);
}

// ---------------------------------------------------------------------------
// Dispatch payload.  Token blocks: 4 waves, TPW tokens per wave; 8 lanes per
// 128-element tile (16 bf16 each, two 16-byte loads), so one wave step covers
// 8 tiles (2 KB of the row) and stores 8 x 1 KB of codes, one full 1 KB run
// per destination row and store instruction.  The tile's amax, scale and codes
// are computed exactly as by the 1x128 activation quantizer (a tile depends
// only on its own 128 values), once per token, whatever k is.
// Padding blocks come first in the grid (blockIdx.x < pad_blocks), so their
// zero rows are written alongside the token blocks rather than after them:
// with a skewed routing padding is a large share of the rows (21120 of 53888
// for 4096 tokens, top-8 of 256 experts, Zipf 1.1).  Each padding row (token
// -1) gets +0 codes and scale 0.  STREAM: the routed rows' codes are stored
// with the non-temporal hint (measured at that size: 98 -> 72 us; the hint
// on the padding rows' zeros made it slower, and so did placing the padding
// blocks after the token blocks or giving a wave more than one token).
__device__ __forceinline__ uint32_t tile16_amax(const uint32_t in[8]) {
  constexpr uint32_t kMag = 0x7FFF7FFFu;
  const uint32_t m2 = max_u16x2(max_u16x2(max_u16x2(in[0] & kMag, in[1] & kMag), max_u16x2(in[2] & kMag, in[3] & kMag)),
                                max_u16x2(max_u16x2(in[4] & kMag, in[5] & kMag), max_u16x2(in[6] & kMag, in[7] & kMag)));
  return max8_u32(max(m2 & 0xFFFFu, m2 >> 16));
}

constexpr int kPadParts = 4;                        // padding workgroups per expert

template <int TPW, bool STREAM>
__global__ __launch_bounds__(256) void moe_dispatch_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t tokens, int hidden,
    const int32_t* __restrict__ slot_rows, int topk, const int32_t* __restrict__ seg,
    const int32_t* __restrict__ row_token, uint8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ scales, int64_t cap, int64_t pad_blocks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int groups = hidden / kGroup;
  if ((int64_t)blockIdx.x < pad_blocks) {
    // padding: expert e's padding rows lie in the last 128 rows of its
    // segment; workgroup (e, part) checks 32 of them, one wave per row
    const int64_t e = (int64_t)blockIdx.x / kPadParts, part = (int64_t)blockIdx.x % kPadParts;
    int64_t hi = seg[e + 1];
    if (hi > cap) hi = cap;
    int64_t lo = seg[e];
    if (lo < 0) lo = 0;
    const int64_t r0 = hi - kGroup + part * (kGroup / kPadParts);
    const uint4 zero = make_uint4(0, 0, 0, 0);
    for (int64_t r = r0 + wave; r < r0 + kGroup / kPadParts; r += 4) {
      if (r < lo || r >= hi || row_token[r] >= 0) continue;
      uint8_t* qr = q + r * ldq;
      for (int c = 16 * lane; c < hidden; c += 1024) *reinterpret_cast<uint4*>(qr + c) = zero;
      for (int c = lane; c < groups; c += 64) scales[r * groups + c] = 0.0f;
    }
  } else {
    // TPW tokens per wave, their steps interleaved (more loads in flight)
    const int64_t t0 = (((int64_t)blockIdx.x - pad_blocks) * 4 + wave) * TPW;
    if (t0 >= tokens) return;
    const int sg = lane & 7;
    const uint4 zero = make_uint4(0, 0, 0, 0);
    int my_row[TPW];                                   // lane j < topk: the row of slot j
    const uint4* xr[TPW];                              // 16 uint4 per tile
    uint4 a[TPW], b[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const bool live = t0 + u < tokens;
      const int64_t t = live ? t0 + u : t0;
      my_row[u] = -1;
      if (live && lane < topk) {
        const int r = slot_rows[t * topk + lane];
        my_row[u] = (r >= 0 && r < cap) ? r : -1;
      }
      xr[u] = reinterpret_cast<const uint4*>(x + t * ldx + 16 * sg);
      a[u] = zero;
      b[u] = zero;
      if ((lane >> 3) < groups) {
        a[u] = xr[u][16 * (lane >> 3)];
        b[u] = xr[u][16 * (lane >> 3) + 1];
      }
    }
    for (int g0 = 0; g0 < groups; g0 += 8) {
      const int g = g0 + (lane >> 3);
      uint4 na[TPW], nb[TPW];                          // next step's loads first
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        na[u] = zero;
        nb[u] = zero;
        if (g + 8 < groups) {
          na[u] = xr[u][16 * (g + 8)];
          nb[u] = xr[u][16 * (g + 8) + 1];
        }
      }
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const uint32_t in[8] = {a[u].x, a[u].y, a[u].z, a[u].w, b[u].x, b[u].y, b[u].z, b[u].w};
        const GroupScale gs = group_scale(tile16_amax(in));
        uint4 o;
        quant_run<8>(in, reinterpret_cast<uint32_t*>(&o), gs);
        for (int j = 0; j < topk; ++j) {              // uniform loop: readlane sees every lane
          const int row = __builtin_amdgcn_readlane(my_row[u], j);
          if (row < 0 || g >= groups) continue;
          uint8_t* d = q + (int64_t)row * ldq + (int64_t)g * kGroup + 16 * sg;
          if (STREAM) store_nt(d, o);
          else *reinterpret_cast<uint4*>(d) = o;
          if (sg == 0) scales[(int64_t)row * groups + g] = gs.s;
        }
        a[u] = na[u];
        b[u] = nb[u];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: TPW tokens per wave, 8 bf16 columns per lane and step (512 columns
// per wave step).  A token's k rows' 16-byte pieces are loaded together, 8
// slots at a time, then folded in slot order: acc = fma(g_j, y_j, acc) in
// FP32, starting from +0; a dropped slot (row -1 or outside the capacity) is
// skipped.  The sum is rounded once to bf16 (nearest, ties to even).
// STREAM: the expert rows are read once, with the non-temporal hint
// (measured on 4096 tokens x top-8, 7168 columns: 110 -> 98.5 us; the hint on
// the output store, or more tokens per wave, did not help).
template <int TPW, bool STREAM>
__global__ __launch_bounds__(256) void moe_combine_kernel(
    const uint16_t* __restrict__ y, int64_t ldy, int64_t cap, const int32_t* __restrict__ slot_rows,
    const float* __restrict__ gates, int64_t tokens, int topk, int n, uint16_t* __restrict__ out,
    int64_t ldo) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = ((int64_t)blockIdx.x * 4 + wave) * TPW;
  if (t0 >= tokens) return;
  int my_row[TPW];
  float my_g[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    my_row[u] = -1;
    my_g[u] = 0.0f;
    if (t0 + u < tokens && lane < topk) {
      const int r = slot_rows[(t0 + u) * topk + lane];
      my_row[u] = (r >= 0 && r < cap) ? r : -1;
      my_g[u] = gates[(t0 + u) * topk + lane];
    }
  }
  for (int c0 = 0; c0 < n; c0 += 512) {              // uniform loop: readlane sees every lane
    const int c = c0 + 8 * lane;
    const bool live = c < n;
    float acc[TPW][8];
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
    for (int j0 = 0; j0 < topk; j0 += 8) {
      uint4 v[TPW][8];
      int rows[TPW][8];
#pragma unroll
      for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          rows[u][jj] = j0 + jj < topk ? __builtin_amdgcn_readlane(my_row[u], j0 + jj) : -1;
          v[u][jj] = rows[u][jj] >= 0 && live
                         ? (STREAM ? load_nt(y + (int64_t)rows[u][jj] * ldy + c)
                                   : *reinterpret_cast<const uint4*>(y + (int64_t)rows[u][jj] * ldy + c))
                         : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
      for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          if (rows[u][jj] < 0) continue;
          const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g[u]), j0 + jj));
          const uint32_t d[4] = {v[u][jj].x, v[u][jj].y, v[u][jj].z, v[u][jj].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[u][2 * i] = __builtin_fmaf(g, bf16_lo(d[i]), acc[u][2 * i]);
            acc[u][2 * i + 1] = __builtin_fmaf(g, bf16_hi(d[i]), acc[u][2 * i + 1]);
          }
        }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      uint4 o;
      o.x = f32_to_bf16_rne(acc[u][0]) | (f32_to_bf16_rne(acc[u][1]) << 16);
      o.y = f32_to_bf16_rne(acc[u][2]) | (f32_to_bf16_rne(acc[u][3]) << 16);
      o.z = f32_to_bf16_rne(acc[u][4]) | (f32_to_bf16_rne(acc[u][5]) << 16);
      o.w = f32_to_bf16_rne(acc[u][6]) | (f32_to_bf16_rne(acc[u][7]) << 16);
      if (live && t0 + u < tokens) *reinterpret_cast<uint4*>(out + (t0 + u) * ldo + c) = o;
    }
  }
}

constexpr int kDispatchTPW = 1;
constexpr int kCombineTPW = 1;

static int64_t max_rows(int64_t tokens, int64_t topk, int64_t num_e) {
  const int64_t pairs = tokens * topk;
  const int64_t busy = num_e < pairs ? num_e : pairs;
  return (pairs + 127 * busy) / kGroup * kGroup;
}

static bool route_sizes_ok(int64_t tokens, int64_t topk, int64_t num_e) {
  return tokens >= 0 && topk >= 1 && topk <= kMaxTopk && num_e >= 1 && num_e <= 65536 &&
         tokens <= 0x7FFFFFFFLL / topk && max_rows(tokens, topk, num_e) <= 0x7FFFFFFFLL;
}

}  // namespace fp8bs

using namespace fp8bs;

extern "C" int64_t fp8bs_moe_max_rows(int64_t tokens, int64_t topk, int64_t num_experts) {
  if (!route_sizes_ok(tokens, topk, num_experts)) return FP8BS_ERR_SHAPE;
  return max_rows(tokens, topk, num_experts);
}

extern "C" int fp8bs_moe_route(const int32_t* topk_ids, int64_t tokens, int64_t topk, int64_t num_experts,
                               int32_t* seg_offsets, int32_t* slot_rows, int32_t* row_token, int64_t rows_cap,
                               void* stream) {
  if (!seg_offsets || (tokens > 0 && (!topk_ids || !slot_rows)) || (rows_cap > 0 && !row_token))
    return FP8BS_ERR_NULL;
  if (!route_sizes_ok(tokens, topk, num_experts) || num_experts > kRouteMaxExperts) return FP8BS_ERR_SHAPE;
  if (rows_cap < max_rows(tokens, topk, num_experts) || rows_cap > 0x7FFFFFFFLL) return FP8BS_ERR_SHAPE;
  if (!aligned(topk_ids, 4) || !aligned(seg_offsets, 4) || !aligned(slot_rows, 4) || !aligned(row_token, 4))
    return FP8BS_ERR_ALIGN;
  const int64_t pairs = tokens * topk;
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(64 * kRouteWaves), 0, (hipStream_t)stream, topk_ids, pairs,
                     (int)num_experts, seg_offsets, slot_rows, row_token, rows_cap);
  if (pairs > 0)
    hipLaunchKernelGGL(moe_route_rows_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, slot_rows, pairs, (int)topk, row_token, rows_cap);
  return launch_status();
}

extern "C" int fp8bs_moe_permute_quantize(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t ldx,
                                          const int32_t* slot_rows, int64_t topk, const int32_t* seg_offsets,
                                          const int32_t* row_token, int64_t num_experts, uint8_t* q,
                                          int64_t ldq, float* scales, int64_t rows_cap, void* stream) {
  if (!seg_offsets || (tokens > 0 && (!x || !slot_rows)) || (rows_cap > 0 && (!row_token || !q || !scales)))
    return FP8BS_ERR_NULL;
  if (!route_sizes_ok(tokens, topk, num_experts)) return FP8BS_ERR_SHAPE;
  if (hidden <= 0 || hidden % kGroup || hidden > (1 << 30) || ldx < hidden || ldq < hidden) return FP8BS_ERR_SHAPE;
  if (rows_cap < 0 || rows_cap > 0x7FFFFFFFLL) return FP8BS_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4) || !aligned(slot_rows, 4) ||
      !aligned(seg_offsets, 4) || !aligned(row_token, 4) || ldx % 8 || ldq % 16)
    return FP8BS_ERR_ALIGN;
  const int64_t token_blocks = (tokens + 4 * kDispatchTPW - 1) / (4 * kDispatchTPW);
  const int64_t pad_blocks = num_experts * kPadParts;
  const int64_t grid = pad_blocks + token_blocks;
  if (grid > kMaxGrid) return FP8BS_ERR_SHAPE;
  // the payload is streamed when it is larger than half the last-level cache;
  // a smaller one stays cached for the grouped GEMM that reads it next
  if (tokens * topk * hidden > kStreamBytes)
    hipLaunchKernelGGL((moe_dispatch_kernel<kDispatchTPW, true>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, x, ldx, tokens, (int)hidden, slot_rows, (int)topk, seg_offsets, row_token,
                       q, ldq, scales, rows_cap, pad_blocks);
  else
    hipLaunchKernelGGL((moe_dispatch_kernel<kDispatchTPW, false>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, x, ldx, tokens, (int)hidden, slot_rows, (int)topk, seg_offsets, row_token,
                       q, ldq, scales, rows_cap, pad_blocks);
  return launch_status();
}

extern "C" int fp8bs_moe_combine(const uint16_t* y, int64_t ldy, int64_t rows_cap, const int32_t* slot_rows,
                                 const float* gates, int64_t tokens, int64_t topk, int64_t n, uint16_t* out,
                                 int64_t ldo, void* stream) {
  if ((rows_cap > 0 && !y) || (tokens > 0 && (!slot_rows || !gates || !out))) return FP8BS_ERR_NULL;
  if (tokens < 0 || topk < 1 || topk > kMaxTopk || tokens > 0x7FFFFFFFLL / topk) return FP8BS_ERR_SHAPE;
  if (n <= 0 || n % 8 || n > (1 << 30) || ldy < n || ldo < n || rows_cap < 0 || rows_cap > 0x7FFFFFFFLL)
    return FP8BS_ERR_SHAPE;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(slot_rows, 4) || !aligned(gates, 4) || ldy % 8 ||
      ldo % 8)
    return FP8BS_ERR_ALIGN;
  if (tokens == 0) return FP8BS_OK;
  const int64_t grid = (tokens + 4 * kCombineTPW - 1) / (4 * kCombineTPW);
  if (grid > kMaxGrid) return FP8BS_ERR_SHAPE;
  // the expert rows are streamed when they are larger than half the
  // last-level cache; smaller ones may still be cached from the GEMM that
  // produced them
  if (tokens * topk * n * 2 > kStreamBytes)
    hipLaunchKernelGGL((moe_combine_kernel<kCombineTPW, true>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, y, ldy, rows_cap, slot_rows, gates, tokens, (int)topk, (int)n, out, ldo);
  else
    hipLaunchKernelGGL((moe_combine_kernel<kCombineTPW, false>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, y, ldy, rows_cap, slot_rows, gates, tokens, (int)topk, (int)n, out, ldo);
  return launch_status();
}
