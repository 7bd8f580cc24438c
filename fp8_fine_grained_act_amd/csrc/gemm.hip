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
// Two kernels share the slab layout below: gemm_kernel (128 x 128 or 64 x 128
// tiles, every wave both copies and multiplies, two workgroups per CU; small
// problems, and the grouped GEMM whose n is not a multiple of 256) and
// gemm_ws_kernel (256 x 128, 192 x 128, 128 x 192
// and, for the MoE grouped GEMM, 128 x 256 tiles; separate copy and MFMA
// waves; persistent over tiles where a workgroup gets several; described
// above that kernel).  The host picks the kernel, tile shape and tile order
// (use_ws, tile_cost, choose_group_m).
//
// Structure of one gemm_kernel workgroup (WAVES_M x WAVES_N waves, each wave a
// (BM/WAVES_M) x (BN/WAVES_N) patch of 16x16 MFMA tiles):
//   * K is walked in 128-deep slabs.  A slab of A (BM rows x 128 bytes), of B
//     and of the scales that go with it is copied from memory straight into
//     LDS with buffer_load ... lds (16 or 4 bytes per lane), STAGES slabs in
//     flight; no VGPRs hold staged data, and rows past the matrix edge read as
//     zero (buffer range check).  Each stage is its own LDS object, so the
//     compiler can tell a slab being filled from the slab being read.
//   * LDS rows are 128 bytes of 16-byte chunks, stored with a per-row XOR
//     swizzle of the chunk index (swz, swz_t below) that keeps every LDS pass
//     of the fragment reads on 64 distinct banks.
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

#include <type_traits>

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
  int64_t tiles_m, tiles_n;
  int accumulate;
  int64_t group_m;  // band height in m-tiles of the XCD-aware order; 0 = column-major, -1 = row-major,
                    // -3 = grouped, experts' first m-tiles (tile_coords)
  float* ws;        // split contraction: FP32 partials [ksplit][m][n] (gridDim.y = ksplit)
  int64_t ksplit;
  int stream_out;   // bf16 output larger than half the last-level cache: non-temporal stores
  const int32_t* row_token;  // grouped: the dispatch's row map (-1: padding row), or null
  const uint16_t* w16;       // grouped from bf16 weights: w [experts, n, k] bf16
  uint8_t* qw;               // and their codes / scales written once per expert, or null
  float* sw;
  int tile_sel;              // grouped: 0 every tile, 1 only each expert's first m-tile, 2 the others
  int keep_all;              // grouped from bf16 weights with qw: 1 every expert's codes stored, 0 only
                             // those of experts with several m-tiles (the ones read back)
};

// Expert whose segment holds row m0: the largest e with seg[e] <= m0 (empty
// segments before it share its start and are passed over).
__device__ __forceinline__ int grouped_expert(const GemmArgs& p, int64_t m0) {
  int lo = 0, hi = (int)p.num_experts;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)p.seg[mid] <= m0) lo = mid; else hi = mid - 1;
  }
  return min(lo, (int)p.num_experts - 1);
}

// Rows of a 128-row grouped tile that are read: up to and including its last
// routed row (row_token >= 0); the rows after it are padding, loaded as zeros
// by the clipped buffer ranges with no memory traffic.  Each lane of the wave
// checks two of the tile's 128 entries.
__device__ __forceinline__ int64_t live_rows_128(const int32_t* rt, int lane) {
  const int t0 = rt[2 * lane], t1 = rt[2 * lane + 1];
  const uint64_t b0 = __ballot(t0 >= 0), b1 = __ballot(t1 >= 0);
  const int e0 = b0 ? 2 * (63 - __clzll((long long)b0)) + 1 : 0;
  const int e1 = b1 ? 2 * (63 - __clzll((long long)b1)) + 2 : 0;
  return __builtin_amdgcn_readfirstlane(max(e0, e1));
}

// Workgroups are dealt to the chip's 8 XCDs round-robin by workgroup id, and
// each XCD has its own L2.  With group_m > 0 the id is first remapped so that
// every XCD owns one contiguous range of logical tiles; logical tiles then
// walk down M inside bands of group_m m-tiles, so one XCD's range covers a
// compact block of about group_m tile rows by range/group_m tile columns,
// and the A rows and B columns its L2 must hold stay few.  With group_m = 0
// consecutive workgroups walk down M inside one N column, with -1 along N
// inside one M row.
constexpr int kXcds = 8;
// Tile counts stay below 2^31 (checked at launch), so the index arithmetic
// is 32-bit.  Returned by value: through references from several branches
// the compiler placed (m, n) in scratch memory.
struct TileMN {
  uint32_t m, n;
};
// The order of the experts' first m-tiles (-3) is compiled only into the
// kernel that codes bf16 weights (ORDER), which calls this once per
// workgroup; the other kernels compile as if it did not exist.
template <int ORDER = 0>
__device__ inline TileMN tile_coords(const GemmArgs& p, uint32_t b) {
  const uint32_t tiles_m = (uint32_t)p.tiles_m, tiles_n = (uint32_t)p.tiles_n;
  if (p.group_m == 0) {
    const uint32_t n = b / tiles_m;
    return TileMN{b - n * tiles_m, n};
  }
  if (p.group_m == -1) {            // row-major: all N tiles of one M tile in a row
    const uint32_t m = b / tiles_n;
    return TileMN{m, b - m * tiles_n};
  }
  if (ORDER == -3 && p.group_m == -3) {
    // grouped, each expert's first m-tile only: the XCDs step through the
    // experts eight at a time, each running all N tiles of its expert, so the
    // tile's rows of A are fetched into one L2.  An expert without rows (or
    // past the last) gets the row past the last tile, which the kernel's
    // end-of-rows check sends away.
    const uint32_t j = b / kXcds;
    const uint32_t e = kXcds * (j / tiles_n) + b % kXcds;
    if (e >= (uint32_t)p.num_experts || p.seg[e] == p.seg[e + 1]) return TileMN{tiles_m, 0};
    return TileMN{(uint32_t)p.seg[e] / 128u, j % tiles_n};
  }
  const uint32_t gm = (uint32_t)p.group_m;
  const uint32_t tiles = tiles_m * tiles_n;
  const uint32_t per = (tiles + kXcds - 1) / kXcds;   // XCDs own ranges of per or per - 1 tiles
  const uint32_t full = tiles - kXcds * (per - 1);    // how many own per (1..8)
  const uint32_t x = b % kXcds, j = b / kXcds;
  const uint32_t l = x < full ? x * per + j : full * per + (x - full) * (per - 1) + j;
  const uint32_t band_tiles = gm * tiles_n;
  const uint32_t band = l / band_tiles, r = l - band * band_tiles;
  const uint32_t first = band * gm;
  const uint32_t rows = tiles_m - first < gm ? tiles_m - first : gm;
  const uint32_t n = r / rows;
  return TileMN{first + (r - n * rows), n};
}

constexpr int BK = 128;
// LDS bank layout, measured on gfx950 (bank-conflict counter, one lane pair
// at a time): 64 banks of 4 bytes; ds_read_b128 serves 16 lanes per pass,
// lanes 0-3, 12-15, 20-23 and 24-27 forming one pass (within each half
// wave, the 4-lane groups whose index has even bit parity form one pass and
// the others the second); ds_read_b64 and ds_read_b64_tr_b8 serve 32
// consecutive lanes per pass.  A pass is conflict-free when its lanes cover
// 64 distinct banks.
//
// Operand rows are 128 bytes (8 chunks of 16 bytes); chunk c of row r is
// stored at chunk c ^ h(r).  MFMA fragments read with ds_read_b128 (lane
// group g takes chunks 2g, 2g + 1 of rows l16 = 0..15) are conflict-free with
// h(r) = (r >> 1) & 5: in every pass the even rows, and the odd rows, land on
// 8 distinct chunks.  The dgrad weight slab (rows = k, read with
// ds_read_b64_tr_b8 at rows 32g + 8q + (l16 >> 1)) needs rows r and r + 32
// apart as well: h_t(r) = ((r >> 1) & 3) | ((r >> 3) & 4).  Measured on the
// read patterns alone: 202 B/clk/CU for the fragment reads (113 with the
// earlier (r >> 1) & 7), 147 for the transposing reads (112).
__device__ __forceinline__ int swz_h(int row) { return (row >> 1) & 5; }
__device__ __forceinline__ int swz_ht(int row) { return ((row >> 1) & 3) | ((row >> 3) & 4); }
// byte offset of 16-byte chunk `chunk` of LDS row `row`, fragment layout
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ swz_h(row)) << 4); }
// the same in the dgrad weight layout
__device__ __forceinline__ int swz_t(int row, int chunk) { return row * BK + ((chunk ^ swz_ht(row)) << 4); }



template <int BM, int BN>
struct Stage {
  uint8_t a[BM * BK];
  uint8_t b[BN * BK];
  float sa[BM];
  float sb[BN];
};

// One LDS object per pipeline stage (a separate variable per IDX), so the
// compiler's alias information separates the stage being filled by DMA from
// the stage being read.
template <int BM, int BN, int IDX>
__device__ __forceinline__ Stage<BM, BN>& lds_stage() {
  __shared__ __attribute__((aligned(16))) Stage<BM, BN> st;
  return st;
}

template <int MODE, int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
struct GemmCfg {
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;   // wave patch
  static constexpr int TM = WM / 16, TN = WN / 16;              // MFMA tiles per wave
  // copies per slab: every wave issues A_CP copies of 8 A rows and B_CP copies
  // of 8 B rows (dgrad: 8 k-rows of the [K, N] slab), 1 KB each; the
  // kScaleJobs 64-entry scale copies (A rows first, then B columns) go to
  // waves 0, 1, ... round-robin
  static constexpr int A_CP = BM / 8 / kWaves;
  static constexpr int B_CP = BN / 8 / kWaves;
  static constexpr int kScaleJobs = (BM + BN) / 64;
  static constexpr int kScaleRounds = (kScaleJobs + kWaves - 1) / kWaves;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave patch must be whole MFMA tiles");
  static_assert(A_CP * 8 * kWaves == BM && B_CP * 8 * kWaves == BN, "copies must split evenly over waves");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "scale copies cover 64 rows each");
  static_assert(MODE != kDgrad || BN == 128, "dgrad slab rows are 128 columns wide");
  static_assert(STAGES == 2 || STAGES == 3, "pipeline depth");
  static_assert((STAGES - 1) * (A_CP + B_CP + kScaleRounds) <= 47, "copies in flight must fit the vmcnt waits");
  static __device__ __forceinline__ int jobs_of(int wave) {
    return A_CP + B_CP + kScaleJobs / kWaves + (wave < kScaleJobs % kWaves ? 1 : 0);
  }
};

// bf16 output of one 16-row MFMA group.  The MFMA leaves lane (g, r)
// (g = lane / 16, r = lane % 16) with columns 4g..4g+3 of output row r of
// each 16x16 tile, so storing a tile as it stands writes four 8-byte pieces
// per row.  Two adjacent tiles are stored together instead: a
// v_permlane16_swap per register pair exchanges the first tile's odd
// 16-lane groups with the second tile's even groups, after which lane g holds
// 8 consecutive columns, 16 * (g % 2) + 8 * (g / 2) onwards, of the 32, and one
// store instruction writes each row's 32 columns as 64 contiguous bytes
// (dgrad 4096x7168x1536 71 -> 62 us, forward 4096x32768x512 142 -> 125 us).
// An odd last tile is stored as it stands.  N is a multiple of 128 and c is
// 16-byte aligned with ldc % 8 == 0, so each 8-column piece is whole and aligned.
// An output larger than half the last-level cache (p.stream_out) is stored
// with the non-temporal hint: every CU finishes its equal tiles at about the
// same time, and the hint lets those bursts drain past the L2 (forward
// 4096x32768x512, 268 MB of bf16: 130 -> 116 us; the MoE grouped GEMM's 535 MB
// row capacity 2.24 -> 2.18 ms; an output that fits, such as dgrad's
// 4096x7168, was 5% slower with it).
template <int TN, int TM>
__device__ __forceinline__ void store_row_bf16(const GemmArgs& p, const v4f (&acc)[TN][TM], int j, int64_t row,
                                               int64_t col0, int g) {
  uint16_t* const crow = reinterpret_cast<uint16_t*>(p.c) + row * p.ldc;
#pragma unroll
  for (int i = 0; i + 1 < TN; i += 2) {
    const uint32_t x0 = f32_to_bf16_rne(acc[i][j][0]) | (f32_to_bf16_rne(acc[i][j][1]) << 16);
    const uint32_t x1 = f32_to_bf16_rne(acc[i][j][2]) | (f32_to_bf16_rne(acc[i][j][3]) << 16);
    const uint32_t y0 = f32_to_bf16_rne(acc[i + 1][j][0]) | (f32_to_bf16_rne(acc[i + 1][j][1]) << 16);
    const uint32_t y1 = f32_to_bf16_rne(acc[i + 1][j][2]) | (f32_to_bf16_rne(acc[i + 1][j][3]) << 16);
    const auto s0 = __builtin_amdgcn_permlane16_swap(x0, y0, false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(x1, y1, false, false);
    const int64_t col = col0 + 16 * i + 16 * (g & 1) + 8 * (g >> 1);
    if (col < p.n) {
      const uint4 v = make_uint4(s0[0], s1[0], s0[1], s1[1]);
      if (p.stream_out)
        store_nt(crow + col, v);
      else
        *reinterpret_cast<uint4*>(crow + col) = v;
    }
  }
  if (TN % 2) {
    const int64_t col = col0 + 16 * (TN - 1) + 4 * g;
    if (col < p.n) {
      uint2 o;
      o.x = f32_to_bf16_rne(acc[TN - 1][j][0]) | (f32_to_bf16_rne(acc[TN - 1][j][1]) << 16);
      o.y = f32_to_bf16_rne(acc[TN - 1][j][2]) | (f32_to_bf16_rne(acc[TN - 1][j][3]) << 16);
      *reinterpret_cast<uint2*>(crow + col) = o;
    }
  }
}

template <int MODE, int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) __attribute__((amdgpu_waves_per_eu(1, 2)))
void gemm_kernel(GemmArgs p) {
  using C = GemmCfg<MODE, BM, BN, WAVES_M, WAVES_N, STAGES>;
  constexpr int WM = C::WM, WN = C::WN, TM = C::TM, TN = C::TN;
  constexpr int NW = C::kWaves;


  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int l16 = lane & 15, g = lane >> 4;

  const TileMN tc = tile_coords(p, blockIdx.x);
  const int64_t m0 = (int64_t)tc.m * BM, n0 = (int64_t)tc.n * BN;
  const int64_t M = p.m, N = p.n, K = p.k;
  const int nkb = (int)(K / BK);

  // grouped: a tile at or past the end of the last segment holds no expert's
  // rows (the row capacity can exceed the padded total); the workgroup leaves
  // before its first barrier and writes nothing
  if (MODE == kGrouped && m0 >= (int64_t)p.seg[p.num_experts]) return;

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
  int64_t rows_a = M - m0 < BM ? M - m0 : BM;
  static_assert(MODE != kGrouped || BM == 128, "grouped tiles are the 128-row segment steps");
  if (MODE == kGrouped && p.row_token) rows_a = min(rows_a, live_rows_128(p.row_token + m0, lane));
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

  // ---- one slab's copies ------------------------------------------------------
  // Copy job q of this wave: q < A_CP an A copy (8 rows, 1 KB), then B_CP B
  // copies, then at most kScaleRounds scale copies (64 floats each).
  auto issue_job = [&](int kb, Stage<BM, BN>& s, int q) {
    const uint32_t ks = (uint32_t)kb * BK;
    if (q < C::A_CP) {
      const int j = q * NW + wave;
      const int c = j * 64 + lane, row = c >> 3, pc = c & 7;
      const int lc = pc ^ swz_h(row);
      dma16(ra, s.a + j * 1024, (uint32_t)(row * K + (lc << 4)), ks);
    } else if (q < C::A_CP + C::B_CP) {
      const int j = (q - C::A_CP) * NW + wave;
      const int c = j * 64 + lane, row = c >> 3, pc = c & 7;
      const int lc = pc ^ (MODE == kDgrad ? swz_ht(row) : swz_h(row));
      if (MODE == kDgrad)
        dma16(rb, s.b + j * 1024, (uint32_t)(row * N + (lc << 4)), ks * (uint32_t)N);
      else
        dma16(rb, s.b + j * 1024, (uint32_t)(row * K + (lc << 4)), ks);
    } else {
      const int js = (q - C::A_CP - C::B_CP) * NW + wave;
      if (js < C::kScaleJobs) {
        const int qq = js * 64 + lane;           // scale slot: [0, BM) rows of A, [BM, BM+BN) columns
        if (js * 64 < BM) {
          dma4(rsa, s.sa + js * 64, (uint32_t)(qq * nkb) * 4u, (uint32_t)kb * 4u);
        } else {
          const int col = qq - BM;
          float* dst = s.sb + (js * 64 - BM);
          if (MODE == kWgrad) {
            dma4(rsb, dst, (uint32_t)(col * nkb) * 4u, (uint32_t)kb * 4u);
          } else {
            // weight-block scale of this column (clipped to the last block past the edge)
            const int64_t nb = min((n0 + col) / 128, N / 128 - 1);
            const uint32_t idx = MODE == kDgrad ? (uint32_t)(kb * (N / 128) + nb) : (uint32_t)(nb * nkb + kb);
            dma4(rsb, dst, idx * 4u, 0u);
          }
        }
      }
    }
  };
  constexpr int kJobs = C::A_CP + C::B_CP + C::kScaleRounds;
  auto issue_slab = [&](int kb, Stage<BM, BN>& s) {
#pragma unroll
    for (int q = 0; q < kJobs; ++q) issue_job(kb, s, q);
  };

  // ---- operand fragments of one slab -----------------------------------------
  struct Frags {
    v8i af[TM], bf[TN];
    float wa[TM];
    v4f wb[TN];
  };
  auto read_a = [&](const Stage<BM, BN>& s, int j) -> v8i {
    const int r = WM * wm + 16 * j + l16;
    const uint4 lo = *reinterpret_cast<const uint4*>(&s.a[swz(r, 2 * g)]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&s.a[swz(r, 2 * g + 1)]);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto load_frags = [&](const Stage<BM, BN>& s, Frags& f) {
#pragma unroll
    for (int j = 0; j < TM; ++j) f.af[j] = read_a(s, j);
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      if (MODE == kDgrad) {
        // rows of s.b are k; lane (g, l16) needs k = 32g .. 32g+31 of column WN*wn + 16i + l16
        const int col16 = (WN * wn + 16 * i) >> 4;
        const int half = (l16 & 1) << 3;               // odd lanes: columns +8 .. +15
        v2i part[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 32 * g + 8 * q + (l16 >> 1);
          part[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) v2i*)(&s.b[swz_t(row, col16) + half]));
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
        const float v = s.sb[WN * wn + 16 * i];
        f.wb[i] = v4f{v, v, v, v};
      }
    }
  };

  v4f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // acc[i][j] += (sa * sb) * P for one 16x16 tile of this slab
  auto rescale = [&](const Frags& f, int i, int j, const v4f& P) {
    if (MODE == kWgrad) {
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(f.wa[j] * f.wb[i][v], P[v], acc[i][j][v]);
    } else {
      const float w = f.wa[j] * f.wb[i][0];
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(w, P[v], acc[i][j][v]);
    }
  };
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  // every fragment of the slab in registers, then the MFMAs
  auto mfma_phase = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.bf[i], f.af[j], zero, 0, 0, 0, 0, 0, 0);
        rescale(f, i, j, P);
      }
    }
  };

  // ---- pipeline ----------------------------------------------------------------
  // Hand-off of a slab: each wave waits for its own copies of that slab (newer
  // slabs may stay in flight) and for its own LDS reads, then the barrier makes
  // every wave's copies visible and guarantees that no wave still reads the
  // stage that is refilled next.
  const int my_jobs = C::jobs_of(wave);
  auto publish = [&](int newer_slabs_in_flight) {
    wait_vmcnt_dyn(newer_slabs_in_flight * my_jobs);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto stage_ref = [&](int s) -> Stage<BM, BN>& {
    if (STAGES == 3 && s == 2) return lds_stage<BM, BN, (STAGES == 3 ? 2 : 1)>();
    return s == 0 ? lds_stage<BM, BN, 0>() : lds_stage<BM, BN, 1>();
  };

  // prologue: slabs 0 .. STAGES-1 in flight
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nkb) issue_slab(s, stage_ref(s));

  // publish slab kb, read its fragments, refill the stage of slab kb-1 (read
  // by every wave before this barrier), run slab kb's MFMAs
  for (int kb0 = 0; kb0 < nkb; kb0 += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      const int kb = kb0 + u;
      if (kb < nkb) {
        // slabs issued so far: 0 .. STAGES-1 (prologue) and kb-2+STAGES
        // (refills), so slab kb has min(STAGES-1 (first) or STAGES-2, rest)
        // newer copies behind it
        publish(kb == 0 ? min(STAGES - 1, nkb - 1) : min(STAGES - 2, nkb - kb - 1));
        Frags f;
        load_frags(stage_ref(u), f);
        if (kb >= 1 && kb - 1 + STAGES < nkb) issue_slab(kb - 1 + STAGES, stage_ref((u + STAGES - 1) % STAGES));
        mfma_phase(f);
      }
    }
  }

  // ---- epilogue --------------------------------------------------------------
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int64_t row = m0 + WM * wm + 16 * j + l16;
    if (row >= M) continue;
    if (MODE != kWgrad) {
      store_row_bf16<TN, TM>(p, acc, j, row, n0 + WN * wn, g);
      continue;
    }
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int64_t col = n0 + WN * wn + 16 * i + 4 * g;
      if (col >= N) continue;
      float* dst = reinterpret_cast<float*>(p.c) + row * p.ldc + col;
      float4 o = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      if (p.accumulate) {
        const float4 old = *reinterpret_cast<const float4*>(dst);
        o.x += old.x; o.y += old.y; o.z += old.z; o.w += old.w;
      }
      *reinterpret_cast<float4*>(dst) = o;
    }
  }
}

// Band height of the XCD-aware tile order (tile_coords).  Each XCD fetches
// the A tile rows and B tile columns its range of tiles touches; this picks
// the height (1..32 m-tiles) that minimises their sum, BM and BN bytes per
// k-byte of a tile row and column, counted exactly per range.  Problems whose
// output outweighs twice their operands keep the plain order: there the
// banded order leaves the XCDs writing narrow column windows a fixed stride
// apart, which measured up to 2x slower on a 4096 x 32768 x 512 forward GEMM
// (the order changes nothing else for them).
static int64_t range_cost(int64_t tiles_m, int64_t tiles_n, int64_t bm, int64_t bn, int64_t gm) {
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t per = (tiles + kXcds - 1) / kXcds, full = tiles - kXcds * (per - 1);
  const int64_t band_tiles = gm * tiles_n;
  int64_t cost = 0, l = 0;
  for (int x = 0; x < kXcds; ++x) {
    int64_t l0 = l;
    const int64_t l1 = l + (x < full ? per : per - 1);
    l = l1;
    while (l0 < l1) {                       // pieces of the range, one per band
      const int64_t band = l0 / band_tiles, first = band * gm;
      const int64_t rows = tiles_m - first < gm ? tiles_m - first : gm;
      const int64_t a = l0 - band * band_tiles;
      const int64_t b = l1 - band * band_tiles < rows * tiles_n ? l1 - band * band_tiles : rows * tiles_n;
      const int64_t cols = (b - 1) / rows - a / rows + 1;
      const int64_t rws = rows < b - a ? rows : b - a;
      cost += rws * bm + cols * bn;
      l0 = band * band_tiles + b;
    }
  }
  return cost;
}
static int64_t choose_group_m(const GemmArgs& a, int64_t bm, int64_t bn, int64_t out_bytes) {
  const int64_t tiles_m = a.tiles_m, tiles_n = a.tiles_n;
  if ((double)a.m * (double)a.n * (double)out_bytes > 2.0 * (double)(a.m + a.n) * (double)a.k) return 0;
  int64_t best = 1, best_cost = -1;
  const int64_t hi = tiles_m < 32 ? tiles_m : 32;
  for (int64_t gm = 1; gm <= hi; ++gm) {
    const int64_t c = range_cost(tiles_m, tiles_n, bm, bn, gm);
    if (best_cost < 0 || c < best_cost) best = gm, best_cost = c;
  }
  return best;
}

template <int MODE, int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
static int launch_gemm(GemmArgs a, hipStream_t s) {
  a.tiles_n = (a.n + BN - 1) / BN;
  a.tiles_m = (a.m + BM - 1) / BM;
  // grouped GEMM: row-major, so an M tile's rows (one expert's tokens) stay
  // in L2 across its N tiles and the expert's next M tile follows one row of
  // tiles later, while that expert's weight columns are still cached
  // (measured on 256 experts of 4096x7168: 4.09 -> 2.55 ms against the
  // column-major order, which re-reads every expert's rows once per N tile)
  a.group_m = MODE == kGrouped ? -1 : choose_group_m(a, BM, BN, MODE == kWgrad ? 4 : 2);
  const int64_t grid = a.tiles_m * a.tiles_n;
  if (grid > kMaxGrid) return FP8BS_ERR_SHAPE;
  hipLaunchKernelGGL((gemm_kernel<MODE, BM, BN, WAVES_M, WAVES_N, STAGES>), dim3((unsigned)grid),
                     dim3(64 * WAVES_M * WAVES_N), 0, s, a);
  return launch_status();
}

// ---------------------------------------------------------------------------
// Copy waves of the grouped GEMM whose expert weights arrive in bf16.
//
// A slab unit (k-block kb of the tile) holds the A slab and its row scales,
// copied by DMA as in the FP8 path (each copy wave a quarter), and the tile's
// 256 weight rows n0 .. n0 + 255 over the same 128 columns: two 128 x 128
// weight blocks, coded here with the arithmetic of quant_w_kernel (the same
// block amax, group_scale and quant4_path), so the codes and scales equal the
// 128x128 block quantizer's bit for bit.  Copy wave c codes rows 64c .. 64c +
// 63, half (c & 1) of block c >> 1.  Lane (r4, j) = (lane / 16, lane % 16)
// holds rows 64c + r4 + 4i (i < 16), bf16 columns 8j .. 8j + 7: one 16-byte
// load per row, 4 rows' 256 contiguous bytes per load instruction; its 8
// codes of a row go to half j % 2 of LDS chunk j / 2 (the swz layout the DMA
// writes), and the weight-column scales of the slab to sb.
//
// A block's scale needs the amax of both halves.  Each wave writes its half's
// maximum to LDS one barrier before the block is coded: the maxima of unit
// v + 1 are written before barrier v (the barrier that publishes unit v), and
// both waves code unit v + 1 between barriers v and v + 1.  A wave so holds
// the bf16 of two units (2 x 64 VGPRs): unit v + 1 being coded while unit
// v + 2 loads.  One barrier more than the FP8 path, before barrier 0, lets
// the maxima of unit 0 cross; the MFMA waves pass it too.
//
// With qw / sw, the expert's first tile (the one at its segment start) also
// stores the codes and block scales there: those of every expert with rows
// (keep_all, codes kept for the GEMMs that follow, such as a backward's
// dgrad), or only those of experts with several m-tiles, whose other m-tiles
// read them back in the call's second launch.
// ---------------------------------------------------------------------------
// a wave-uniform float moved to a scalar register
__device__ __forceinline__ float uniform_f32(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

template <int BM, int BN>
__device__ __forceinline__ void copy_waves_bf16_weights(const GemmArgs& p, int c, int lane, int units,
                                                        int64_t m0, int64_t n0, Stage<BM, BN>& st0,
                                                        Stage<BM, BN>& st1, Stage<BM, BN>& st2) {
  static_assert(BM == 128 && BN == 256, "two weight blocks per slab, one 64-row half per copy wave");
  __shared__ uint32_t half_amax[2][4];         // [unit parity][copy wave]
  const int64_t M = p.m, N = p.n, K = p.k;
  const int nkb = (int)(K / BK);
  constexpr int A_CP = BM / 8 / 4, SA_JOBS = BM / 64;
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

  const int e = grouped_expert(p, m0);
  int64_t rows_a = M - m0 < BM ? M - m0 : BM;
  if (p.row_token) rows_a = min(rows_a, live_rows_128(p.row_token + m0, lane));
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.qa + m0 * K, rows_a * K);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.sa + m0 * nkb, rows_a * nkb * 4);
  const int crow = 8 * c + (lane >> 3);
  const uint32_t voff_a = (uint32_t)(crow * K + (((lane & 7) ^ swz_h(crow)) << 4));
  const uint32_t voff_sa = (uint32_t)((64 * c + lane) * nkb) * 4u;

  const int j = lane & 15;
  const int wrow = 64 * c + (lane >> 4);       // the lane's first weight row in the tile
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w16 + ((int64_t)e * N + n0) * K, (int64_t)BN * K * 2);
  const uint32_t voff_w = (uint32_t)((wrow * K + 8 * j) * 2);
  const bool store_q = p.qw != nullptr && m0 == (int64_t)p.seg[e] &&
                       (p.keep_all || (int64_t)p.seg[e + 1] - m0 > BM);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qw + ((int64_t)e * N + n0) * K, store_q ? (int64_t)BN * K : 0);
  const uint32_t voff_q = (uint32_t)(wrow * K + 8 * j);

  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // bf16 weights are read once per tile: loads with the non-temporal hint
  // (and so are the code stores), which keeps the re-read A rows in the caches
  constexpr int kNT = 2;
  auto load_row = [&](int kb, int i) -> uint4 {
    const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)voff_w, (4 * i * (int)K + kb * BK) * 2, kNT);
    return make_uint4(t.x, t.y, t.z, t.w);
  };
  auto load_w = [&](int kb, uint4 (&b)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) b[i] = load_row(kb, i);
  };
  auto issue_a = [&](int kb, Stage<BM, BN>& s) {
    const uint32_t ks = (uint32_t)kb * BK;
#pragma unroll
    for (int i = 0; i < A_CP; ++i)                                  // A copies j = c + 4i
      dma16(ra, s.a + (c + 4 * i) * 1024, voff_a, ks + (uint32_t)(32 * i) * (uint32_t)K);
    if (c < SA_JOBS) dma4(rsa, s.sa + 64 * c, voff_sa, (uint32_t)kb * 4u);
  };
  auto post_half_max = [&](int kb, const uint4 (&b)[16]) {
    constexpr uint32_t kMag = 0x7FFF7FFFu;
    uint32_t m2 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      m2 = max_u16x2(m2, max_u16x2(max_u16x2(b[i].x & kMag, b[i].y & kMag), max_u16x2(b[i].z & kMag, b[i].w & kMag)));
    const uint32_t m = wave_max_u32(max(m2 & 0xFFFFu, m2 >> 16));
    if (lane == 0) half_amax[kb & 1][c] = m;
  };
  // quant4_path with the tiny-tile factor as a multiplier (1 or 2^64): one
  // code path for both (a product with 1 is exact, so the codes are the same).
  // The magnitudes come from the abs source modifier of the first multiply,
  // the signs from the bf16 sign bits; the first conversion's upper half is a
  // placeholder (x01) that the second overwrites.
  auto quant4 = [&](uint32_t x01, uint32_t x23, const GroupScale& gs, float mul) -> uint32_t {
    const float a[4] = {bf16_lo(x01), bf16_hi(x01), bf16_lo(x23), bf16_hi(x23)};
    float qv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float ai = __builtin_fabsf(a[t]) * mul;
      qv[t] = __builtin_fmaf(ai, gs.r, ai * gs.rl);
    }
    int d = __builtin_amdgcn_cvt_pk_fp8_f32(qv[0], qv[1], (int)x01, false);
    d = __builtin_amdgcn_cvt_pk_fp8_f32(qv[2], qv[3], d, true);
    return (uint32_t)d | (__builtin_amdgcn_perm(x23, x01, 0x07050301u) & 0x80808080u);
  };
  // code unit kb from b into stage s; with LOAD, load rows 2i, 2i + 1 of unit
  // kn into next beside the coding of row i < 8 (the loads go out in the first
  // half of the coding, so most of their latency passes under the second)
  auto code = [&](auto load_tag, int kb, const uint4 (&b)[16], Stage<BM, BN>& s, uint4 (&next)[16], int kn) {
    constexpr bool LOAD = decltype(load_tag)::value;
    // the block's scale is the same in every lane: kept in scalar registers
    GroupScale gs = group_scale(max(half_amax[kb & 1][c], half_amax[kb & 1][c ^ 1]));
    gs.r = uniform_f32(gs.r);
    gs.rl = uniform_f32(gs.rl);
    const float mul = uniform_f32(gs.slow ? kTinyScale : 1.0f);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (LOAD && i < 8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) next[2 * i + h] = load_row(kn, 2 * i + h);
      }
      const int row = wrow + 4 * i;
      uint2 o;
      o.x = quant4(b[i].x, b[i].y, gs, mul);
      o.y = quant4(b[i].z, b[i].w, gs, mul);
      *reinterpret_cast<uint2*>(s.b + row * BK + (((j >> 1) ^ swz_h(row)) << 4) + ((j & 1) << 3)) = o;
      if (store_q) {
        const u32x2_t w2 = {o.x, o.y};
        __builtin_amdgcn_raw_buffer_store_b64(w2, rq, (int)voff_q, 4 * i * (int)K + kb * BK, kNT);
      }
      __builtin_amdgcn_sched_barrier(0);       // keep row i's load beside row i's coding
    }
    s.sb[64 * c + lane] = gs.s;
    if (store_q && (c & 1) == 0 && lane == 0)
      p.sw[((int64_t)e * (N / 128) + n0 / 128 + (c >> 1)) * nkb + kb] = gs.s;
  };

  uint4 b0[16], b1[16];
  // prologue: unit 0 loaded, its maxima cross the extra barrier
  load_w(0, b0);
  issue_a(0, st0);
  wait_vmcnt<0>();
  post_half_max(0, b0);
  __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0): the maximum is in LDS
  barrier();
  // phase v, between barriers v and v + 1 (phase -1 ends at barrier 0): start
  // unit v + 2 (weights into the registers unit v left, A into the stage slab
  // v - 1 left), code unit v + 1, post the maxima of unit v + 2
  // the stage of unit v (wave-uniform: a scalar select between the three)
  auto stage = [&](int v) -> Stage<BM, BN>& {
    const int r = v % 3;
    return r == 0 ? st0 : (r == 1 ? st1 : st2);
  };
  auto phase = [&](int v, const uint4 (&b_code)[16], uint4 (&b_load)[16]) {
    if (v + 2 < units && v + 1 < units) {
      // the loads of unit v + 2 between the rows of unit v + 1's coding: a
      // wave that issues its 16 loads at once is held by the queue of the
      // CU's address unit, and its coding would wait behind them (256
      // experts of 4096 x 7168, codes stored: 6.66 ms all at once, 5.92 ms
      // one load per row, 5.6 ms two per row over the first 8 rows with the
      // non-temporal hint)
      issue_a(v + 2, stage(v + 2));
      code(std::true_type{}, v + 1, b_code, stage(v + 1), b_load, v + 2);
    } else {
      if (v + 2 < units) {
        load_w(v + 2, b_load);
        issue_a(v + 2, stage(v + 2));
      }
      if (v + 1 < units) code(std::false_type{}, v + 1, b_code, stage(v + 1), b_load, 0);
    }
    wait_vmcnt<0>();
    if (v + 2 < units) post_half_max(v + 2, b_load);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    barrier();                                 // barrier v + 1
  };
  for (int v = -1; v < units; v += 2) {        // the register buffers alternate
    phase(v, b0, b1);
    if (v + 1 < units) phase(v + 1, b1, b0);
  }
}

// ---------------------------------------------------------------------------
// Warp-specialized tiles: MW MFMA waves (4 or 8) + 4 copy waves.
//
// Measured on gfx950: a copy of 1 KB (buffer_load ... lds or a plain vector
// load) holds its wave for ~70-100 issue cycles, so a wave that both copies
// and multiplies spends most of a slab issuing copies, and the MFMA pipe
// idles while the waves of a workgroup copy in lockstep.  The MFMAs of one
// wave per SIMD, on the other hand, run at the full rate (one 16x16x128 FP8
// MFMA per 32 cycles) while another wave on the same SIMD copies, loads or
// reads LDS.  So the roles are split: the MFMA waves only read fragments and
// run MFMAs and the per-block fold; the last 4 waves (one per SIMD) only copy
// slabs into a 3-deep LDS ring (each stage its own LDS object, so the
// compiler sees that a copy never touches the slab being read).
//
// Barriers (forward, weight gradient): the MFMA waves multiply slab kb and,
// in its last 16-row group, once every LDS read of slab kb has returned, pass
// barrier kb + 1 and read the head of slab kb + 1 (its B fragments, first A
// fragment and scales) between that group's MFMAs, so no slab starts with an
// LDS round trip.  Between barriers kb and kb + 1 the copy waves start the
// copies of slab kb + 2 into the stage slab kb - 1 left (fully read before
// barrier kb), then wait until their copies of slab kb + 1 have landed.
// Every wave passes nkb + 1 barriers.  dgrad passes barrier kb at the start
// of slab kb instead (nkb barriers), see kEarly.
//
// Fragment reads: A rows (and B rows in the forward / weight-gradient
// layouts) are 128-byte LDS rows of 16-byte chunks in the swz layout; the
// activation-gradient B slab is stored as copied ([k][n], swz_t layout) and
// gathered with ds_read_b64_tr_b8 as in gemm_kernel.
// ---------------------------------------------------------------------------
template <int MODE, int MW, int BM, int BN, bool PERSIST, bool SPLIT = false, bool W16 = false>
__global__ __launch_bounds__(64 * (MW + 4)) void gemm_ws_kernel(GemmArgs p) {
  // MW MFMA waves: 4 (one per SIMD) or 8 (two per SIMD, so one wave's fold
  // VALU work runs under the other's MFMAs; register budget 168 per lane for
  // three waves per SIMD).  Tiles: 256 x 128 or 192 x 128 (launcher's choice,
  // tile_cost), 128 x 192 for forward GEMMs whose larger tiles leave CUs idle,
  // and 128 x 256 for the grouped GEMM, whose expert segments come in 128-row
  // steps.  Wave grid: BN / 64 waves across N (patches 64 wide), except
  // 192-wide tiles: 2 waves of 96 columns (MW = 4) or 4 of 48 (MW = 8).
  constexpr int WAVES_N = BN == 192 ? (MW == 4 ? 2 : 4) : BN / 64;
  constexpr int WAVES_M = MW / WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, TM = WM / 16, TN = WN / 16;
  // a patch narrower or wider than 64 columns can straddle a 128-column
  // weight block: then each 16-column MFMA tile takes its own weight scale
  constexpr bool kWbPerTile = MODE != kWgrad && WN != 64;
  constexpr int A_CP = BM / 8 / 4;            // A copies (8 rows each) per copy wave
  constexpr int B_CP = BN / 8 / 4;            // B copies per copy wave
  constexpr int SA_JOBS = BM / 64;            // 64-row scale copies of A
  constexpr int SB_JOBS = BN / 64;            // 64-column scale copies of B
  static_assert(MODE == kFprop || MODE == kDgrad || MODE == kWgrad || MODE == kGrouped, "mode");
  static_assert(MW == 4 || MW == 8, "MFMA wave count");
  static_assert((BN == 128 && (BM == 256 || BM == 192)) ||
                    ((BN == 256 || BN == 192) && BM == 128 && MODE != kDgrad),
                "tile shape");
  static_assert(WAVES_M * WAVES_N == MW && WM % 16 == 0, "whole MFMA tiles per wave");
  static_assert(!W16 || (MODE == kGrouped && !PERSIST && !SPLIT && BM == 128 && BN == 256 && MW == 8),
                "bf16 weights: grouped 128 x 256 tiles");

  Stage<BM, BN>& st0 = lds_stage<BM, BN, 0>();
  Stage<BM, BN>& st1 = lds_stage<BM, BN, 1>();
  Stage<BM, BN>& st2 = lds_stage<BM, BN, 2>();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar registers
  const int l16 = lane & 15, g = lane >> 4;

  // Persistent: workgroup w takes tiles w, w + G, w + 2G, ... (G = gridDim.x,
  // a multiple of 8 whenever a workgroup gets more than one tile, so all its
  // tiles stay on its own XCD and tile_coords' XCD-aware order holds) and
  // walks them as one sequence of slab units: unit u is slab u % nkb of its
  // (u / nkb)-th tile.  The LDS ring and the barriers run across tile
  // boundaries, so the next tile's first slabs are copied while the MFMA
  // waves store the previous tile.
  const int64_t M = p.m, N = p.n, K = p.k;
  const int nkb = (int)(K / BK);               // K blocks of a row (the width of the scale rows)
  // SPLIT: workgroup (x, y) runs slabs [y * nslab, (y + 1) * nslab) of tile x
  // and stores its FP32 partial to ws[y]; a second kernel sums the partials
  static_assert(!SPLIT || (MODE != kGrouped && !PERSIST), "split contraction: plain tiles");
  const int nslab = SPLIT ? nkb / (int)p.ksplit : nkb;
  const int kb0 = SPLIT ? (int)blockIdx.y * nslab : 0;
  // PERSIST = false: one tile per workgroup (grid = tiles), with the tile
  // bookkeeping and the store outside the slab loop, which keeps the MFMA
  // waves' registers as in a plain kernel.
  const int64_t G = gridDim.x;
  const int my_tiles = PERSIST ? (int)((p.tiles_m * p.tiles_n - 1 - (int64_t)blockIdx.x) / G + 1) : 1;
  const int units = my_tiles * nslab;
  struct Origin {
    int64_t m0, n0;
  };
  // grouped (one tile per workgroup): the tile is found once, here
  TileMN grouped_tile{0, 0};
  if constexpr (MODE == kGrouped) grouped_tile = tile_coords<W16 ? -3 : 0>(p, blockIdx.x);
  auto tile_origin = [&](int i) {
    const TileMN t = MODE == kGrouped ? grouped_tile : tile_coords(p, (uint32_t)((int64_t)blockIdx.x + (int64_t)i * G));
    return Origin{(int64_t)t.m * BM, (int64_t)t.n * BN};
  };

  // grouped: a tile at or past the end of the last segment holds no expert's
  // rows (the row capacity can exceed the padded total); the whole workgroup
  // leaves before its first barrier and writes nothing
  static_assert(!(MODE == kGrouped && PERSIST), "grouped tiles are one per workgroup");
  if (MODE == kGrouped && tile_origin(0).m0 >= (int64_t)p.seg[p.num_experts]) return;
  // grouped, split in two launches: the workgroups of the other launch's tiles
  // leave here too (an expert's first m-tile starts at its segment start)
  if (MODE == kGrouped && p.tile_sel != 0) {
    const int64_t m0 = tile_origin(0).m0;
    const bool first = (int64_t)p.seg[grouped_expert(p, m0)] == m0;
    if (first != (p.tile_sel == 1)) return;
  }

  if (wave >= MW) {
    // ======================= copy waves ==========================================
    const int c = wave - MW;
    if constexpr (W16) {
      copy_waves_bf16_weights<BM, BN>(p, c, lane, units, tile_origin(0).m0, tile_origin(0).n0, st0, st1, st2);
      return;
    }
    // per-tile copy state: buffer resources (ranges clip ragged edges to zeros)
    // and the weight-scale offset of this wave's columns
    __amdgpu_buffer_rsrc_t ra, rsa, rb, rsb;
    uint32_t voff_sb = 0;
    const int scol = 64 * c + lane;
    auto set_tile = [&](int i) {
      const Origin o = tile_origin(i);
      const int64_t m0 = o.m0, n0 = o.n0;
      int64_t rows_a = M - m0 < BM ? M - m0 : BM;
      static_assert(MODE != kGrouped || BM == 128, "grouped tiles are the 128-row segment steps");
      if (MODE == kGrouped && p.row_token) rows_a = min(rows_a, live_rows_128(p.row_token + m0, lane));
      const int64_t rows_b = N - n0 < BN ? N - n0 : BN;
      const uint8_t* qb = p.qb;
      const float* sb = p.sb;
      if (MODE == kGrouped) {
        // expert whose segment holds row m0: the largest e with seg[e] <= m0
        int lo = 0, hi = (int)p.num_experts;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if ((int64_t)p.seg[mid] <= m0) lo = mid; else hi = mid - 1;
        }
        lo = min(lo, (int)p.num_experts - 1);
        qb += (int64_t)lo * N * K;
        sb += (int64_t)lo * (N / 128) * nkb;
      }
      ra = make_rsrc(p.qa + m0 * K, rows_a * K);
      rsa = make_rsrc(p.sa + m0 * nkb, rows_a * nkb * 4);
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
      if (MODE == kWgrad) {
        voff_sb = (uint32_t)(scol * nkb) * 4u;
      } else {
        const int64_t nb = min((n0 + scol) / 128, N / 128 - 1);   // clipped past the edge
        voff_sb = (uint32_t)(MODE == kDgrad ? nb : nb * nkb) * 4u;
      }
    };
    // A copy j (8 rows of 128 bytes) = 64 lanes x 16 bytes; lane (row r8,
    // chunk pc) writes LDS chunk pc of row 8j + r8 from global chunk
    // pc ^ swz_h(row).  This wave copies j = c + 4i, rows 8c + 32i + r8,
    // whose swizzle does not depend on i, so one lane offset serves every
    // copy and the copy index goes into the scalar offset.  The dgrad weight
    // slab is copied in blocks instead (rows 32c + 8i + r8), for which
    // swz_ht does not depend on i.
    const int crow = 8 * c + (lane >> 3);
    const int cchunk = (lane & 7) ^ swz_h(crow);
    const uint32_t voff_a = (uint32_t)(crow * K + (cchunk << 4));
    const int crow_t = 32 * c + (lane >> 3);
    const int cchunk_t = (lane & 7) ^ swz_ht(crow_t);
    const uint32_t voff_b = MODE == kDgrad ? (uint32_t)(crow_t * N + (cchunk_t << 4)) : voff_a;
    // scale jobs: wave c < SA_JOBS copies A rows 64c .. 64c+63, wave
    // c < SB_JOBS also B columns 64c .. 64c+63 (voff_sb, set per tile)
    const uint32_t voff_sa = (uint32_t)((64 * c + lane) * nkb) * 4u;
    const int my_jobs = A_CP + B_CP + (c < SA_JOBS ? 1 : 0) + (c < SB_JOBS ? 1 : 0);
    auto issue = [&](int kb, Stage<BM, BN>& s) {
      const uint32_t ks = (uint32_t)kb * BK;
#pragma unroll
      for (int i = 0; i < A_CP; ++i)                                // A copies j = c + 4i
        dma16(ra, s.a + (c + 4 * i) * 1024, voff_a, ks + (uint32_t)(32 * i) * (uint32_t)K);
#pragma unroll
      for (int i = 0; i < B_CP; ++i) {                              // B copies j = c + 4i (dgrad: 4c + i)
        if (MODE == kDgrad)
          dma16(rb, s.b + (4 * c + i) * 1024, voff_b, (ks + (uint32_t)(8 * i)) * (uint32_t)N);
        else
          dma16(rb, s.b + (c + 4 * i) * 1024, voff_b, ks + (uint32_t)(32 * i) * (uint32_t)K);
      }
      if (c < SA_JOBS) dma4(rsa, s.sa + 64 * c, voff_sa, (uint32_t)kb * 4u);
      if (c < SB_JOBS) {
        if (MODE == kDgrad)
          dma4(rsb, s.sb + 64 * c, voff_sb, (uint32_t)kb * (uint32_t)(N / 128) * 4u);
        else
          dma4(rsb, s.sb + 64 * c, voff_sb, (uint32_t)kb * 4u);
      }
    };
    auto barrier = [&]() {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    // units are issued in order: tile `it`, slab `ikb` next
    int it = 0, ikb = 0;
    set_tile(0);
    auto issue_next = [&](Stage<BM, BN>& s) {
      if (PERSIST && ikb == nslab) {
        ikb = 0;
        set_tile(++it);
      }
      issue(kb0 + ikb++, s);
    };
    // prologue: units 0 and 1; unit 0 landed before the first barrier
    issue_next(st0);
    if (units > 1) {
      issue_next(st1);
      wait_vmcnt_dyn(my_jobs);
    } else {
      wait_vmcnt<0>();
    }
    barrier();
    // with the early head the MFMA waves pass the prologue barrier plus one
    // per unit (in its last group), else one per unit (at its start); the
    // copy waves pass the prologue barrier plus one per phase, except the
    // last phase in the second case
    constexpr bool kEarly = MODE != kDgrad;
    auto phase = [&](int u, Stage<BM, BN>& fill) {
      if (u + 2 < units) {
        issue_next(fill);
        wait_vmcnt_dyn(my_jobs);                                    // unit u + 1 landed
      } else {
        wait_vmcnt<0>();
      }
      if (kEarly || u + 1 < units) barrier();
    };
    for (int u = 0; u < units; u += 3) {
      phase(u, st2);
      if (u + 1 < units) phase(u + 1, st0);
      if (u + 2 < units) phase(u + 2, st1);
    }
    return;
  }

  // ========================= MFMA waves ==========================================
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int ra0 = WM * wm + l16, rb0 = WN * wn + l16;
  // rows ra0 + 16t share ra0's swizzle, so tile t adds 16t rows
  const int a_lo = swz(ra0, 2 * g), a_hi = swz(ra0, 2 * g + 1);
  const int b_lo = swz(rb0, 2 * g), b_hi = swz(rb0, 2 * g + 1);
  auto frag = [&](const uint8_t* base, int lo, int hi, int t) -> v8i {
    const uint4 x = *reinterpret_cast<const uint4*>(base + lo + t * 16 * BK);
    const uint4 y = *reinterpret_cast<const uint4*>(base + hi + t * 16 * BK);
    return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  };
  // dgrad: rows of the B slab are k; lane (g, l16) gathers k = 32g .. 32g+31 of
  // column WN*wn + 16i + l16 with ds_read_b64_tr_b8
  auto frag_b_tr = [&](const uint8_t* base, int i) -> v8i {
    const int col16 = (WN * wn + 16 * i) >> 4;
    const int half = (l16 & 1) << 3;
    v2i part[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 32 * g + 8 * q + (l16 >> 1);
      part[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i*)(base + swz_t(row, col16) + half));
    }
    return v8i{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
  };

  v4f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // The head of a slab: what its first 16-row groups need (all B fragments,
  // the first two A fragments and row scales, the column scales).  A
  // fragments are read two groups ahead of their MFMAs (one group, 3-4 MFMAs,
  // is shorter than an LDS round trip under load).  With the early head the
  // slab's A fragments and scales are read right after the barrier that
  // publishes it, while the MFMAs of the previous slab's last group still
  // run, and each B fragment (with its column scales) is read into the
  // registers of the previous slab's fragment i right after that fragment's
  // last MFMA, so the head is never held twice (this frees the registers the
  // deeper A prefetch takes: forward 4096x1536x7168 52 -> 51 us, weight
  // gradient over 16384 tokens 235 -> 228 us).
  struct Head {
    v8i bf[TN];
    v8i a0, a1;
    float wa0, wa1;
    float wb0;      // forward / dgrad: one weight block covers the patch's columns
    float wbs[TN];  // or one per 16-column MFMA tile (kWbPerTile)
    v4f wb[TN];     // weight gradient: a scale per column
  };
  // reads in the order of first use: B fragment 0 and A fragment 0 (the
  // first MFMA), the scales (its fold), then the other B fragments
  auto read_head = [&](const Stage<BM, BN>& s) {
    Head h;
    h.bf[0] = MODE == kDgrad ? frag_b_tr(s.b, 0) : frag(s.b, b_lo, b_hi, 0);
    h.a0 = frag(s.a, a_lo, a_hi, 0);
    h.wa0 = s.sa[WM * wm + l16];
    h.a1 = frag(s.a, a_lo, a_hi, TM > 1 ? 1 : 0);
    h.wa1 = s.sa[WM * wm + (TM > 1 ? 16 : 0) + l16];
    if (MODE == kWgrad) {
#pragma unroll
      for (int i = 0; i < TN; ++i) h.wb[i] = *reinterpret_cast<const v4f*>(&s.sb[WN * wn + 16 * i + 4 * g]);
      h.wb0 = 0.f;
    } else {
      h.wb0 = kWbPerTile ? 0.f : s.sb[WN * wn];
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        h.wbs[i] = kWbPerTile ? s.sb[WN * wn + 16 * i] : 0.f;
        h.wb[i] = v4f{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int i = 1; i < TN; ++i) h.bf[i] = MODE == kDgrad ? frag_b_tr(s.b, i) : frag(s.b, b_lo, b_hi, i);
    return h;
  };
  // LDS instructions of one head, spread over the MFMAs of the group that
  // reads it (issued all at once they queue behind each other and hold up
  // that group's MFMAs)
  constexpr int kHeadReads = (MODE == kDgrad ? 4 * TN : 2 * TN) + 2 * (2 + 1) + (MODE == kWgrad || kWbPerTile ? TN : 1);
  constexpr int kHeadPerMfma = (kHeadReads + TN - 1) / TN;
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Rescale lag: the partial of each MFMA tile is folded into its accumulator
  // after the next MFMA has been issued (its result is ready by then); the
  // lag runs across slabs, so a slab's first MFMA also has independent VALU
  // work beside it.  pw (times pwb per column for the weight gradient) is the
  // pending partial's weight, (pi, pj) its tile.
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f P_prev = zero;
  float pw = 0.f;
  v4f pwb = zero;
  auto fold = [&](int i, int j) {
    if (MODE == kWgrad) {
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(pw * pwb[v], P_prev[v], acc[i][j][v]);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(pw, P_prev[v], acc[i][j][v]);
    }
  };

  // Early head (forward, weight gradient): barrier kb + 1 sits in the last
  // group of slab kb and the head of slab kb + 1 is read under that group's
  // MFMAs.  dgrad keeps the barrier at the start of each slab: its head is
  // 16 transposing LDS reads, more than one group's MFMAs hide, and it
  // measured 7% slower with the early head.
  constexpr bool kEarly = MODE != kDgrad;
  if (W16) barrier();                          // the copy waves' exchange of slab 0's block maxima
  Head hd;
  if (kEarly) {
    barrier();                                 // slab 0 landed
    hd = read_head(st0);
  }

  // Slab kb from stage s; the last group passes barrier kb + 1 (every LDS read
  // of slab kb has returned by then, so the copy waves may refill its stage)
  // and reads the head of slab kb + 1 from stage sn (A fragments and scales
  // first, then each B fragment after its last MFMA here).  After the final
  // slab that head is never used.
  auto slab = [&](const Stage<BM, BN>& s, const Stage<BM, BN>& sn) {
    if (!kEarly) {
      barrier();
      hd = read_head(s);
    }
    v8i a_cur = hd.a0, a_n1 = hd.a1;
    float wa_cur = hd.wa0, wa_n1 = hd.wa1;
    v8i na0 = a_cur, na1 = a_n1;
    float nwa0 = 0.f, nwa1 = 0.f, nwb0 = 0.f;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const bool last = j + 1 == TM;
      v8i a_n2 = a_n1;
      float wa_n2 = wa_n1;
      if (j + 2 < TM) {
        a_n2 = frag(s.a, a_lo, a_hi, j + 2);
        wa_n2 = s.sa[WM * wm + 16 * (j + 2) + l16];
      } else if (last && kEarly) {
        __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0): slab kb fully read
        barrier();
        na0 = frag(sn.a, a_lo, a_hi, 0);
        nwa0 = sn.sa[WM * wm + l16];
        nwb0 = (MODE == kWgrad || kWbPerTile) ? 0.f : sn.sb[WN * wn];
        na1 = frag(sn.a, a_lo, a_hi, TM > 1 ? 1 : 0);
        nwa1 = sn.sa[WM * wm + (TM > 1 ? 16 : 0) + l16];
      }
      const float wj = MODE == kWgrad ? wa_cur : wa_cur * hd.wb0;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int t = j * TN + i;
        const v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(hd.bf[i], a_cur, zero, 0, 0, 0, 0, 0, 0);
        // t = 0 folds the previous slab's last tile (before slab 0: a zero
        // partial of weight 0 into a zero accumulator, which changes nothing)
        if (t > 0) fold((t - 1) % TN, (t - 1) / TN);
        else fold(TN - 1, TM - 1);
        P_prev = P;
        pw = kWbPerTile ? wa_cur * hd.wbs[i] : wj;
        if (MODE == kWgrad) pwb = hd.wb[i];
        if (kEarly && last) {                 // fragment i's last use: refill it for slab kb + 1
          hd.bf[i] = frag(sn.b, b_lo, b_hi, i);
          if (MODE == kWgrad) hd.wb[i] = *reinterpret_cast<const v4f*>(&sn.sb[WN * wn + 16 * i + 4 * g]);
          else if (kWbPerTile) hd.wbs[i] = sn.sb[WN * wn + 16 * i];
        }
      }
      if (!last || !kEarly) {
        if (j + 2 < TM) __builtin_amdgcn_sched_group_barrier(0x0100, 3, 0); // DS reads
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);               // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x0002, MODE == kWgrad ? 8 : 4, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x0100, kHeadPerMfma, 0);
          __builtin_amdgcn_sched_group_barrier(0x0002, MODE == kWgrad ? 8 : 4, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      a_cur = a_n1;
      a_n1 = a_n2;
      wa_cur = wa_n1;
      wa_n1 = wa_n2;
    }
    if (kEarly) {
      hd.a0 = na0;
      hd.a1 = na1;
      hd.wa0 = nwa0;
      hd.wa1 = nwa1;
      hd.wb0 = nwb0;
    }
  };
  // ---- tile end: fold the pending partial, store, start the next tile ------
  Origin org = tile_origin(0);
  auto store_tile = [&]() {
    const int64_t m0 = org.m0, n0 = org.n0;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int64_t row = m0 + WM * wm + 16 * j + l16;
      if (row >= M) continue;
      if (SPLIT) {
        float* prow = p.ws + ((int64_t)blockIdx.y * M + row) * N;
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          const int64_t col = n0 + WN * wn + 16 * i + 4 * g;
          if (col < N)
            *reinterpret_cast<float4*>(prow + col) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      } else if (MODE != kWgrad) {
        store_row_bf16<TN, TM>(p, acc, j, row, n0 + WN * wn, g);
      } else {
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          const int64_t col = n0 + WN * wn + 16 * i + 4 * g;
          if (col >= N) continue;
          float* dst = reinterpret_cast<float*>(p.c) + row * p.ldc + col;
          float4 o = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
          if (p.accumulate) {
            const float4 old = *reinterpret_cast<const float4*>(dst);
            o.x += old.x; o.y += old.y; o.z += old.z; o.w += old.w;
          }
          *reinterpret_cast<float4*>(dst) = o;
        }
      }
      __builtin_amdgcn_sched_barrier(0);     // one row of stores at a time: few live temporaries
    }
  };
  int ti = 0, tkb = 0;
  auto after_slab = [&]() {
    if (!PERSIST || ++tkb < nslab) return;
    fold(TN - 1, TM - 1);
    store_tile();
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = zero;
    P_prev = zero;                             // the next slab's first fold adds nothing
    pw = 0.f;
    pwb = zero;
    tkb = 0;
    if (++ti < my_tiles) org = tile_origin(ti);
  };
  for (int u = 0; u < units; u += 3) {
    slab(st0, st1);
    after_slab();
    if (u + 1 < units) {
      slab(st1, st2);
      after_slab();
    }
    if (u + 2 < units) {
      slab(st2, st0);
      after_slab();
    }
  }
  if (!PERSIST) {
    fold(TN - 1, TM - 1);
    store_tile();
  }
}

// Workgroups of the persistent kernel: one per CU (the LDS ring allows no
// more), a multiple of 8 so every tile of a workgroup stays on its XCD; 0
// when a workgroup's unit count (tiles x K slabs) would not fit an int.
static int64_t persistent_grid(const GemmArgs& a, int cus) {
  const int64_t tiles = a.tiles_m * a.tiles_n;
  int64_t g = cus - cus % kXcds;
  if (g < kXcds) g = kXcds;
  if (tiles < g) g = tiles;
  if (tiles > kMaxGrid || ((tiles + g - 1) / g) * (a.k / BK) >= (int64_t)1 << 31) return 0;
  return g;
}

// MFMA waves per workgroup: two per SIMD for the forward and dgrad GEMMs on
// 256x128 and 192x128 tiles (one wave's fold and LDS reads issue under the
// other's MFMAs; with one wave of twice the patch they ran 9% slower); one
// per SIMD for the weight gradient, whose 8-instruction fold per MFMA does
// not fit 168 VGPRs without spills, and for the 128x192 forward tiles, whose
// 64x96 patches read 29% less LDS per slab than two waves' 64x48 ones
// (4096x1536x7168: 51.3 -> 49.9 us; with the single-slab A prefetch two
// waves per SIMD had been faster, 61.5 against 56.7 us).
template <int MODE, int MW>
static int launch_wide(GemmArgs a, hipStream_t s, int cus) {
  a.tiles_n = (a.n + 191) / 192;
  a.tiles_m = (a.m + 127) / 128;
  a.group_m = choose_group_m(a, 128, 192, 2);
  const int64_t tiles = a.tiles_m * a.tiles_n;
  const int64_t grid = persistent_grid(a, cus);
  if (grid <= 0) return FP8BS_ERR_SHAPE;
  if (grid < tiles)
    hipLaunchKernelGGL((gemm_ws_kernel<MODE, MW, 128, 192, true>), dim3((unsigned)grid), dim3(64 * (MW + 4)), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_ws_kernel<MODE, MW, 128, 192, false>), dim3((unsigned)grid), dim3(64 * (MW + 4)), 0, s, a);
  return launch_status();
}

// Tile shape: rounds of one tile per CU times the tile area times the shape's
// cost per unit of area, smallest wins.  Measured relative costs: 256x128
// 1.0, 192x128 1.1 (smaller MFMA patches read more LDS per MFMA), 128x192
// 1.21 (forward only: 64x48 patches; it pays where 256x128 tiles leave CUs
// idle, forward 4096x1536x7168 56.9 -> 51.7 us).
static int64_t tile_cost(int64_t m, int64_t n, int bm, int bn, int cost100, int cus) {
  const int64_t tiles = ((m + bm - 1) / bm) * ((n + bn - 1) / bn);
  return ((tiles + cus - 1) / cus) * bm * bn * cost100;
}

template <int MODE>
static int launch_gemm_ws(GemmArgs a, hipStream_t s, int cus) {
  constexpr int MW = MODE == kWgrad ? 4 : 8;
  const int64_t c256 = tile_cost(a.m, a.n, 256, 128, 100, cus), c192 = tile_cost(a.m, a.n, 192, 128, 110, cus);
  if (MODE == kFprop && tile_cost(a.m, a.n, 128, 192, 121, cus) < (c256 < c192 ? c256 : c192))
    return launch_wide<kFprop, 4>(a, s, cus);
  a.tiles_n = (a.n + 127) / 128;
  const bool tall = c256 <= c192;
  a.tiles_m = tall ? (a.m + 255) / 256 : (a.m + 191) / 192;
  a.group_m = choose_group_m(a, tall ? 256 : 192, 128, MODE == kWgrad ? 4 : 2);
  const int64_t tiles = a.tiles_m * a.tiles_n;
  int64_t grid = persistent_grid(a, cus);
  if (grid <= 0) return FP8BS_ERR_SHAPE;
  if (MODE == kWgrad && tall) grid = tiles;
  const dim3 block(64 * (MW + 4));
  // the persistent form only where a workgroup gets more than one tile
  // (its in-loop store costs registers: forward 4096x1536x7168, one tile
  // per workgroup, measured 20% slower with it), and not for the weight
  // gradient's 256-row tiles, whose persistent form spills (32768x512 over
  // 4096 tokens: 101 -> 121 us)
  if (grid < tiles) {
    if (tall)
      hipLaunchKernelGGL((gemm_ws_kernel<MODE, MW, 256, 128, true>), dim3((unsigned)grid), block, 0, s, a);
    else
      hipLaunchKernelGGL((gemm_ws_kernel<MODE, MW, 192, 128, true>), dim3((unsigned)grid), block, 0, s, a);
  } else {
    if (tall)
      hipLaunchKernelGGL((gemm_ws_kernel<MODE, MW, 256, 128, false>), dim3((unsigned)grid), block, 0, s, a);
    else
      hipLaunchKernelGGL((gemm_ws_kernel<MODE, MW, 192, 128, false>), dim3((unsigned)grid), block, 0, s, a);
  }
  return launch_status();
}

// Grouped GEMM on 128 x 256 tiles (n % 256 == 0), 8 MFMA waves, row-major
// tile order (see launch_gemm).
template <bool W16 = false>
static int launch_grouped_ws(GemmArgs a, hipStream_t s) {
  a.tiles_n = a.n / 256;
  a.tiles_m = a.m / 128;
  // the launch of only the experts' first m-tiles takes a grid of N tiles
  // per expert (rounded up to whole steps of the eight XCDs)
  if (a.tile_sel == 1 && !W16) return FP8BS_ERR_SHAPE;   // the order is compiled into the bf16 kernel only
  a.group_m = a.tile_sel == 1 ? -3 : -1;
  const int64_t grid = a.tile_sel == 1 ? (a.num_experts + kXcds - 1) / kXcds * kXcds * a.tiles_n
                                       : a.tiles_m * a.tiles_n;
  if (grid > kMaxGrid) return FP8BS_ERR_SHAPE;
  // one tile per workgroup: the persistent form measured 9% slower here
  // (256 experts of 4096x7168), its in-loop store spilling registers
  hipLaunchKernelGGL((gemm_ws_kernel<kGrouped, 8, 128, 256, false, false, W16>), dim3((unsigned)grid),
                     dim3(64 * 12), 0, s, a);
  return launch_status();
}

}  // namespace fp8bs

using namespace fp8bs;

// Kernel choice.  The warp-specialized kernel (gemm_ws_kernel) is the faster
// one per CU, but it runs one large tile per CU; when a problem's 192 x 128
// tiles would cover fewer than half the CUs (a quarter for the weight
// gradient, whose long contraction gains more from the faster kernel than
// it loses to idle CUs), gemm_kernel (smaller tiles, two workgroups per CU)
// keeps more of the chip busy.  Counting 256 x 128 tiles against three
// quarters of the CUs, as before the 192-row tiles existed, sent shapes the
// warp-specialized kernel runs 18-41% faster to gemm_kernel (1536x3584 weight
// gradient over 16384 tokens: 188 -> 110 us; forward 3072x1536x7168: 55.7 ->
// 41.6 us); below a quarter (forward) it loses (768x2048x7168: 35.6 -> 38.9 us).
static bool use_ws(int64_t m, int64_t n, bool wgrad) {
  const int64_t tiles = ((m + 191) / 192) * ((n + 127) / 128);
  return (wgrad ? 4 : 2) * tiles >= cu_count();
}

// Offsets inside one operand are 32-bit (buffer addressing): a tile's rows of
// A or B, and the dgrad weight as a whole, must stay below 4 GiB.
static bool fits_u32(int64_t bytes) { return bytes < 0xFFFFFFFFLL; }

// gemm_kernel tiles: 128 x 128 (2 x 2 waves of 64 x 64, 2 stages) for the
// grouped GEMM whose n is not a multiple of 256, and 64 x 128 (2 x 2 waves of
// 32 x 64, 3 stages) for problems too small for the warp-specialized kernel
// (they have fewer 128 x 128 tiles than CUs: the output 4096x512 over a
// 32768-long contraction, 128 tiles, measured 209 -> 168 us with them).
#define FP8BS_TILE_MID 128, 128, 2, 2, 2
#define FP8BS_TILE_SMALL 64, 128, 2, 2, 3
// Split contraction for forward and activation-gradient GEMMs with few output
// tiles and a long contraction (dX [4096, 512] over 32768: 64 tiles of
// 256x128 leave three quarters of the CUs idle; the MLA latent projection
// 4096x640x7168, 80 tiles).  ksplit workgroups per tile each run one
// contiguous range of K slabs on the warp-specialized kernel and store an
// FP32 partial; splitk_reduce_kernel sums the partials in split order and
// rounds once to bf16.  fp8bs_gemm takes the partials from a stream-ordered
// allocation (hipMallocAsync / hipFreeAsync on the call's stream), so calls
// on different streams never share them; when that allocation fails it runs
// the unsplit kernels instead.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int64_t ksplit,
                                                            int64_t m, int64_t n, uint16_t* __restrict__ c,
                                                            int64_t ldc) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one 4-column group per thread
  const int64_t qpr = n / 4;
  if (q >= m * qpr) return;
  const int64_t row = q / qpr, col = (q - row * qpr) * 4;
  const int64_t plane = m * n;
  float4 acc = *reinterpret_cast<const float4*>(ws + row * n + col);
  for (int64_t k = 1; k < ksplit; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(ws + k * plane + row * n + col);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  uint2 o;
  o.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
  o.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
  *reinterpret_cast<uint2*>(c + row * ldc + col) = o;
}

// The weight gradient's summing kernel: f32 out, c = sum (or c + sum with
// accumulate), the partials added in split order first.
__global__ __launch_bounds__(256) void splitk_reduce_f32_kernel(const float* __restrict__ ws, int64_t ksplit,
                                                                int64_t m, int64_t n, float* __restrict__ c,
                                                                int64_t ldc, int accumulate) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one 4-column group per thread
  const int64_t qpr = n / 4;
  if (q >= m * qpr) return;
  const int64_t row = q / qpr, col = (q - row * qpr) * 4;
  const int64_t plane = m * n;
  float4 acc = *reinterpret_cast<const float4*>(ws + row * n + col);
  for (int64_t k = 1; k < ksplit; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(ws + k * plane + row * n + col);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  float* dst = c + row * ldc + col;
  if (accumulate) {
    const float4 old = *reinterpret_cast<const float4*>(dst);
    acc.x += old.x;
    acc.y += old.y;
    acc.z += old.z;
    acc.w += old.w;
  }
  *reinterpret_cast<float4*>(dst) = acc;
}

// Contraction split: 1 (none) unless 256x128 tiles would fill at most half
// the CUs; then the largest power of two that keeps tiles x split within the
// CUs, divides the K blocks and leaves each split 16 or more.
static int64_t gemm_ksplit(int64_t m, int64_t n, int64_t k, int cus) {
  if (use_ws(m, n, false)) return 1;
  const int64_t tiles = ((m + 255) / 256) * (n / 128);
  const int64_t nkb = k / BK;
  int64_t ks = 1;
  while (2 * ks * tiles <= cus && nkb % (2 * ks) == 0 && nkb / (2 * ks) >= 16) ks *= 2;
  return ks;
}

static int64_t split_bytes(int64_t m, int64_t n, int64_t ks) {
  return ks * m * n * (int64_t)sizeof(float);
}

// Enqueue the split GEMM (MODE: forward or dgrad) with its FP32 partials in
// `ws` (at least split_bytes(m, n, ks) bytes, not read before it is written).
template <int MODE>
static int launch_split(GemmArgs a, hipStream_t s, int64_t ks, float* ws) {
  a.tiles_n = a.n / 128;
  a.tiles_m = (a.m + 255) / 256;
  a.group_m = choose_group_m(a, 256, 128, 2);
  a.ksplit = ks;
  a.ws = ws;
  const int64_t tiles = a.tiles_m * a.tiles_n;
  const int64_t groups = a.m * a.n / 4;
  hipLaunchKernelGGL((gemm_ws_kernel<MODE, 8, 256, 128, false, true>), dim3((unsigned)tiles, (unsigned)ks),
                     dim3(64 * 12), 0, s, a);
  int st = launch_status();
  if (st == FP8BS_OK) {
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, a.ws, ks,
                       a.m, a.n, static_cast<uint16_t*>(a.c), a.ldc);
    st = launch_status();
  }
  return st;
}

static bool split_grid_ok(int64_t m, int64_t n, int64_t ks) {
  const int64_t tiles = ((m + 255) / 256) * (n / 128);
  return tiles <= kMaxGrid && ks <= 65535 && (m * n / 4 + 255) / 256 <= kMaxGrid;
}

// fp8bs_gemm without a contraction split: the warp-specialized kernel for
// problems with enough large tiles, else gemm_kernel's small tiles.  (A
// problem that use_ws turns away has fewer 128 x 128 tiles than CUs, since
// those are at most twice its 192 x 128 tiles, so gemm_kernel's 128 x 128
// tiles serve only the grouped GEMM.)
static int gemm_unsplit(GemmArgs a, int b_layout, hipStream_t stream) {
  const int64_t m = a.m, n = a.n;
  if (use_ws(m, n, false)) {
    if (b_layout == 0) return launch_gemm_ws<kFprop>(a, stream, cu_count());
    return launch_gemm_ws<kDgrad>(a, stream, cu_count());
  }
  if (b_layout == 0) return launch_gemm<kFprop, FP8BS_TILE_SMALL>(a, stream);
  return launch_gemm<kDgrad, FP8BS_TILE_SMALL>(a, stream);
}

// Argument checks of fp8bs_gemm; on success fills *a.
static int gemm_check(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb, int64_t m,
                      int64_t n, int64_t k, int b_layout, uint16_t* c, int64_t ldc, GemmArgs* a) {
  if (!qa || !sa || !qb || !sb || !c) return FP8BS_ERR_NULL;
  if (b_layout != 0 && b_layout != 1) return FP8BS_ERR_FLAG;
  if (m <= 0 || n <= 0 || k <= 0 || n % 128 || k % BK || ldc < n) return FP8BS_ERR_SHAPE;
  if (!fits_u32(256 * k) || (b_layout == 1 && !fits_u32(k * n))) return FP8BS_ERR_SHAPE;
  if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(c, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
      ldc % 8)
    return FP8BS_ERR_ALIGN;
  *a = GemmArgs{qa, sa, qb, sb, c, ldc, m, n, k, nullptr, 0, 0, 0, 0, 0, nullptr, 1, m * n * 2 > kStreamBytes};
  return FP8BS_OK;
}

extern "C" int fp8bs_gemm(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb,
                          int64_t m, int64_t n, int64_t k, int b_layout, uint16_t* c, int64_t ldc,
                          void* stream) {
  GemmArgs a;
  const int chk = gemm_check(qa, sa, qb, sb, m, n, k, b_layout, c, ldc, &a);
  if (chk != FP8BS_OK) return chk;
  hipStream_t s = (hipStream_t)stream;
  const int64_t ks = gemm_ksplit(m, n, k, cu_count());
  if (ks > 1) {
    if (!split_grid_ok(m, n, ks)) return FP8BS_ERR_SHAPE;
    void* ws = nullptr;
    if (hipMallocAsync(&ws, (size_t)split_bytes(m, n, ks), s) == hipSuccess) {
      int st = b_layout == 0 ? launch_split<kFprop>(a, s, ks, static_cast<float*>(ws))
                             : launch_split<kDgrad>(a, s, ks, static_cast<float*>(ws));
      if (hipFreeAsync(ws, s) != hipSuccess && st == FP8BS_OK) st = FP8BS_ERR_LAUNCH;
      return st;
    }
    // no memory for the partials: clear the runtime's error state and run
    // the unsplit kernels (same result within rounding, other bits)
    (void)hipGetLastError();
  }
  return gemm_unsplit(a, b_layout, s);
}

// ---- fp8bs_gemm without allocation -------------------------------------------
// The split GEMM's FP32 partials live in one fixed device array per GPU.  A
// split is chosen only when tiles x split <= CUs, so its partials take at most
// CUs x 256 x 128 floats: 32 MiB on the 256 CUs of an MI355X.  In host code
// the array's name stands for no device address: kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up once per device
// and kept in scratch_ptrs.  No kernel needs the array zeroed: every split
// workgroup writes its whole partial tile before the summing kernel reads it.
constexpr int64_t kScratchBytes = 32LL << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

static float* scratch_device_ptr() {
  static std::atomic<float*> scratch_ptrs[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  float* ptr = scratch_ptrs[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    ptr = static_cast<float*>(q);
    scratch_ptrs[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

extern "C" int fp8bs_gemm_noalloc(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb,
                                  int64_t m, int64_t n, int64_t k, int b_layout, uint16_t* c, int64_t ldc,
                                  void* stream) {
  GemmArgs a;
  const int chk = gemm_check(qa, sa, qb, sb, m, n, k, b_layout, c, ldc, &a);
  if (chk != FP8BS_OK) return chk;
  hipStream_t s = (hipStream_t)stream;
  const int64_t ks = gemm_ksplit(m, n, k, cu_count());
  if (ks > 1) {
    if (!split_grid_ok(m, n, ks)) return FP8BS_ERR_SHAPE;
    if (split_bytes(m, n, ks) > kScratchBytes) return FP8BS_ERR_SCRATCH;
    float* ws = scratch_device_ptr();
    if (ws == nullptr) return FP8BS_ERR_LAUNCH;
    return b_layout == 0 ? launch_split<kFprop>(a, s, ks, ws) : launch_split<kDgrad>(a, s, ks, ws);
  }
  return gemm_unsplit(a, b_layout, s);
}

extern "C" int fp8bs_grouped_gemm(const uint8_t* qa, const float* sa, const int32_t* seg_offsets,
                                  const int32_t* row_token, int64_t num_experts, int64_t total_rows,
                                  const uint8_t* qb, const float* sb, int64_t n, int64_t k, uint16_t* c,
                                  void* stream) {
  if (!qa || !sa || !seg_offsets || !qb || !sb || !c) return FP8BS_ERR_NULL;
  if (num_experts < 1 || num_experts > 65536 || total_rows <= 0 || total_rows % 128 || n <= 0 ||
      k <= 0 || n % 128 || k % BK)
    return FP8BS_ERR_SHAPE;
  if (!fits_u32(256 * k)) return FP8BS_ERR_SHAPE;
  if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(c, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
      !aligned(seg_offsets, 4) || !aligned(row_token, 4))
    return FP8BS_ERR_ALIGN;
  GemmArgs a{qa, sa, qb, sb, c, n, total_rows, n, k, seg_offsets, num_experts, 0, 0, 0, 0, nullptr, 1,
             total_rows * n * 2 > kStreamBytes, row_token};
  if (n % 256 == 0) return launch_grouped_ws(a, (hipStream_t)stream);
  return launch_gemm<kGrouped, FP8BS_TILE_MID>(a, (hipStream_t)stream);
}

extern "C" int fp8bs_grouped_gemm_bf16w(const uint8_t* qa, const float* sa, const int32_t* seg_offsets,
                                        const int32_t* row_token, int64_t num_experts, int64_t total_rows,
                                        const uint16_t* w, int64_t n, int64_t k, uint16_t* c, uint8_t* qw,
                                        float* sw, int keep_codes, void* stream) {
  if (!qa || !sa || !seg_offsets || !w || !c || (qw == nullptr) != (sw == nullptr)) return FP8BS_ERR_NULL;
  if (keep_codes != 0 && keep_codes != 1) return FP8BS_ERR_FLAG;
  if (keep_codes && !qw) return FP8BS_ERR_NULL;
  if (num_experts < 1 || num_experts > 65536 || total_rows <= 0 || total_rows % 128 || n <= 0 ||
      k <= 0 || n % 256 || k % BK)
    return FP8BS_ERR_SHAPE;
  if (!fits_u32(256 * k * 2)) return FP8BS_ERR_SHAPE;
  if (!aligned(qa, 16) || !aligned(w, 16) || !aligned(c, 16) || !aligned(qw, 16) || !aligned(sa, 4) ||
      !aligned(sw, 4) || !aligned(seg_offsets, 4) || !aligned(row_token, 4))
    return FP8BS_ERR_ALIGN;
  GemmArgs a{qa, sa, nullptr, nullptr, c, n, total_rows, n, k, seg_offsets, num_experts, 0, 0, 0, 0, nullptr, 1,
             total_rows * n * 2 > kStreamBytes, row_token, w, qw, sw, 0, keep_codes};
  if (!qw) return launch_grouped_ws<true>(a, (hipStream_t)stream);
  // With qw / sw: each expert's first m-tile codes the expert's weights from
  // bf16 (each weight read once) and stores them (all experts, or only those
  // with several m-tiles); then the expert's other m-tiles read the stored
  // codes, as fp8bs_grouped_gemm would.
  a.tile_sel = 1;
  const int st = launch_grouped_ws<true>(a, (hipStream_t)stream);
  if (st != FP8BS_OK) return st;
  GemmArgs b = a;
  b.qb = qw;
  b.sb = sw;
  b.w16 = nullptr;
  b.qw = nullptr;
  b.sw = nullptr;
  b.tile_sel = 2;
  return launch_grouped_ws<false>(b, (hipStream_t)stream);
}

// Contraction (token) split of a weight gradient whose output tiles fill at
// most half the CUs: 1 (none) otherwise; then the largest power of two that
// keeps tiles x split within the CUs, divides the token blocks and leaves each
// split 16 or more.  Tiles of 256 or 192 rows, whichever pads m less.
static int64_t wgrad_ksplit(int64_t m, int64_t n, int64_t t, int cus, bool* tall) {
  *tall = (m + 255) / 256 * 256 - m <= (m + 191) / 192 * 192 - m;
  const int64_t tiles = (*tall ? (m + 255) / 256 : (m + 191) / 192) * ((n + 127) / 128);
  const int64_t nkb = t / BK;
  int64_t ks = 1;
  while (2 * ks * tiles <= cus && nkb % (2 * ks) == 0 && nkb / (2 * ks) >= 16) ks *= 2;
  return ks;
}

// Enqueue the split weight gradient with its FP32 partials in `ws` (at least
// split_bytes(m, n, ks) bytes, not read before it is written).
template <int BM>
static int launch_wgrad_split(GemmArgs a, hipStream_t s, int64_t ks, float* ws) {
  a.tiles_n = (a.n + 127) / 128;
  a.tiles_m = (a.m + BM - 1) / BM;
  a.group_m = choose_group_m(a, BM, 128, 4);
  a.ksplit = ks;
  a.ws = ws;
  const int64_t tiles = a.tiles_m * a.tiles_n;
  const int64_t groups = a.m * a.n / 4;
  hipLaunchKernelGGL((gemm_ws_kernel<kWgrad, 4, BM, 128, false, true>), dim3((unsigned)tiles, (unsigned)ks),
                     dim3(64 * 8), 0, s, a);
  int st = launch_status();
  if (st == FP8BS_OK) {
    hipLaunchKernelGGL(splitk_reduce_f32_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, a.ws, ks,
                       a.m, a.n, static_cast<float*>(a.c), a.ldc, a.accumulate);
    st = launch_status();
  }
  return st;
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
  GemmArgs a{qa, sa, qb, sb, c, ldc, m, n, t, nullptr, 0, 0, 0, accumulate, 0};
  hipStream_t s = (hipStream_t)stream;
  bool tall = false;
  const int64_t ks = wgrad_ksplit(m, n, t, cu_count(), &tall);
  if (ks > 1) {
    if (m * n / 4 / 256 + 1 > kMaxGrid) return FP8BS_ERR_SHAPE;
    void* ws = nullptr;
    if (hipMallocAsync(&ws, (size_t)split_bytes(m, n, ks), s) == hipSuccess) {
      int st = tall ? launch_wgrad_split<256>(a, s, ks, static_cast<float*>(ws))
                    : launch_wgrad_split<192>(a, s, ks, static_cast<float*>(ws));
      if (hipFreeAsync(ws, s) != hipSuccess && st == FP8BS_OK) st = FP8BS_ERR_LAUNCH;
      return st;
    }
    // no memory for the partials: clear the runtime's error state and run
    // the unsplit kernels (same result within rounding, other bits)
    (void)hipGetLastError();
  }
  if (use_ws(m, n, true)) return launch_gemm_ws<kWgrad>(a, s, cu_count());
  return launch_gemm<kWgrad, FP8BS_TILE_SMALL>(a, s);
}
