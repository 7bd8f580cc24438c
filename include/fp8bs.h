/*
 * fp8bs -- block-scaled FP8 quantization and GEMMs for AMD MI355X (gfx950).
 *
 * C ABI of the library libfp8bs.so.  Every entry point takes plain device
 * pointers and sizes, enqueues its kernels on the caller's HIP stream and
 * returns at once.  The caller owns every buffer it passes.
 *
 * Memory and state:
 *   - Two calls allocate: fp8bs_gemm and fp8bs_gemm_wgrad, when they split
 *     the contraction over workgroups, take their FP32 partials from a
 *     stream-ordered allocation on the call's stream (hipMallocAsync, freed
 *     with hipFreeAsync after use).  If that allocation fails they clear the
 *     runtime's error and run the unsplit kernels instead.
 *     fp8bs_gemm_noalloc is fp8bs_gemm without allocation.
 *   - The library caches one value per device: its compute-unit count (an
 *     atomic per device ordinal, filled on first use).  Tile shapes and the
 *     contraction split are chosen from it, so the bits of a GEMM result can
 *     differ between devices with different CU counts (always within the
 *     same error bound).
 *   - fp8bs_gemm_noalloc keeps its split partials in one fixed device array
 *     per GPU (see its declaration).
 *   Apart from that shared array, calls are re-entrant and thread-safe.
 *
 * The method (pages cited by title and section):
 *   "DeepSeek-V3 技术报告深度解读" (sherconan.github.io), section 3 "FP8 混合精度训练":
 *     all three GEMMs of a linear layer (forward, activation gradient, weight
 *     gradient) take FP8 inputs; activations are scaled per 1x128 tile and
 *     weights per 128x128 block; partial sums are promoted to FP32 after each
 *     128-element stretch of the contraction.
 *   deepseek.csdn.net page, section 二(四) "FP8 低精度训练", and the qqstock.cn
 *   page, section "FP8 低精度訓練：精度與效率的平衡": the same tile/block
 *   granularity in place of per-tensor scaling, FP32 accumulation of the
 *   matrix-multiply partials, routed MoE experts among the FP8 GEMMs.
 *
 * Readings where the pages are silent (fixed here, tested against a CPU
 * reference):
 *   - FP8 format: OCP E4M3 "fn" (max 448, NaN only at S.1111.111, no Inf).
 *   - Scale of a group: s = amax / 448 in IEEE binary32 (a dequantization
 *     multiplier, not rounded to a power of two).  Code of x: E4M3
 *     round-to-nearest-even of the binary32 quotient x / s, saturating at
 *     +-448, sign kept also for zeros.  A group with amax == 0 gets s = 0 and
 *     signed-zero codes.  No flush-to-zero anywhere.
 *   - Every 128-element scale group lies along the contraction of the GEMM
 *     that consumes it, so each 128-long partial is multiplied by one
 *     activation scale and one weight scale and added into an FP32
 *     accumulator: C = sum_kb sa(m,kb) * sb(n,kb) * P_kb.
 *   - Layouts are row-major.  bf16 travels as raw uint16_t bits, E4M3 as raw
 *     uint8_t codes, scales as float.
 *
 * Inputs must be finite.  Non-finite inputs give unspecified codes and results.
 *
 * Status codes: 0 on success; negative values are argument errors detected on
 * the host before any kernel is enqueued (nothing has been written), or a
 * launch error reported by the HIP runtime right after enqueueing.  Faults of
 * enqueued kernels surface at the caller's next synchronization.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BS_OK 0
#define FP8BS_ERR_NULL (-1)   /* a required pointer is NULL                          */
#define FP8BS_ERR_SHAPE (-2)  /* a size is <= 0, not a required multiple, or too big  */
#define FP8BS_ERR_ALIGN (-3)  /* a pointer or leading dimension is misaligned         */
#define FP8BS_ERR_FLAG (-4)   /* an enum-like flag has an unknown value               */
#define FP8BS_ERR_LAUNCH (-5) /* the HIP runtime rejected a kernel launch             */
#define FP8BS_ERR_SCRATCH (-6) /* needs more than fp8bs_gemm_noalloc's fixed array     */

/*
 * Activation quantization in 1x128 tiles: one FP32 scale per row and 128
 * consecutive elements ("DeepSeek-V3 技术报告深度解读", section 3 "FP8 混合精度训练":
 * activations are quantized per 1x128 tile; deepseek.csdn.net page, section
 * 二(四) "FP8 低精度训练": tile-wise activations instead of per-tensor scaling).
 *
 * transpose == 0: tiles run along the columns.
 *   x       bf16 [rows, cols], row stride ldx elements
 *   q       E4M3 [rows, cols], row stride ldq bytes
 *   scales  f32  [rows, cols/128], row-major, contiguous
 *   cols % 128 == 0, rows >= 1 (any value).
 * transpose == 1: tiles run along the rows (128 consecutive rows of one
 *   column), the output is the transposed matrix.  This feeds the weight
 *   gradient, whose contraction runs over tokens (the rows of x).
 *   x       bf16 [rows, cols], row stride ldx elements
 *   q       E4M3 [cols, rows], row stride ldq bytes
 *   scales  f32  [cols, rows/128], row-major, contiguous
 *   rows % 128 == 0, cols >= 1 with cols % 8 == 0.
 *   The result equals transpose == 0 applied to x^T.
 * Alignment: x and q 16-byte aligned, ldx % 8 == 0, ldq % 16 == 0, scales
 * 4-byte aligned; ldx >= cols and ldq >= the output row length.
 */
int fp8bs_quantize_act_1x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             int transpose, uint8_t* q, int64_t ldq, float* scales,
                             void* stream);

/*
 * 1x128 tiles along the columns of the routed rows of an expert-major
 * padded activation only.  The routed experts take each token's row into
 * 128-row segments whose padding rows carry no token (deepseek.csdn.net
 * page, section 一(二) "DeepSeekMoE 架构": 256 routed experts, 8 per token);
 * the expert GEMM reads only the routed rows of its FP8 input when it is
 * given the same row map (fp8bs_grouped_gemm and fp8bs_grouped_gemm_bf16w,
 * argument row_token), so the padding rows need no codes.  Each routed row
 * is coded exactly as by fp8bs_quantize_act_1x128 with transpose == 0
 * ("DeepSeek-V3 技术报告深度解读", section 3: one scale per 1x128 tile).
 *   x          bf16 [rows, cols], row stride ldx elements (device)
 *   row_token  int32 [rows] (device): row r is coded when row_token[r] >= 0
 *              (the token of the row, as fp8bs_moe_route writes it) and left
 *              alone, not read and not written, when it is negative
 *   q          E4M3 [rows, cols], row stride ldq bytes
 *   scales     f32 [rows, cols/128], contiguous
 *   cols % 128 == 0.
 * Errors: FP8BS_ERR_NULL for a null pointer, FP8BS_ERR_SHAPE, FP8BS_ERR_ALIGN
 * (x and q 16 bytes, ldx % 8 == 0, ldq % 16 == 0, scales and row_token
 * 4 bytes), FP8BS_ERR_LAUNCH.  The outputs of skipped rows keep their
 * previous contents.
 */
int fp8bs_quantize_act_1x128_routed(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                    const int32_t* row_token, uint8_t* q, int64_t ldq, float* scales,
                                    void* stream);

/*
 * Both orientations of the 1x128 activation tiles from one read of x.
 * In a training step an activation (and its output gradient) is the FP8
 * input of two GEMMs with different contractions ("DeepSeek-V3 技术报告深度解读",
 * section 3: forward / activation gradient contract over the columns, the
 * weight gradient over the tokens), so it is quantized along both.  The
 * outputs are bit-identical to fp8bs_quantize_act_1x128 with transpose == 0
 * (q, scales) and with transpose == 1 (qt, scales_t); x is read once.
 *   x         bf16 [rows, cols], row stride ldx elements
 *   q         E4M3 [rows, cols], row stride ldq bytes;   scales   f32 [rows, cols/128]
 *   qt        E4M3 [cols, rows], row stride ldqt bytes;  scales_t f32 [cols, rows/128]
 *   rows % 128 == 0, cols % 128 == 0.
 * Alignment: x, q, qt 16-byte aligned, ldx % 8 == 0, ldq % 16 == 0,
 * ldqt % 16 == 0, scales and scales_t 4-byte aligned.  The four outputs must
 * not overlap each other or x.
 */
int fp8bs_quantize_act_1x128_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                  uint8_t* q, int64_t ldq, float* scales, uint8_t* qt,
                                  int64_t ldqt, float* scales_t, void* stream);

/*
 * Re-tiling of a cached FP8 activation along its rows.  Activations are kept
 * in FP8 for the backward pass (deepseek.csdn.net page, section 二(四);
 * qqstock.cn page, FP8 section); the weight gradient contracts over the
 * tokens, so it needs tiles along the rows, made here from the cache alone
 * (the bf16 activation is no longer needed):
 *   x_hat[t, c] = fl32(scales[t, c/128] * dec(q[t, c]))   (binary32 multiply)
 *   qt, scales_t = the transpose == 1 tiles of x_hat, with the same rules
 *   applied to the binary32 values (amax, s' = fl32(amax/448), E4M3
 *   nearest-even of the binary32 quotient |x_hat| / s', sign kept; s' = 0
 *   gives signed zeros).  The value is rounded twice: once in the forward
 *   tiles, once here (a reading: the pages do not say how the cache is
 *   re-tiled).
 *   q         E4M3 [rows, cols], row stride ldq bytes (1x128 tiles along cols)
 *   scales    f32  [rows, cols/128], contiguous
 *   qt        E4M3 [cols, rows], row stride ldqt bytes (tiles along rows)
 *   scales_t  f32  [cols, rows/128], contiguous
 *   rows % 128 == 0, cols % 128 == 0.
 * Alignment: q and qt 16 bytes, ldq % 16 == 0, ldqt % 16 == 0, scales and
 * scales_t 4 bytes.  Outputs must not overlap the inputs.
 */
int fp8bs_requantize_act_1x128_t(const uint8_t* q, const float* scales, int64_t rows, int64_t cols,
                                 int64_t ldq, uint8_t* qt, int64_t ldqt, float* scales_t, void* stream);

/*
 * Weight quantization in 128x128 blocks: one FP32 scale per block
 * ("DeepSeek-V3 技术报告深度解读", section 3 "FP8 混合精度训练": weights are
 * quantized per 128x128 block; deepseek.csdn.net page, section 二(四)).
 *   w       bf16 [n, k], row stride ldw elements
 *   q       E4M3 [n, k], row stride ldq bytes
 *   scales  f32  [n/128, k/128], row-major, contiguous
 *   n % 128 == 0, k % 128 == 0.  Stacked expert weights [E, N, K] are passed
 *   as n = E * N (blocks never straddle experts because N % 128 == 0).
 * Alignment: w and q 16-byte aligned, ldw % 8 == 0, ldq % 16 == 0.
 */
int fp8bs_quantize_w_128x128(const uint16_t* w, int64_t n, int64_t k, int64_t ldw,
                             uint8_t* q, int64_t ldq, float* scales, void* stream);

/*
 * Block-scaled GEMM with bf16 output: C[m, n] = sum_k A[m, k] * B(k, n), the
 * contraction in 128-long blocks, each block's FP32 partial multiplied by
 * sa[m, kb] * sb(kb, n-block) and added to an FP32 accumulator; the result is
 * rounded to bf16 (nearest, ties to even).  The forward and the
 * activation-gradient GEMMs run in FP8 and their partial sums move to FP32
 * after every 128 elements of the contraction ("DeepSeek-V3 技术报告深度解读",
 * section 3 "FP8 混合精度训练"; deepseek.csdn.net page, section 二(四): the
 * matrix-multiply partials accumulate in FP32 registers).
 *   qa  E4M3 [m, k] contiguous,  sa f32 [m, k/128] contiguous (1x128 tiles)
 *   b_layout == 0 (forward, y = x W^T):
 *       qb E4M3 [n, k] contiguous, sb f32 [n/128, k/128] (128x128 blocks)
 *   b_layout == 1 (activation gradient, dx = dy W, with the forward weight
 *       used as stored): qb E4M3 [k, n] contiguous, sb f32 [k/128, n/128]
 *   c   bf16 [m, n], row stride ldc elements
 *   m >= 1 (any), n % 128 == 0, k % 128 == 0.
 * Alignment: qa, qb, c 16-byte aligned; ldc % 8 == 0, ldc >= n.
 * Workspace: when the output's 192x128 tiles would cover fewer than half the
 * compute units (so its 256x128 tiles fill at most half of them) and the
 * contraction is long (at least 32 blocks), the contraction is split over
 * workgroups.  Their FP32 partials,
 * split x m x n x 4 bytes (split <= the compute-unit count / tiles, so at most
 * CUs x 128 KiB), take a stream-ordered allocation on `stream`
 * (hipMallocAsync, freed with hipFreeAsync after the summing kernel; graph
 * capture records both).  The partials are summed in split order and rounded
 * once: the result is deterministic for a given device and split, but not
 * bit-identical to an unsplit run.  If the allocation fails, the runtime's
 * error is cleared and the unsplit kernels run instead (same error bound).
 */
int fp8bs_gemm(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb,
               int64_t m, int64_t n, int64_t k, int b_layout, uint16_t* c, int64_t ldc,
               void* stream);

/*
 * fp8bs_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture that must record no allocation, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * fp8bs_gemm; it never allocates.  Where fp8bs_gemm would split the
 * contraction (either b_layout), the FP32 partials go to a fixed
 * device array of 32 MiB per GPU, part of the library's code object and held
 * until the process ends; the split is chosen only when
 * split x tiles <= compute units, so on a 256-CU MI355X it always fits.
 * Every call on one GPU shares that array: calls whose splits overlap in
 * time on one GPU (other streams, other host threads) race and give wrong
 * results; order them on one stream.  Nothing in the array needs clearing (each
 * call writes the partials it reads).
 * Returns FP8BS_ERR_SCRATCH, before anything is enqueued, if a split would
 * need more than 32 MiB (devices with more than 256 compute units), and
 * FP8BS_ERR_LAUNCH if the array's device address cannot be obtained.
 */
int fp8bs_gemm_noalloc(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb,
                       int64_t m, int64_t n, int64_t k, int b_layout, uint16_t* c, int64_t ldc,
                       void* stream);

/*
 * MoE grouped GEMM (forward) over expert row segments.  The rows of expert e
 * are [seg_offsets[e], seg_offsets[e+1]); each segment gets fp8bs_gemm
 * (b_layout 0) with that expert's weight.  Each token is routed to 8 of 256
 * routed experts (deepseek.csdn.net page, section 一(二) "DeepSeekMoE 架构"),
 * and the expert FFN GEMMs are among the GEMMs that run in FP8 with 1x128
 * activation tiles and 128x128 weight blocks ("DeepSeek-V3 技术报告深度解读",
 * section 3 "FP8 混合精度训练").
 *   qa          E4M3 [total_rows, k], sa f32 [total_rows, k/128]
 *   seg_offsets int32 [num_experts + 1], DEVICE memory
 *   row_token   int32 [total_rows], DEVICE memory, or NULL: the row map that
 *               fp8bs_moe_route writes (-1 marks a padding row)
 *   qb          E4M3 [num_experts, n, k], sb f32 [num_experts, n/128, k/128]
 *   c           bf16 [total_rows, n] contiguous
 *   total_rows % 128 == 0, n % 128 == 0, k % 128 == 0, 1 <= num_experts <= 65536.
 * Preconditions on seg_offsets (not checked: they live on the device):
 * seg_offsets[0] == 0, non-decreasing, every entry a multiple of 128,
 * seg_offsets[num_experts] <= total_rows.  Empty segments are allowed.
 * Rows from seg_offsets[num_experts] to total_rows belong to no expert: their
 * 128-row tiles end at once and those rows of c are not written (total_rows
 * may be a capacity such as fp8bs_moe_max_rows, so that no host
 * synchronization is needed to learn the padded total).
 * Padding rows (rows of a segment beyond the expert's routed rows):
 *   row_token NULL: every row of a segment is read; padding rows are expected
 *     to hold zeros in the bf16 source, so their codes and scales are zero
 *     and their outputs are exactly 0.
 *   row_token given: in each 128-row tile, the rows after its last row with
 *     row_token >= 0 are not read (their codes and scales count as zero,
 *     whatever memory holds) and their outputs are exactly 0.  The padding
 *     then costs no memory traffic; the other rows give the same bits as
 *     with NULL.
 * Alignment: qa, qb, c 16-byte aligned; sa, sb, seg_offsets, row_token 4-byte.
 */
int fp8bs_grouped_gemm(const uint8_t* qa, const float* sa, const int32_t* seg_offsets,
                       const int32_t* row_token, int64_t num_experts, int64_t total_rows,
                       const uint8_t* qb, const float* sb, int64_t n, int64_t k, uint16_t* c,
                       void* stream);

/*
 * MoE grouped GEMM from bf16 expert weights: fp8bs_quantize_w_128x128 of w
 * followed by fp8bs_grouped_gemm, in one kernel.  The expert weights are
 * quantized in 128x128 blocks for the FP8 GEMM ("DeepSeek-V3 技术报告深度解读",
 * section 3 "FP8 混合精度训练"); here each block is coded where the GEMM
 * reads it, so the FP8 weights are not read back from memory.
 *   w    bf16 [num_experts, n, k] contiguous
 *   qw   E4M3 [num_experts, n, k] and sw f32 [num_experts, n/128, k/128], or
 *        both NULL.  Codes and scales are stored there once, by an expert's
 *        first 128-row tile, bit for bit those of fp8bs_quantize_w_128x128(w):
 *          keep_codes == 1: for every expert that owns at least one row (the
 *            FP8 weights kept for later GEMMs, e.g. a backward's dgrad);
 *          keep_codes == 0: only for experts with more than one 128-row tile,
 *            whose other tiles read them back; qw / sw then serve as the
 *            call's workspace and hold nothing defined for the other experts.
 *        With qw == NULL nothing is stored and every tile codes its weights
 *        from bf16 (keep_codes must be 0).  Blocks of experts without rows
 *        are never written.
 *   qa, sa, seg_offsets, row_token, num_experts, total_rows, c: as for
 *        fp8bs_grouped_gemm, whose preconditions hold here too; n % 256 == 0.
 * c equals, bit for bit, fp8bs_grouped_gemm over the codes and scales that
 * fp8bs_quantize_w_128x128(w) gives, in every mode.
 * Alignment: qa, w, qw, c 16-byte aligned; sa, sw, seg_offsets, row_token
 * 4-byte.  Errors: FP8BS_ERR_NULL also when exactly one of qw, sw is NULL or
 * when keep_codes == 1 without them; FP8BS_ERR_FLAG when keep_codes is not 0
 * or 1.
 */
int fp8bs_grouped_gemm_bf16w(const uint8_t* qa, const float* sa, const int32_t* seg_offsets,
                             const int32_t* row_token, int64_t num_experts, int64_t total_rows,
                             const uint16_t* w, int64_t n, int64_t k, uint16_t* c, uint8_t* qw,
                             float* sw, int keep_codes, void* stream);

/*
 * Weight-gradient GEMM: C[m, n] (+)= sum_t A[m, t] * B[n, t] over tokens t,
 * with per-row scales on both operands (both come from
 * fp8bs_quantize_act_1x128 with transpose == 1), FP32 output.  The weight
 * gradient is the third GEMM of a layer that runs in FP8
 * ("DeepSeek-V3 技术报告深度解读", section 3 "FP8 混合精度训练"); its scale groups
 * lie along its contraction, the tokens (a reading: the pages give only the
 * 1x128 activation granularity).
 *   qa  E4M3 [m, t] contiguous, sa f32 [m, t/128]
 *   qb  E4M3 [n, t] contiguous, sb f32 [n, t/128]
 *   c   f32 [m, n], row stride ldc elements
 *   accumulate == 0 overwrites c, == 1 adds to it (gradient accumulation).
 *   t % 128 == 0, m >= 1, n >= 1 with n % 4 == 0.
 * Alignment: qa, qb, c 16-byte aligned; ldc % 4 == 0, ldc >= n.
 * Workspace: when the output's tiles (256 or 192 rows by 128 columns) fill at
 * most half the compute units and there are at least 32 token blocks, the
 * token contraction is split over workgroups.  Their FP32 partials, split x
 * m x n x 4 bytes (at most CUs x 128 KiB), take a stream-ordered allocation on
 * `stream` (hipMallocAsync, freed with hipFreeAsync after the summing kernel).
 * The partials are summed in split order, then added to c when accumulating:
 * deterministic for a given device and split, not bit-identical to an
 * unsplit run.  If the allocation fails, the runtime's error is cleared and
 * the unsplit kernels run instead (same error bound).
 */
int fp8bs_gemm_wgrad(const uint8_t* qa, const float* sa, const uint8_t* qb, const float* sb,
                     int64_t m, int64_t n, int64_t t, float* c, int64_t ldc, int accumulate,
                     void* stream);

/*
 * ---- MoE dispatch and combine around the grouped GEMM ----------------------
 * Each token is routed to topk of the routed experts (deepseek.csdn.net page,
 * section 一(二) "DeepSeekMoE 架构": 8 of 256); a layer's chunk dispatches the
 * tokens to their experts before the expert MLP and combines the expert
 * outputs after it (qqstock.cn page, section "DualPipe 流水線并行"); the
 * dispatched activations travel in FP8, the combined outputs in BF16
 * (deepseek.csdn.net page, section 二(四) "FP8 低精度训练").
 *
 * Layout (a reading; the pages do not fix it): expert-major rows.  The
 * (token, slot) pairs that chose expert e take consecutive rows in
 * (token, slot) order, starting at seg_offsets[e]; each expert's run is
 * padded with zero rows up to a multiple of 128, so each 128-row tile of
 * fp8bs_grouped_gemm belongs to one expert.  A pair whose expert id is
 * outside [0, num_experts) is dropped: slot row -1, no row, no contribution
 * to the combine.  slot_rows [tokens, topk] and row_token [rows_cap] are the
 * two directions of the map.  Routing -> dispatch -> grouped GEMM -> combine
 * runs with no host synchronization: every buffer is sized by
 * fp8bs_moe_max_rows.  A pointer may be NULL only when its buffer has no
 * elements (no tokens, or a zero row capacity).
 */

/*
 * Largest padded row count any routing of tokens x topk pairs over
 * num_experts experts can need: (P + 127 * min(num_experts, P)) rounded down
 * to a multiple of 128, P = tokens * topk.  Host only.  Returns
 * FP8BS_ERR_SHAPE (negative) unless tokens >= 0, 1 <= topk <= 64,
 * 1 <= num_experts <= 65536 and the result fits in int32.
 */
int64_t fp8bs_moe_max_rows(int64_t tokens, int64_t topk, int64_t num_experts);

/*
 * Routing layout on the device (one workgroup; a stable counting sort).
 *   topk_ids     int32 [tokens, topk]  expert of each (token, slot) pair
 *   seg_offsets  int32 [num_experts + 1] out: padded segment starts,
 *                seg_offsets[num_experts] = padded total
 *   slot_rows    int32 [tokens, topk]  out: row of each pair (-1: dropped id)
 *   row_token    int32 [rows_cap]      out: token of each row; -1 for padding
 *                rows and for every row from the padded total to rows_cap
 *   1 <= num_experts <= 512, 1 <= topk <= 64, tokens >= 0 (0: all segments
 *   empty), rows_cap >= fp8bs_moe_max_rows(tokens, topk, num_experts).
 *   All pointers 4-byte aligned.  No output may overlap topk_ids.
 */
int fp8bs_moe_route(const int32_t* topk_ids, int64_t tokens, int64_t topk, int64_t num_experts,
                    int32_t* seg_offsets, int32_t* slot_rows, int32_t* row_token, int64_t rows_cap,
                    void* stream);

/*
 * Dispatch payload: each token row of x is coded once in 1x128 tiles and its
 * codes and scales are stored to each of its slot rows, so row r of q equals
 * row row_token[r] of fp8bs_quantize_act_1x128(x) bit for bit.  Padding rows
 * (row_token == -1 within the last 128 rows of a segment) get +0 codes and
 * scale 0; rows from seg_offsets[num_experts] to rows_cap are not written.
 *   x            bf16 [tokens, hidden], row stride ldx elements
 *   slot_rows    int32 [tokens, topk], seg_offsets int32 [num_experts + 1],
 *   row_token    int32 [rows_cap]  (the outputs of fp8bs_moe_route)
 *   q            E4M3 [rows_cap, hidden], row stride ldq bytes
 *   scales       f32  [rows_cap, hidden/128], contiguous
 *   hidden % 128 == 0, 1 <= topk <= 64, 1 <= num_experts <= 65536.
 * A slot row outside [0, rows_cap) is treated as dropped; segment bounds are
 * clipped to [0, rows_cap].  Alignment: x and q 16 bytes, ldx % 8 == 0,
 * ldq % 16 == 0, the int32 and float pointers 4 bytes.
 */
int fp8bs_moe_permute_quantize(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t ldx,
                               const int32_t* slot_rows, int64_t topk, const int32_t* seg_offsets,
                               const int32_t* row_token, int64_t num_experts, uint8_t* q, int64_t ldq,
                               float* scales, int64_t rows_cap, void* stream);

/*
 * Combine: out[t, :] = sum over slots j of gates[t, j] * y[slot_rows[t, j], :],
 * accumulated in FP32 in slot order (acc = fma(g, y, acc) from +0), rounded
 * once to bf16 (nearest, ties to even).  Dropped slots (row -1, or a row
 * outside [0, rows_cap)) add nothing and their gates are not used.
 *   y          bf16 [rows_cap, n], row stride ldy elements (expert outputs)
 *   slot_rows  int32 [tokens, topk], gates f32 [tokens, topk]
 *   out        bf16 [tokens, n], row stride ldo elements
 *   n % 8 == 0, 1 <= topk <= 64, tokens >= 0 (0: nothing is written).
 * Alignment: y and out 16 bytes, ldy % 8 == 0, ldo % 8 == 0, slot_rows and
 * gates 4 bytes.  out must not overlap y.
 */
int fp8bs_moe_combine(const uint16_t* y, int64_t ldy, int64_t rows_cap, const int32_t* slot_rows,
                      const float* gates, int64_t tokens, int64_t topk, int64_t n, uint16_t* out,
                      int64_t ldo, void* stream);

/* Short English text for a status code (static storage, never NULL). */
const char* fp8bs_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
