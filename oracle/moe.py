"""MoE dispatch and combine around the grouped GEMM.  TEST INFRASTRUCTURE ONLY.

What the pages fix:
* deepseek.csdn.net page, section 一(二) "DeepSeekMoE 架构": every token is
  sent to 8 of the 256 routed experts (top-k routing).
* qqstock.cn page, section "DualPipe 流水線并行": a layer's chunk runs
  attention, then the all-to-all dispatch of tokens to their experts, the
  expert MLP, then the all-to-all combine of the expert outputs.
* deepseek.csdn.net page, section 二(四) "FP8 低精度训练": activations are
  stored and communicated in FP8 or BF16 (low-precision dispatch payloads).

What the pages leave open, and the reading taken here (plainest one that the
rest of the method supports):
* Layout of the dispatched rows: expert-major.  The (token, slot) pairs that
  chose expert e occupy consecutive rows, ordered by token then slot (a stable
  counting sort of the row-major pair index by expert id); each expert's run
  is padded with zero rows up to a multiple of 128, so every 128-row tile of
  the grouped GEMM belongs to one expert.  seg_offsets[e] is the first row of
  expert e, seg_offsets[E] the padded total.
* Pairs whose expert id lies outside [0, E) are dropped: they get slot row -1,
  take no row, and add nothing in the combine.
* Dispatch payload: the routed rows are quantized in 1x128 tiles, exactly as
  the activation quantizer does for any row (a tile depends only on its own
  row), so dispatch = gather the token rows into the expert-major layout, then
  quantize.  Padding rows get +0 codes and scale 0.
* Combine: out[t] = sum over the token's slots j of g[t, j] * Y[row(t, j)],
  with gate weights g in float32 and expert outputs Y in bf16, the sum taken
  exactly (float64 here) and rounded once to bf16 (nearest, ties to even).
"""

import numpy as np

from .bf16 import bf16_to_f32, f64_to_bf16_rne
from .quantize import GROUP, quantize_act_1x128


def moe_max_rows(tokens, topk, num_experts):
    """Largest padded row count any routing of tokens x topk pairs can need.

    Each non-empty expert adds at most 127 padding rows and at most
    min(E, tokens*topk) experts are non-empty; the total is a multiple of 128.
    """
    pairs = int(tokens) * int(topk)
    busy = min(int(num_experts), pairs)
    return (pairs + 127 * busy) // GROUP * GROUP


def moe_route(topk_ids, num_experts, rows_cap=None):
    """Expert-major padded layout of the routed (token, slot) pairs.

    topk_ids  int [T, k]: the expert chosen by each token in each slot.
    Returns dict with
      counts      int64 [E]    routed pairs per expert
      seg_offsets int64 [E+1]  padded segment starts (multiples of 128)
      slot_rows   int64 [T, k] the row of each pair (-1: dropped id)
      row_token   int64 [rows_cap] the token of each row (-1: padding or unused)
    rows_cap defaults to moe_max_rows(T, k, E).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    if ids.ndim != 2:
        raise ValueError("moe_route: topk_ids must be [T, k]")
    t, k = ids.shape
    e_n = int(num_experts)
    cap = moe_max_rows(t, k, e_n) if rows_cap is None else int(rows_cap)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < e_n)
    counts = np.bincount(flat[valid], minlength=e_n).astype(np.int64)
    padded = (counts + GROUP - 1) // GROUP * GROUP
    seg = np.zeros(e_n + 1, dtype=np.int64)
    seg[1:] = np.cumsum(padded)
    if seg[-1] > cap:
        raise ValueError("moe_route: rows_cap too small for this routing")
    slot_rows = np.full(t * k, -1, dtype=np.int64)
    row_token = np.full(cap, -1, dtype=np.int64)
    nxt = seg[:-1].copy()
    for p in range(t * k):          # pairs in row-major (token, slot) order
        if valid[p]:
            e = flat[p]
            slot_rows[p] = nxt[e]
            row_token[nxt[e]] = p // k
            nxt[e] += 1
    return dict(counts=counts, seg_offsets=seg, slot_rows=slot_rows.reshape(t, k), row_token=row_token)


def moe_permute_quantize(x_bits, row_token, total_rows):
    """Dispatch payload: the routed rows in expert-major order, 1x128-quantized.

    x_bits     bf16 bits [T, H] (H % 128 == 0), tokens in token order.
    row_token  int [>= total_rows]: token of each row, -1 for a padding row.
    Returns (codes uint8 [total_rows, H], scales float32 [total_rows, H/128]);
    rows past total_rows (= seg_offsets[E]) are not part of the result.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2 or x_bits.shape[1] % GROUP:
        raise ValueError("moe_permute_quantize: need x [T, H] with H % 128 == 0")
    rows = np.asarray(row_token, dtype=np.int64)[:int(total_rows)]
    gathered = np.zeros((rows.shape[0], x_bits.shape[1]), dtype=np.uint16)   # +0.0 rows
    real = rows >= 0
    gathered[real] = x_bits[rows[real]]
    return quantize_act_1x128(gathered)


def moe_combine_exact(y_bits, slot_rows, gates):
    """Un-rounded combine: float64 [T, N], sum_j g[t, j] * Y[slot_rows[t, j]].

    Each product of a bf16 value and a float32 gate is exact in float64
    (8 + 24 significant bits); dropped pairs (slot row -1) add nothing.
    """
    y = bf16_to_f32(np.asarray(y_bits, dtype=np.uint16)).astype(np.float64)
    rows = np.asarray(slot_rows, dtype=np.int64)
    g = np.asarray(gates, dtype=np.float32).astype(np.float64)
    if rows.shape != g.shape or rows.ndim != 2:
        raise ValueError("moe_combine: slot_rows and gates must both be [T, k]")
    t, k = rows.shape
    out = np.zeros((t, y.shape[1]), dtype=np.float64)
    for j in range(k):
        live = rows[:, j] >= 0
        out[live] += g[live, j][:, None] * y[rows[live, j]]
    return out


def moe_combine(y_bits, slot_rows, gates):
    """Combine of the expert outputs back into token order, as bf16 bits [T, N]."""
    return f64_to_bf16_rne(moe_combine_exact(y_bits, slot_rows, gates))
