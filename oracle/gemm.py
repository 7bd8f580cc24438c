"""Block-scaled FP8 GEMMs with float64 accumulation.  TEST INFRASTRUCTURE ONLY.

The pages ("DeepSeek-V3 技术报告深度解读", section 3) run all three GEMMs of a
linear layer in FP8 -- forward, activation gradient (dgrad) and weight
gradient (wgrad) -- and move the partial sums into FP32 after every 128
elements of the contraction; the deepseek.csdn.net page, section 二(四), and the
qqstock.cn page, FP8 section, add that the matrix-multiply partials accumulate
in FP32.  Because the scale groups are exactly 128 long along the contraction,
each 128-element partial has one activation scale per output row and one
weight scale per output column, so the result is

    C[m, n] = sum over K-blocks kb of  sa(m, kb) * sb(n, kb) * P_kb[m, n]
    P_kb[m, n] = sum over k in block kb of dec(qa[m, k]) * dec(qb[k, n])

The oracle evaluates exactly this, block by block in ascending kb, in float64:

* P_kb is computed with a float64 matrix product of decoded codes.  It is
  exact in any summation order: every E4M3 value is an integer multiple of
  2^-9, every product a multiple of 2^-18 of magnitude <= 448^2 < 2^18, so
  every partial sum of <= 128 products is a multiple of 2^-18 below 2^25,
  i.e. an integer below 2^43 in units of 2^-18 -- well inside 53 bits.
* sa * sb is exact in float64 (two 24-bit significands).
* w * P and the running sum round in float64 (relative error ~1e-16).

The result is returned in float64; the bf16 view of a forward/dgrad output is
``f64_to_bf16_rne`` of it.  Scales and codes come from ``quantize``.

Which scale goes with which block (readings of the pages, which give only the
tile and block shapes):
  forward   A [M,K] tiles along K, sa [M, K/128]; B [N,K] blocks, sb [N/128, K/128]
  dgrad     dY [M,K] tiles along K (= along the forward output dim), sa [M, K/128];
            forward weight used as stored, [K, N] (contraction first), sb [K/128, N/128]
  wgrad     dY^T [M,T] and X^T [N,T], tiles along tokens T: sa [M, T/128], sb [N, T/128]
  grouped   rows of expert e are [off[e], off[e+1]); each segment is a forward
            GEMM with that expert's weight W_e [N,K], sb_e [N/128, K/128]
"""

import numpy as np

from .e4m3 import e4m3_decode

GROUP = 128


def _accumulate_blocks(dec_a, dec_b_kn, scale_rows, scale_cols):
    """C = sum_kb scale_rows[:, kb] x scale_cols[:, kb] * (dec_a_kb @ dec_b_kb).

    dec_a      float64 [M, K]      decoded left operand (contraction last)
    dec_b_kn   float64 [K, N]      decoded right operand (contraction first)
    scale_rows float64 [M, K/128]  per output row, per K-block
    scale_cols float64 [N, K/128]  per output column, per K-block
    """
    m, k = dec_a.shape
    n = dec_b_kn.shape[1]
    c = np.zeros((m, n), dtype=np.float64)
    for kb in range(k // GROUP):
        sl = slice(kb * GROUP, (kb + 1) * GROUP)
        p = dec_a[:, sl] @ dec_b_kn[sl, :]                       # exact (see module doc)
        w = scale_rows[:, kb][:, None] * scale_cols[:, kb][None, :]   # exact
        c += w * p
    return c


def _check_k(k):
    if k % GROUP or k <= 0:
        raise ValueError("contraction length must be a positive multiple of 128")


def gemm_fprop(qa, sa, qb, sb):
    """Forward GEMM C = A B^T.  qa [M,K], sa [M,K/128], qb [N,K], sb [N/128,K/128]."""
    qa, qb = np.asarray(qa, np.uint8), np.asarray(qb, np.uint8)
    m, k = qa.shape
    n = qb.shape[0]
    _check_k(k)
    if qb.shape[1] != k or n % GROUP:
        raise ValueError("gemm_fprop: qb must be [N, K] with N % 128 == 0")
    sa = np.asarray(sa, np.float32).astype(np.float64).reshape(m, k // GROUP)
    sb = np.asarray(sb, np.float32).astype(np.float64).reshape(n // GROUP, k // GROUP)
    cols = np.repeat(sb, GROUP, axis=0)                           # [N, K/128]
    return _accumulate_blocks(e4m3_decode(qa), e4m3_decode(qb).T, sa, cols)


def gemm_dgrad(qa, sa, qb_kn, sb_kn):
    """Activation-gradient GEMM C = A B with B stored [K, N] (the forward weight).

    qa [M,K] with sa [M,K/128]; qb_kn [K,N] with sb_kn [K/128, N/128].
    """
    qa, qb_kn = np.asarray(qa, np.uint8), np.asarray(qb_kn, np.uint8)
    m, k = qa.shape
    n = qb_kn.shape[1]
    _check_k(k)
    if qb_kn.shape[0] != k or n % GROUP:
        raise ValueError("gemm_dgrad: qb must be [K, N] with N % 128 == 0")
    sa = np.asarray(sa, np.float32).astype(np.float64).reshape(m, k // GROUP)
    sb = np.asarray(sb_kn, np.float32).astype(np.float64).reshape(k // GROUP, n // GROUP)
    cols = np.repeat(sb.T, GROUP, axis=0)                         # [N, K/128]
    return _accumulate_blocks(e4m3_decode(qa), e4m3_decode(qb_kn), sa, cols)


def gemm_wgrad(qa, sa, qb, sb):
    """Weight-gradient GEMM C = A B^T over tokens, per-row scales on both sides.

    qa [M,T] with sa [M,T/128]; qb [N,T] with sb [N,T/128]; result float64 [M,N].
    """
    qa, qb = np.asarray(qa, np.uint8), np.asarray(qb, np.uint8)
    m, t = qa.shape
    n = qb.shape[0]
    _check_k(t)
    if qb.shape[1] != t:
        raise ValueError("gemm_wgrad: operands must share the token length")
    sa = np.asarray(sa, np.float32).astype(np.float64).reshape(m, t // GROUP)
    sb = np.asarray(sb, np.float32).astype(np.float64).reshape(n, t // GROUP)
    return _accumulate_blocks(e4m3_decode(qa), e4m3_decode(qb).T, sa, sb)


def grouped_gemm(qa, sa, seg_offsets, qb, sb, rows=None):
    """MoE grouped forward GEMM over expert row segments.

    qa [R,K], sa [R,K/128]; seg_offsets [E+1] non-decreasing multiples of 128
    with seg_offsets[E] == R; qb [E,N,K], sb [E,N/128,K/128].  Row r belongs to
    the expert e with seg_offsets[e] <= r < seg_offsets[e+1] and gets
    gemm_fprop(row r, W_e).  ``rows`` (optional) restricts the evaluation to
    those row indices and returns [len(rows), N].
    """
    qa = np.asarray(qa, np.uint8)
    off = np.asarray(seg_offsets, np.int64)
    num_e = off.shape[0] - 1
    r_total, k = qa.shape
    n = qb.shape[1]
    if off[0] != 0 or off[-1] != r_total or np.any(np.diff(off) < 0) or np.any(off % GROUP):
        raise ValueError("grouped_gemm: bad segment offsets")
    rows = np.arange(r_total) if rows is None else np.asarray(rows, np.int64)
    expert = np.searchsorted(off, rows, side="right") - 1
    sa = np.asarray(sa, np.float32).reshape(r_total, k // GROUP)
    out = np.zeros((rows.shape[0], n), dtype=np.float64)
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        if e < 0 or e >= num_e:
            raise ValueError("grouped_gemm: row outside every segment")
        out[sel] = gemm_fprop(qa[rows[sel]], sa[rows[sel]], qb[e], sb[e])
    return out


def gemm_dequant_reference(qa, sa_full, qb_kn, sb_full):
    """One float64 matmul of fully dequantized operands (a check, not the scheme).

    sa_full [M,K] and sb_full [K,N] hold each element's own scale.  dec(q)*s is
    exact in float64 (4 + 24 significant bits), so this differs from the
    block-by-block result only by float64 rounding of the sums; the CPU tests
    use it to cross-check the block bookkeeping of the functions above.
    """
    a = e4m3_decode(qa) * np.asarray(sa_full, np.float64)
    b = e4m3_decode(qb_kn) * np.asarray(sb_full, np.float64)
    return a @ b
