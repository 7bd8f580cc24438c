"""Fine-grained FP8 quantizers.  TEST INFRASTRUCTURE ONLY.

Granularity is the pages' ("DeepSeek-V3 技术报告深度解读", section 3;
deepseek.csdn.net page, section 二(四); qqstock.cn page, FP8 section):
activations get one scale per 1x128 tile (one row, 128 consecutive elements
of the contraction), weights one scale per 128x128 block, in place of a
single per-tensor scale.

Per group G (a tile or a block), with x the bf16 inputs read exactly as
binary32:
    amax = max over G of |x|
    s    = fl32(amax / 448)                 (IEEE binary32 division)
    q    = e4m3_rne_sat(fl32(x / s))        (binary32 division, then encode)
and x is approximated by s * dec(q).  A group whose amax is 0 gets s = 0 and
every code is the signed zero of its input; no division happens there.

The scale is the dequantization multiplier, stored as float32, not rounded
to a power of two.  Layouts are row-major:
    activation tiles   x [R, C] -> q [R, C],  s [R, C/128]
    transposed tiles   x [T, C] -> q [C, T],  s [C, T/128]  (tiles run along T)
    weight blocks      w [N, K] -> q [N, K],  s [N/128, K/128]

FP8 activation caching (deepseek.csdn.net page, section 二(四), and the
qqstock.cn page, FP8 section: activations are stored in FP8 for the backward
pass).  The cached form of x [T, C] is the forward's own 1x128 tiles
(q [T, C], s [T, C/128]); the weight gradient needs tiles along T, so the
backward re-tiles from the cache (the pages do not say how; plainest reading):
    x_hat[t, c] = fl32(s[t, c/128] * dec(q[t, c]))     (one binary32 multiply)
    then the transposed tile quantizer above, applied to x_hat as binary32
    values (amax, fl32(amax/448), fl32(x_hat/s'), E4M3 RNE with saturation).
The value is rounded twice (once to E4M3 in the forward tiles, once in the
tiles along T); this composition is the definition.
"""

import numpy as np

from .bf16 import bf16_to_f32
from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode

GROUP = 128


def _quantize_groups(xg):
    """Quantize groups laid out along the last axis of ``xg`` (float32).

    ``xg`` has shape [..., g]; each slice along the last axis is one group.
    Returns (codes with the same shape, float32 scales of shape [...]).
    """
    xg = np.asarray(xg, dtype=np.float32)
    amax = np.max(np.abs(xg), axis=-1)                       # exact in binary32
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)      # binary32 division, RN
    nonzero = s != 0
    q = np.empty(xg.shape, dtype=np.uint8)
    if np.any(nonzero):
        quot = (xg[nonzero] / s[nonzero][..., None]).astype(np.float32)
        q[nonzero] = e4m3_encode(quot)
    if np.any(~nonzero):
        # amax == 0: all inputs are +-0; keep each input's sign bit
        z = xg[~nonzero]
        q[~nonzero] = np.where(np.signbit(z), 0x80, 0x00).astype(np.uint8)
    return q, s.astype(np.float32)


def quantize_act_1x128(x_bits):
    """1x128 tile quantization along the columns of x [R, C] (C % 128 == 0)."""
    x = bf16_to_f32(x_bits)
    if x.ndim != 2 or x.shape[1] % GROUP:
        raise ValueError("quantize_act_1x128: need x [R, C] with C % 128 == 0")
    r, c = x.shape
    q, s = _quantize_groups(x.reshape(r, c // GROUP, GROUP))
    return q.reshape(r, c), s.reshape(r, c // GROUP)


def quantize_act_1x128_t(x_bits):
    """Transposed 1x128 tiles: x [T, C] -> codes of x^T [C, T], tiles along T.

    Defined as the row-wise tile quantizer applied to x^T; T % 128 == 0.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2 or x_bits.shape[0] % GROUP:
        raise ValueError("quantize_act_1x128_t: need x [T, C] with T % 128 == 0")
    return quantize_act_1x128(np.ascontiguousarray(x_bits.T))


def quantize_w_128x128(w_bits):
    """128x128 block quantization of w [N, K] (N % 128 == 0, K % 128 == 0)."""
    w = bf16_to_f32(w_bits)
    if w.ndim != 2 or w.shape[0] % GROUP or w.shape[1] % GROUP:
        raise ValueError("quantize_w_128x128: need w [N, K] with N, K multiples of 128")
    n, k = w.shape
    nb, kb = n // GROUP, k // GROUP
    # [nb, 128, kb, 128] -> [nb, kb, 128*128]: each block becomes one group
    blocks = w.reshape(nb, GROUP, kb, GROUP).transpose(0, 2, 1, 3).reshape(nb, kb, GROUP * GROUP)
    q, s = _quantize_groups(blocks)
    q = q.reshape(nb, kb, GROUP, GROUP).transpose(0, 2, 1, 3).reshape(n, k)
    return np.ascontiguousarray(q), s.reshape(nb, kb)


def dequantize_act_1x128(q, s):
    """Cached 1x128 tiles back to binary32: x_hat [R, C] = fl32(s[r, c/128] * dec(q[r, c]))."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32)
    if q.ndim != 2 or q.shape[1] % GROUP or s.shape != (q.shape[0], q.shape[1] // GROUP):
        raise ValueError("dequantize_act_1x128: need q [R, C] (C % 128 == 0) and s [R, C/128]")
    dec = e4m3_decode(q).astype(np.float32)              # exact: every E4M3 value is a binary32
    return (dec * np.repeat(s, GROUP, axis=1)).astype(np.float32)   # binary32 multiply, RN


def requantize_act_1x128_t(q, s):
    """Tiles along the rows of a cached activation: codes [C, T], scales [C, T/128] (T % 128 == 0)."""
    x_hat = dequantize_act_1x128(q, s)
    t, c = x_hat.shape
    if t % GROUP:
        raise ValueError("requantize_act_1x128_t: need T % 128 == 0")
    xt = np.ascontiguousarray(x_hat.T)
    qt, st = _quantize_groups(xt.reshape(c, t // GROUP, GROUP))
    return qt.reshape(c, t), st.reshape(c, t // GROUP)


def quantize_per_tensor(x_bits):
    """One scale for the whole tensor: the scaling that the 1x128 / 128x128 groups replace
    (qqstock.cn page, FP8 section).  The same rules with a single group: amax over the
    tensor, s = fl32(amax/448), codes of fl32(x/s).  Returns (codes, float32 scalar scale)."""
    x = bf16_to_f32(x_bits)
    q, s = _quantize_groups(x.reshape(1, -1))
    return q.reshape(x.shape), np.float32(s[0])
