"""Pins of the oracle's re-tiling of a cached FP8 activation (tiles along the tokens).

Activations are kept in FP8 for the backward pass (deepseek.csdn.net page,
section 二(四)); the weight gradient needs tiles along the tokens.  Pins that
do not come from the oracle's own code:
  * the hand-worked 128x128 case in tests/golden/requant_worked.txt (scales from
    an exact-rational nearest-binary32 search, signed zero, saturation);
  * the lossless special case reduces to the (pinned) transposed quantizer of
    the original values;
  * power-of-two scaling of the cached scales scales the new scales and keeps
    every code;
  * the E4M3 rounding bound between x_hat and its re-tiled reconstruction, and
    x_hat itself against an exact-rational product.
"""

import os
from fractions import Fraction

import numpy as np

from oracle import (bf16_to_f32, dequantize_act_1x128, e4m3_decode, quantize_act_1x128,
                    quantize_act_1x128_t, requantize_act_1x128_t)
from workloads import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    f = {}
    for line in open(os.path.join(GOLDEN, "requant_worked.txt"), encoding="utf-8"):
        line = line.strip()
        if line and not line.startswith("#"):
            k, _, v = line.partition(" ")
            f[k] = [item.split(",") for item in v.split()]
    return f


def test_golden_worked_case():
    f = _golden()
    q = np.zeros((128, 128), np.uint8)
    s = np.zeros((128, 1), np.float32)
    for t, c, code in f["codes"]:
        q[int(t), int(c)] = int(code, 16)
    for t, v in f["scales"]:
        s[int(t), 0] = float(v)
    qt, st = requantize_act_1x128_t(q, s)
    want = np.zeros((128, 128), np.uint8)
    for c, t, code in f["expect_codes"]:
        want[int(c), int(t)] = int(code, 16)
    assert np.array_equal(qt, want)
    want_s = np.zeros((128, 1), np.uint32)
    for c, bits in f["expect_scales"]:
        want_s[int(c), 0] = int(bits, 16)
    assert np.array_equal(st.view(np.uint32), want_s)


def test_lossless_case_reduces_to_transposed_quantizer():
    # tiles whose 1x128 quantization is exact (power-of-two scale, values on the E4M3 grid)
    rng = np.random.default_rng(3)
    t, c = 256, 384
    codes = rng.integers(0, 0x7F, size=(t, c)).astype(np.uint8) | (rng.integers(0, 2, size=(t, c)) << 7).astype(np.uint8)
    codes[codes == 0xFF] = 0xFE
    codes[:, ::128] = 0x7E                                  # each tile's amax element is 448
    exps = rng.integers(-20, 10, size=(t, c // 128))
    s = np.ldexp(1.0, exps).astype(np.float32)
    x = e4m3_decode(codes) * np.repeat(s, 128, axis=1).astype(np.float64)
    bits = f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(bf16_to_f32(bits).astype(np.float64), x)      # exact in bf16
    q, sq = quantize_act_1x128(bits)
    assert np.array_equal(sq, s) and np.array_equal(q, codes)           # the forward tiles are lossless
    qt, st = requantize_act_1x128_t(q, sq)
    qt_ref, st_ref = quantize_act_1x128_t(bits)
    assert np.array_equal(qt, qt_ref) and np.array_equal(st.view(np.uint32), st_ref.view(np.uint32))


def test_power_of_two_scaling_of_cached_scales():
    rng = np.random.default_rng(4)
    x = f32_to_bf16_bits(rng.standard_normal((256, 256)).astype(np.float32))
    q, s = quantize_act_1x128(x)
    qt, st = requantize_act_1x128_t(q, s)
    for j in (-7, 3):
        qt2, st2 = requantize_act_1x128_t(q, (s * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(qt2, qt) and np.array_equal(st2, (st * np.float32(2.0 ** j)).astype(np.float32))


def test_rounding_bounds_and_exact_product():
    rng = np.random.default_rng(5)
    x = f32_to_bf16_bits((rng.standard_normal((128, 256)) * np.exp(rng.uniform(-8, 8, (128, 1)))).astype(np.float32))
    q, s = quantize_act_1x128(x)
    x_hat = dequantize_act_1x128(q, s).astype(np.float64)
    # x_hat is the binary32 rounding of the exact product: within half a binary32 ulp
    dec = e4m3_decode(q)
    for (r, c) in [(0, 0), (5, 17), (77, 200), (127, 255)]:
        exact = Fraction(float(s[r, c // 128])) * Fraction(float(dec[r, c]))
        ulp = Fraction(2) ** (np.frexp(float(exact))[1] - 24) if exact != 0 else Fraction(0)
        assert abs(Fraction(float(x_hat[r, c])) - exact) <= ulp / 2
    qt, st = requantize_act_1x128_t(q, s)
    rec = e4m3_decode(qt) * np.repeat(st, 128, axis=1).astype(np.float64)     # [C, T]
    xt = x_hat.T
    # E4M3 round to nearest: relative 2^-4 in the normal range, absolute s' * 2^-10 below it
    allow = np.maximum(np.abs(xt) * 2.0 ** -4, np.repeat(st, 128, axis=1) * 2.0 ** -10) * 1.0001
    assert np.all(np.abs(rec - xt) <= allow)
    # the largest element of each new tile encodes to +-448
    mags = e4m3_decode(qt & 0x7F).reshape(256, 1, 128)
    assert np.all(mags.max(axis=2) == 448.0)
