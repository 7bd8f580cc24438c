"""Pins of the oracle's 1x128 tile, 128x128 block and transposed-tile quantizers.

Granularity from "DeepSeek-V3 技术报告深度解读", section 3 (activations per 1x128
tile, weights per 128x128 block); scale rule and rounding are the stated readings
(amax/448 in binary32; codes = E4M3 RNE of the binary32 quotient).

Pins: hand-worked tile (tests/golden), a scalar-loop second statement of the
definition on tiny inputs, the amax->448 property, power-of-two scaling
invariance, permutation equivariance, reconstruction bounds, the all-zero tile,
and the lossless special case that reduces quantization to the identity.
"""

import os

import numpy as np

from oracle import (bf16_to_f32, e4m3_decode, e4m3_encode, quantize_act_1x128,
                    quantize_act_1x128_t, quantize_w_128x128)
from workloads import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_bf16(rng, shape, scale=1.0):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def test_golden_worked_tile():
    entries, scale = [], None
    with open(os.path.join(GOLDEN, "quant_tile_worked.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line.startswith("# scale"):
                scale = float.fromhex(line.split()[2])
            if not line or line.startswith("#"):
                continue
            i, v, c = line.split()[:3]
            entries.append((int(i), float.fromhex(v), int(c, 16)))
    x = np.zeros((1, 128), np.float32)
    for i, v, _ in entries:
        x[0, i] = v
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_to_f32(bits), x)          # every golden value is a bf16
    q, s = quantize_act_1x128(bits)
    assert s.shape == (1, 1) and s[0, 0] == np.float32(scale)
    want = np.zeros(128, np.uint8)
    for i, _, c in entries:
        want[i] = c
    assert q[0].tolist() == want.tolist()


def _scalar_quantize_group(vals):
    """Second statement of the definition, one element at a time."""
    amax = np.float32(0)
    for v in vals:
        amax = max(amax, abs(np.float32(v)))
    s = np.float32(amax / np.float32(448))
    out = []
    for v in vals:
        if s == 0:
            out.append(0x80 if np.signbit(v) else 0)
        else:
            out.append(int(e4m3_encode(np.array([np.float32(v) / s], np.float32))[0]))
    return out, s


def test_tile_quantizer_matches_scalar_loops():
    rng = np.random.default_rng(1)
    x = _rand_bf16(rng, (3, 256), 2.0)
    xf = bf16_to_f32(x)
    q, s = quantize_act_1x128(x)
    for r in range(3):
        for t in range(2):
            codes, sc = _scalar_quantize_group(xf[r, t * 128:(t + 1) * 128])
            assert s[r, t] == sc
            assert q[r, t * 128:(t + 1) * 128].tolist() == codes


def test_block_quantizer_matches_scalar_loops():
    rng = np.random.default_rng(2)
    w = _rand_bf16(rng, (256, 384), 0.02)
    w[5, 300] = f32_to_bf16_bits(np.array([3.0], np.float32))[0]   # one block with an outlier
    wf = bf16_to_f32(w)
    q, s = quantize_w_128x128(w)
    assert s.shape == (2, 3)
    for bn in range(2):
        for bk in range(3):
            blk = wf[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128]
            codes, sc = _scalar_quantize_group(blk.ravel())
            assert s[bn, bk] == sc
            assert q[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128].ravel().tolist() == codes


def test_transposed_tiles_are_tiles_of_the_transpose():
    rng = np.random.default_rng(3)
    x = _rand_bf16(rng, (256, 40))                       # [T, C]
    q, s = quantize_act_1x128_t(x)
    assert q.shape == (40, 256) and s.shape == (40, 2)
    xf = bf16_to_f32(x)
    for c in range(40):
        for tb in range(2):
            codes, sc = _scalar_quantize_group(xf[tb * 128:(tb + 1) * 128, c])
            assert s[c, tb] == sc and q[c, tb * 128:(tb + 1) * 128].tolist() == codes


def test_amax_element_encodes_to_448_and_codes_bounded():
    rng = np.random.default_rng(4)
    for scale in (1e-30, 1e-3, 1.0, 50.0, 1e30):
        x = _rand_bf16(rng, (64, 512), scale)
        q, s = quantize_act_1x128(x)
        xf = bf16_to_f32(x).reshape(64, 4, 128)
        arg = np.argmax(np.abs(xf), axis=-1)
        qt = q.reshape(64, 4, 128)
        top = np.take_along_axis(qt, arg[..., None], -1)[..., 0]
        assert np.all((top == 0x7E) | (top == 0xFE))
        assert not np.any((q == 0x7F) | (q == 0xFF))
        assert np.all(np.abs(e4m3_decode(q)) <= 448)


def test_power_of_two_scaling_invariance():
    rng = np.random.default_rng(5)
    x = _rand_bf16(rng, (16, 256), 1.0)
    q0, s0 = quantize_act_1x128(x)
    for j in (-20, -3, 1, 7, 30):
        xs = f32_to_bf16_bits(bf16_to_f32(x) * np.float32(2.0 ** j))   # exact: power of two
        q, s = quantize_act_1x128(xs)
        assert np.array_equal(q, q0)
        assert np.array_equal(s, (s0 * np.float32(2.0 ** j)).astype(np.float32))


def test_permutation_within_tile():
    rng = np.random.default_rng(6)
    x = _rand_bf16(rng, (4, 384))
    q, s = quantize_act_1x128(x)
    perm = rng.permutation(128)
    xp = x.copy()
    xp[:, 128:256] = x[:, 128:256][:, perm]
    qp, sp = quantize_act_1x128(xp)
    assert np.array_equal(sp, s)
    assert np.array_equal(qp[:, 128:256], q[:, 128:256][:, perm])
    assert np.array_equal(qp[:, :128], q[:, :128]) and np.array_equal(qp[:, 256:], q[:, 256:])


def test_reconstruction_error_bound():
    rng = np.random.default_rng(7)
    x = _rand_bf16(rng, (128, 1024), 1.0)
    xf = bf16_to_f32(x).astype(np.float64)
    q, s = quantize_act_1x128(x)
    rec = e4m3_decode(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(rec - xf)
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    # half an E4M3 ulp: 2^-4 relative in the normal range, s * 2^-10 absolute below it,
    # plus the binary32 rounding of the quotient (relative 2^-24 of |x|)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, srep * 2.0 ** -10) + np.abs(xf) * 2.0 ** -22
    assert np.all(err <= bound)


def test_all_zero_tile_signed_zeros():
    x = np.zeros((2, 256), np.uint16)
    x[0, 5] = 0x8000                                      # -0.0
    x[1, 128:] = f32_to_bf16_bits(np.ones(128, np.float32))
    q, s = quantize_act_1x128(x)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and s[1, 1] == np.float32(1.0) / np.float32(448)
    assert q[0, 5] == 0x80 and np.count_nonzero(q[0]) == 1
    assert np.all(q[1, :128] == 0)


def test_lossless_special_case():
    """x = 2^i * (E4M3 value) with amax = 448 * 2^i quantizes exactly: s = 2^i, s*dec(q) == x."""
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 0x7F, size=(32, 512)).astype(np.uint8) | (rng.integers(0, 2, (32, 512)) << 7).astype(np.uint8)
    codes[:, ::128] = 0x7E                                 # force amax = 448 per tile
    exps = rng.integers(-8, 9, size=(32, 4))
    x = e4m3_decode(codes) * np.repeat(np.ldexp(1.0, exps), 128, axis=1)
    xb = f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(bf16_to_f32(xb).astype(np.float64), x)   # representable in bf16
    q, s = quantize_act_1x128(xb)
    assert np.array_equal(s.astype(np.float64), np.ldexp(1.0, exps))
    assert np.array_equal(e4m3_decode(q) * np.repeat(s.astype(np.float64), 128, axis=1), x)
