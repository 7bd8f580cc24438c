"""Pins of the oracle's block-scaled GEMMs (forward, dgrad, wgrad, MoE grouped).

The pages ("DeepSeek-V3 技术报告深度解读", section 3) run all three GEMMs in FP8
with 1x128 / 128x128 scale groups and promote partial sums every 128 elements
of the contraction.  Pins that do not come from the oracle's own code:
  * exact brute force: integer arithmetic for each 128-element partial and exact
    rationals for the scaled sum, on tiny shapes with random codes (including
    +-448, subnormals and +-0) and random scales, for each GEMM variant;
  * the hand-worked two-block example in tests/golden/gemm_worked.txt;
  * a textbook reduction: inputs that quantize losslessly give exactly the
    float64 matrix product of the original bf16 values;
  * one-hot rows, linearity in the scales, the dequantized single-matmul form;
  * grouped == per-expert forward GEMM; zero padding rows give exact zeros.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (bf16_to_f32, e4m3_decode, gemm_dequant_reference, gemm_dgrad, gemm_fprop,
                    gemm_wgrad, grouped_gemm, quantize_act_1x128, quantize_w_128x128)
from workloads import f32_to_bf16_bits, gemm_inputs, grouped_inputs_host

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dec_int(codes):
    """E4M3 value in integer units of 2^-9 (independent of the oracle's table)."""
    codes = np.asarray(codes, np.int64)
    s, e, m = codes >> 7, (codes >> 3) & 15, codes & 7
    mag = np.where(e == 0, m, (8 + m) << np.maximum(e - 1, 0))
    return np.where(s == 1, -mag, mag)


def _random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c == 0x7F)] = 0x7E
    c[(c == 0xFF)] = 0xFE
    flat = c.reshape(-1)
    pick = rng.choice(flat.size, size=min(24, flat.size), replace=False)
    flat[pick[:6]] = 0x7E
    flat[pick[6:12]] = 0xFE
    flat[pick[12:16]] = 0x80
    flat[pick[16:20]] = rng.integers(1, 8, 4)        # subnormals
    return c


def _random_scales(rng, shape):
    s = np.exp(rng.uniform(np.log(1e-6), np.log(1e3), size=shape)).astype(np.float32)
    s.reshape(-1)[0] = 0.0
    return s


def _exact_blocked(ia_blocks, ib_blocks, w_fracs):
    """sum_kb w[kb] * P_kb * 2^-18 with integer P_kb, as Fractions."""
    total = Fraction(0)
    for p, w in zip(ia_blocks, w_fracs):
        total += w * Fraction(int(p), 1 << 18)
    return total


def _check_close(c64, exact, mag):
    for idx in np.ndindex(c64.shape):
        err = abs(Fraction(float(c64[idx])) - exact[idx])
        assert err <= Fraction(1, 10 ** 15) * Fraction(float(mag[idx])) + Fraction(0), (idx, float(err))


def test_fprop_exact_brute_force():
    rng = np.random.default_rng(21)
    m, n, k = 3, 256, 256
    qa, qb = _random_codes(rng, (m, k)), _random_codes(rng, (n, k))
    sa, sb = _random_scales(rng, (m, k // 128)), _random_scales(rng, (n // 128, k // 128))
    c64 = gemm_fprop(qa, sa, qb, sb)
    ia, ib = _dec_int(qa), _dec_int(qb)
    exact = np.empty((m, n), dtype=object)
    mag = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            ps = [int(ia[i, kb * 128:(kb + 1) * 128] @ ib[j, kb * 128:(kb + 1) * 128]) for kb in range(2)]
            pabs = [int(np.abs(ia[i, kb * 128:(kb + 1) * 128]) @ np.abs(ib[j, kb * 128:(kb + 1) * 128])) for kb in range(2)]
            ws = [Fraction(float(sa[i, kb])) * Fraction(float(sb[j // 128, kb])) for kb in range(2)]
            exact[i, j] = _exact_blocked(ps, None, ws)
            mag[i, j] = float(sum(w * Fraction(p, 1 << 18) for p, w in zip(pabs, ws)))
    _check_close(c64, exact, mag)


def test_dgrad_exact_brute_force():
    rng = np.random.default_rng(22)
    m, k, n = 3, 256, 256                                 # contraction k, output n
    qa, qw = _random_codes(rng, (m, k)), _random_codes(rng, (k, n))
    sa, sw = _random_scales(rng, (m, k // 128)), _random_scales(rng, (k // 128, n // 128))
    c64 = gemm_dgrad(qa, sa, qw, sw)
    ia, iw = _dec_int(qa), _dec_int(qw)
    exact = np.empty((m, n), dtype=object)
    mag = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            ps = [int(ia[i, kb * 128:(kb + 1) * 128] @ iw[kb * 128:(kb + 1) * 128, j]) for kb in range(2)]
            pabs = [int(np.abs(ia[i, kb * 128:(kb + 1) * 128]) @ np.abs(iw[kb * 128:(kb + 1) * 128, j])) for kb in range(2)]
            ws = [Fraction(float(sa[i, kb])) * Fraction(float(sw[kb, j // 128])) for kb in range(2)]
            exact[i, j] = _exact_blocked(ps, None, ws)
            mag[i, j] = float(sum(w * Fraction(p, 1 << 18) for p, w in zip(pabs, ws)))
    _check_close(c64, exact, mag)


def test_wgrad_exact_brute_force():
    rng = np.random.default_rng(23)
    m, n, t = 3, 5, 384
    qa, qb = _random_codes(rng, (m, t)), _random_codes(rng, (n, t))
    sa, sb = _random_scales(rng, (m, t // 128)), _random_scales(rng, (n, t // 128))
    c64 = gemm_wgrad(qa, sa, qb, sb)
    ia, ib = _dec_int(qa), _dec_int(qb)
    for i in range(m):
        for j in range(n):
            ps = [int(ia[i, kb * 128:(kb + 1) * 128] @ ib[j, kb * 128:(kb + 1) * 128]) for kb in range(3)]
            pabs = [int(np.abs(ia[i, kb * 128:(kb + 1) * 128]) @ np.abs(ib[j, kb * 128:(kb + 1) * 128])) for kb in range(3)]
            ws = [Fraction(float(sa[i, kb])) * Fraction(float(sb[j, kb])) for kb in range(3)]
            exact = _exact_blocked(ps, None, ws)
            mag = sum(w * Fraction(p, 1 << 18) for p, w in zip(pabs, ws))
            assert abs(Fraction(float(c64[i, j])) - exact) <= Fraction(1, 10 ** 15) * mag


def test_golden_worked_two_block_example():
    qa = np.zeros((1, 256), np.uint8)
    qa[0, 0], qa[0, 1], qa[0, 128] = 0x38, 0x40, 0x30
    sa = np.array([[0.5, 2.0]], np.float32)
    qb = np.zeros((128, 256), np.uint8)
    qb[0, 0], qb[0, 1], qb[1, 0], qb[1, 1], qb[0, 128] = 0x38, 0xB8, 0x3C, 0x38, 0x48
    sb = np.array([[0.25, 0.5]], np.float32)
    c = gemm_fprop(qa, sa, qb, sb)
    want = np.zeros(128)
    with open(os.path.join(GOLDEN, "gemm_worked.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                j, v = line.split()
                want[int(j)] = float(v)
    assert np.array_equal(c[0], want)


def test_lossless_inputs_give_textbook_matmul():
    """Quantize + GEMM of exactly representable inputs == float64 A @ W^T, bit for bit."""
    rng = np.random.default_rng(24)
    m, n, k = 8, 256, 256

    def lossless(shape, exps_shape, expand):
        codes = rng.integers(0, 0x7F, size=shape).astype(np.uint8) | (rng.integers(0, 2, shape) << 7).astype(np.uint8)
        exps = rng.integers(-2, 3, size=exps_shape)
        return codes, exps, expand(np.ldexp(1.0, exps))

    ca, ea, fa = lossless((m, k), (m, k // 128), lambda s: np.repeat(s, 128, axis=1))
    ca[:, ::128] = 0x7E
    cw, ew, fw = lossless((n, k), (n // 128, k // 128), lambda s: np.repeat(np.repeat(s, 128, 0), 128, 1))
    cw[::128, ::128] = 0xFE
    a = e4m3_decode(ca) * fa
    w = e4m3_decode(cw) * fw
    a_bits, w_bits = f32_to_bf16_bits(a.astype(np.float32)), f32_to_bf16_bits(w.astype(np.float32))
    qa, sa = quantize_act_1x128(a_bits)
    qw, sw = quantize_w_128x128(w_bits)
    assert np.array_equal(qa, ca) and np.array_equal(qw, cw)
    c = gemm_fprop(qa, sa, qw, sw)
    assert np.array_equal(c, a @ w.T)


def test_single_block_and_one_hot():
    rng = np.random.default_rng(25)
    qa, qb = _random_codes(rng, (4, 128)), _random_codes(rng, (128, 128))
    sa, sb = _random_scales(rng, (4, 1)), _random_scales(rng, (1, 1))
    c = gemm_fprop(qa, sa, qb, sb)
    ref = (sa.astype(np.float64) * np.float64(sb[0, 0])) * (e4m3_decode(qa) @ e4m3_decode(qb).T)
    assert np.allclose(c, ref, rtol=1e-15, atol=0)
    # one-hot row selects one column of B times the scales
    qa1 = np.zeros((1, 384), np.uint8)
    qa1[0, 200] = 0x38                                    # 1.0 at k = 200 (block 1)
    sa1 = np.array([[3.0, 0.75, 5.0]], np.float32)
    qb1, sb1 = _random_codes(rng, (256, 384)), _random_scales(rng, (2, 3))
    c1 = gemm_fprop(qa1, sa1, qb1, sb1)
    want = 0.75 * np.repeat(sb1[:, 1].astype(np.float64), 128) * e4m3_decode(qb1[:, 200])
    assert np.array_equal(c1[0], want)


def test_linearity_in_scales_and_dequant_form():
    rng = np.random.default_rng(26)
    qa, qb = _random_codes(rng, (16, 512)), _random_codes(rng, (256, 512))
    sa, sb = _random_scales(rng, (16, 4)), _random_scales(rng, (2, 4))
    c = gemm_fprop(qa, sa, qb, sb)
    assert np.array_equal(gemm_fprop(qa, sa * np.float32(2), qb, sb), 2 * c)
    assert np.array_equal(gemm_fprop(qa, sa, qb, sb * np.float32(0.5)), 0.5 * c)
    sa_full = np.repeat(sa.astype(np.float64), 128, axis=1)
    sb_full = np.repeat(np.repeat(sb.astype(np.float64), 128, 0), 128, 1).T
    d = gemm_dequant_reference(qa, sa_full, qb.T, sb_full)
    assert np.linalg.norm(d - c) <= 1e-13 * np.linalg.norm(c)


def test_dgrad_is_fprop_of_transposed_weight():
    rng = np.random.default_rng(27)
    qa, qw = _random_codes(rng, (5, 256)), _random_codes(rng, (256, 384))
    sa, sw = _random_scales(rng, (5, 2)), _random_scales(rng, (2, 3))
    assert np.array_equal(gemm_dgrad(qa, sa, qw, sw), gemm_fprop(qa, sa, qw.T.copy(), sw.T.copy()))


def test_wgrad_equals_fprop_when_scales_are_blockwise():
    rng = np.random.default_rng(28)
    qa, qb = _random_codes(rng, (4, 256)), _random_codes(rng, (128, 256))
    sa, sbb = _random_scales(rng, (4, 2)), _random_scales(rng, (1, 2))
    sb_rows = np.repeat(sbb, 128, axis=0)
    assert np.array_equal(gemm_wgrad(qa, sa, qb, sb_rows), gemm_fprop(qa, sa, qb, sbb))


def test_grouped_equals_per_expert_and_padding_is_zero():
    cfg = dict(kind="grouped", seed=9, tokens=96, topk=4, experts=6, N=256, K=256, zipf_s=1.1,
               a_std=1.0, b_std=0.02)
    g = grouped_inputs_host(cfg)
    off, counts = g["offsets"], g["counts"]
    qa, sa = quantize_act_1x128(g["x"])
    qws = [quantize_w_128x128(g["w"][e]) for e in range(cfg["experts"])]
    qb = np.stack([q for q, _ in qws])
    sb = np.stack([s for _, s in qws])
    c = grouped_gemm(qa, sa, off, qb, sb)
    for e in range(cfg["experts"]):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            assert np.array_equal(c[lo:hi], gemm_fprop(qa[lo:hi], sa[lo:hi], qb[e], sb[e]))
        pad = slice(lo + counts[e], hi)
        assert np.all(c[pad] == 0)
    rows = np.array([0, int(off[2]) + 1, int(off[-1]) - 1])
    assert np.array_equal(grouped_gemm(qa, sa, off, qb, sb, rows=rows), c[rows])
    # an empty expert segment is allowed
    off2 = np.concatenate([off[:1], off])
    qb2, sb2 = np.concatenate([qb[:1], qb]), np.concatenate([sb[:1], sb])
    assert np.array_equal(grouped_gemm(qa, sa, off2, qb2, sb2), c)
    with pytest.raises(ValueError):
        grouped_gemm(qa, sa, off + 1, qb, sb)


def test_end_to_end_fine_grained_close_to_float64_product():
    """c1: quantize + GEMM tracks the unquantized product; tiles beat one per-tensor scale."""
    d = gemm_inputs("c1")
    a, b = bf16_to_f32(d["a"]).astype(np.float64), bf16_to_f32(d["b"]).astype(np.float64)
    exact = a @ b.T
    qa, sa = quantize_act_1x128(d["a"])
    qb, sb = quantize_w_128x128(d["b"])
    c = gemm_fprop(qa, sa, qb, sb)
    err_fine = np.linalg.norm(c - exact) / np.linalg.norm(exact)
    # one scale for the whole tensor (the contrast the pages draw)
    amax_a = np.max(np.abs(a))
    s_a = np.float32(np.float32(amax_a) / np.float32(448))
    from oracle import e4m3_encode
    qa_t = e4m3_encode((bf16_to_f32(d["a"]) / s_a).astype(np.float32))
    c_tensor = (e4m3_decode(qa_t) * np.float64(s_a)) @ (e4m3_decode(qb) * np.repeat(np.repeat(sb.astype(np.float64), 128, 0), 128, 1)).T
    err_tensor = np.linalg.norm(c_tensor - exact) / np.linalg.norm(exact)
    assert err_fine < 0.05
    assert err_fine < err_tensor
