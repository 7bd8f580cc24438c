"""Pins of the oracle's bf16 conversions.

Decode: all 65536 bit patterns against torch's own bfloat16 -> float32 cast.
Encode (the bf16 output rounding of the forward / dgrad GEMMs): against torch's
float32 -> bfloat16 cast (round to nearest even) on float32-exact inputs, and
against exact-rational nearest-value search on float64 inputs, midpoints
included.
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import bf16_to_f32, f32_to_bf16_rne, f64_to_bf16_rne


def test_decode_all_patterns_against_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_encode_float32_against_torch_rne():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(7.0),
        (rng.standard_normal(50000) * 1e-30).astype(np.float32),
        # exact ties: bf16 value + half a bf16 ulp
        (bf16_to_f32(rng.integers(0, 0x7F00, 20000).astype(np.uint16)).view(np.uint32)
         | np.uint32(0x8000)).view(np.float32),
    ]).astype(np.float32)
    ours = f32_to_bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _nearest_bf16_exact(v):
    x = Fraction(v)
    f32 = np.float32(v)
    # candidate neighbours: the bf16 values bracketing v
    b = int(f32_to_bf16_rne(np.array([f32]))[0])
    cands = []
    for d in (-2, -1, 0, 1, 2):
        c = (b + d) & 0xFFFF
        val = float(bf16_to_f32(np.array([c], np.uint16))[0])
        if np.isfinite(val) and (np.signbit(val) == np.signbit(v) or val == 0):
            cands.append((abs(Fraction(val) - x), c & 1, c, val))
    cands.sort(key=lambda t: (t[0], t[1]))
    return cands[0][2]


def test_encode_float64_exact_rational():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(3000) * 3.0, rng.standard_normal(1000) * 1e-3])
    # float64 midpoints between adjacent bf16 values, and just off them
    base = bf16_to_f32(rng.integers(0x3000, 0x5000, 500).astype(np.uint16)).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(base)[1] - 8)
    v = np.concatenate([v, base + ulp / 2, base + ulp / 2 + 1e-12 * base, base + ulp / 2 - 1e-12 * base])
    got = f64_to_bf16_rne(v)
    for x, g in zip(v, got):
        assert g == _nearest_bf16_exact(float(x)), (x, hex(g))


def test_encode_signed_zero():
    assert f64_to_bf16_rne(np.array([-0.0, 0.0])).tolist() == [0x8000, 0x0000]
