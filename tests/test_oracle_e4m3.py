"""Pins of the oracle's E4M3 decode/encode against facts that do not come from it.

Format: OCP E4M3 "fn" (the reading for the pages' unnamed "FP8",
"DeepSeek-V3 技术报告深度解读", section 3).  Pins: closed-form values of the
format definition, hand-worked encodings (tests/golden), exhaustive round trip,
every midpoint and its float32 neighbours, and an exact-rational brute-force
nearest-value search.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import E4M3_MAX, e4m3_decode, e4m3_decode_table, e4m3_encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(x):
    return np.array([x], dtype=np.float32)


def test_decode_closed_form_values():
    t = e4m3_decode_table()
    assert t[0x7E] == 448.0 == E4M3_MAX
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9
    assert t[0x38] == 1.0 and t[0x3C] == 1.5 and t[0x40] == 2.0
    assert t[0x77] == 240.0
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    nan_codes = [c for c in range(256) if np.isnan(t[c])]
    assert nan_codes == [0x7F, 0xFF]


def test_decode_sign_symmetry_and_order():
    t = e4m3_decode_table()
    for c in range(0x80):
        if c == 0x7F:
            continue
        assert t[c | 0x80] == -t[c]
    pos = t[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)      # strictly increasing over 0x00..0x7E
    finite = t[np.isfinite(t)]
    assert finite.size == 254
    assert np.unique(finite).size == 253  # +0 and -0 compare equal


def test_decode_every_code_from_bits():
    # Independent restatement per code with integer exponent arithmetic.
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 0xF, c & 7
        got = e4m3_decode(np.array([c], np.uint8))[0]
        if e == 15 and m == 7:
            assert np.isnan(got)
            continue
        mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        assert Fraction(abs(got)) == mag
        assert np.signbit(got) == bool(s)


def test_encode_golden_worked_examples():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_encode_worked.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((float.fromhex(parts[0]), int(parts[1], 16)))
    assert len(rows) >= 20
    vals = np.array([r[0] for r in rows], dtype=np.float32)
    for (v, _), v32 in zip(rows, vals):
        assert float(v32) == v, "golden value must be exact in float32"
    got = e4m3_encode(vals)
    want = np.array([r[1] for r in rows], dtype=np.uint8)
    bad = [(rows[i][0].hex(), hex(got[i]), hex(want[i])) for i in range(len(rows)) if got[i] != want[i]]
    assert not bad, bad


def test_encode_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)


def test_encode_midpoints_ties_to_even_and_neighbours():
    t = e4m3_decode_table()
    for c in range(0x00, 0x7E):
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2          # midpoints are exact in float32
        even = c if c % 2 == 0 else c + 1
        for sign in (1.0, -1.0):
            sbit = 0x80 if sign < 0 else 0
            v = np.float32(sign * mid)
            assert e4m3_encode(_f32(v))[0] == even | sbit
            up = np.nextafter(np.float32(mid), np.float32(np.inf))
            dn = np.nextafter(np.float32(mid), np.float32(0))
            assert e4m3_encode(_f32(sign * up))[0] == (c + 1) | sbit
            assert e4m3_encode(_f32(sign * dn))[0] == c | sbit


def test_encode_saturation():
    for v, code in [(448.0, 0x7E), (464.0, 0x7E), (500.0, 0x7E), (1e30, 0x7E), (3.4e38, 0x7E),
                    (-448.0, 0xFE), (-464.0, 0xFE), (-1e30, 0xFE),
                    (float(np.nextafter(np.float32(464), np.float32(0))), 0x7E)]:
        assert e4m3_encode(_f32(v))[0] == code, v


def test_encode_tiny_and_signed_zero():
    assert e4m3_encode(_f32(2.0 ** -10))[0] == 0x00
    assert e4m3_encode(_f32(-(2.0 ** -11)))[0] == 0x80
    assert e4m3_encode(_f32(3 * 2.0 ** -10))[0] == 0x02
    assert e4m3_encode(_f32(-0.0))[0] == 0x80
    assert e4m3_encode(_f32(0.0))[0] == 0x00
    sub = np.float32(1e-40)                          # binary32 subnormal
    assert e4m3_encode(np.array([sub, -sub], np.float32)).tolist() == [0x00, 0x80]


def test_encode_monotone():
    rng = np.random.default_rng(7)
    v = np.sort(np.concatenate([
        rng.uniform(0, 500, 20000), np.exp(rng.uniform(np.log(1e-6), np.log(600), 20000))
    ]).astype(np.float32))
    codes = e4m3_encode(v).astype(np.int64)
    assert np.all(np.diff(codes) >= 0)               # positive codes order like magnitudes


def _nearest_exact(v):
    """Brute force: nearest E4M3 magnitude by exact rational distance; ties -> even code."""
    t = e4m3_decode_table()
    x = Fraction(abs(float(v)))
    if x > 448:
        best = 0x7E
    else:
        best, best_d = None, None
        for c in range(0x7F):
            d = abs(x - Fraction(float(t[c])))
            if best is None or d < best_d or (d == best_d and c % 2 == 0):
                best, best_d = c, d
    return best | (0x80 if np.signbit(v) else 0)


def test_encode_brute_force_exact_rational():
    rng = np.random.default_rng(11)
    t = e4m3_decode_table()
    samples = [
        rng.uniform(-470, 470, 1500),
        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(470), 1500)) * rng.choice([-1, 1], 1500),
    ]
    mids = []
    for c in range(0x7E):
        m = np.float32((t[c] + t[c + 1]) / 2)
        mids += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    v = np.concatenate(samples + [np.array(mids)]).astype(np.float32)
    got = e4m3_encode(v)
    for x, g in zip(v, got):
        assert g == _nearest_exact(x), (float(x), hex(g))


def test_encode_rejects_non_finite():
    with pytest.raises(ValueError):
        e4m3_encode(np.array([np.inf], np.float32))
    with pytest.raises(ValueError):
        e4m3_encode(np.array([np.nan], np.float32))
