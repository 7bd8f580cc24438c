"""Helpers for the GPU parity tests: host <-> device transfers and the GEMM parity bar.

The bar for floating-point GEMM outputs is normwise relative error <= 2e-3
against the oracle's float64 result (the tolerance stated for this path), plus
stricter element-level diagnostics that catch localized mistakes.  Codes and
scales of the quantizers are compared bit for bit.
"""

import numpy as np
import torch

from oracle import e4m3_decode, f64_to_bf16_rne

NORMWISE_TOL = 2e-3


def to_dev_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_dev(arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def bf16_bits_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values_host(t):
    return (bf16_bits_host(t).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def magnitude_codes(q):
    """Codes with the sign bit cleared (|value| for the magnitude bound)."""
    return np.asarray(q, np.uint8) & np.uint8(0x7F)


def assert_gemm_parity(got, c64, mag=None, out_bf16=True, label=""):
    """got: float64 values of the GPU result; c64: oracle float64 result.

    * normwise relative error <= 2e-3;
    * bf16 outputs: every element within one bf16 ulp of the oracle value, except
      where cancellation makes the oracle value tiny against the magnitude sum
      ``mag`` (|C64| < 2^-12 * mag), and >= 99% of elements exactly equal to the
      bf16 rounding of the oracle value;
    * f32 outputs: normwise <= 1e-5.
    """
    got = np.asarray(got, np.float64)
    c64 = np.asarray(c64, np.float64)
    assert got.shape == c64.shape, (got.shape, c64.shape)
    nrm = np.linalg.norm(c64)
    err = np.linalg.norm(got - c64) / nrm if nrm > 0 else np.linalg.norm(got)
    assert err <= NORMWISE_TOL, f"{label}: normwise error {err:.3e} > {NORMWISE_TOL}"
    if not out_bf16:
        assert err <= 1e-5, f"{label}: f32 output normwise error {err:.3e} > 1e-5"
        return err
    ref_bits = f64_to_bf16_rne(c64)
    ref = (ref_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = np.mean(got == ref)
    assert exact >= 0.99, f"{label}: only {exact:.4f} of elements equal bf16(oracle)"
    ulp = np.ldexp(1.0, np.frexp(np.abs(c64))[1] - 8)       # bf16 ulp at |c64|
    off = np.abs(got - c64) > ulp * 1.0001
    if mag is not None:
        off &= ~(np.abs(c64) < 2.0 ** -12 * np.asarray(mag, np.float64))
    assert not np.any(off), f"{label}: {int(off.sum())} elements off by more than one bf16 ulp"
    return err


def random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[c == 0x7F] = 0x7E
    c[c == 0xFF] = 0xFE
    return c


def random_scales(rng, shape, lo=1e-4, hi=1e2):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape)).astype(np.float32)


def decode(q):
    return e4m3_decode(q)
