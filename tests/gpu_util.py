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


# Element-level allowance for the matrix core's own summation inside one
# 128-long K block.  v_mfma_f32_16x16x128_f8f6f4 does not add its 128 FP8
# products exactly: a probe against exact sums measured errors up to 2^-10.1 of
# the block's largest |product| and 2^-12 of the block's sum of |products|
# (products confined to a narrow exponent range are summed exactly).  This is
# the limited in-block accumulation that the per-128-element FP32 promotion is
# there to contain.  The allowance below is 4x the measured worst case.
MFMA_BLOCK_REL = 2.0 ** -10


def assert_gemm_parity(got, c64, mag=None, out_bf16=True, label=""):
    """got: float64 values of the GPU result; c64: oracle float64 result.

    Bar: normwise relative error <= 2e-3.  Diagnostics that catch localized
    mistakes (a wrong scale or a dropped block gives errors far above these):
      * every element within  r * |C64| + MFMA_BLOCK_REL * mag  of the oracle,
        with r = one bf16 ulp (bf16 outputs) or 2^-20 (f32 outputs) and
        mag = sum over blocks of |sa*sb| * sum |a*b| (oracle on |codes|);
      * bf16 outputs: >= 90% of elements exactly equal to bf16(C64) (an
        output rounding other than nearest-even would give ~50%).
    Returns the normwise error (printed for the record).
    """
    got = np.asarray(got, np.float64)
    c64 = np.asarray(c64, np.float64)
    assert got.shape == c64.shape, (got.shape, c64.shape)
    nrm = np.linalg.norm(c64)
    err = np.linalg.norm(got - c64) / nrm if nrm > 0 else np.linalg.norm(got)
    exact = float("nan")
    if out_bf16:
        ref_bits = f64_to_bf16_rne(c64)
        ref = (ref_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        exact = float(np.mean(got == ref))
        rel = np.ldexp(1.0, np.frexp(np.abs(c64))[1] - 8)          # one bf16 ulp at |c64|
    else:
        rel = np.abs(c64) * 2.0 ** -20
    allow = rel * 1.0001
    if mag is not None:
        allow = allow + MFMA_BLOCK_REL * np.asarray(mag, np.float64)
    worst = float(np.max(np.abs(got - c64) / np.maximum(allow, 1e-300)))
    print(f"[parity] {label}: normwise {err:.3e}  exact-bf16 {exact:.4f}  worst/allowance {worst:.3f}")
    assert err <= NORMWISE_TOL, f"{label}: normwise error {err:.3e} > {NORMWISE_TOL}"
    if mag is not None:
        assert worst <= 1.0, f"{label}: an element exceeds its allowance ({worst:.3f}x)"
    if out_bf16:
        assert exact >= 0.90, f"{label}: only {exact:.4f} of elements equal bf16(oracle)"
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
