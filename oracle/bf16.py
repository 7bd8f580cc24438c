"""bfloat16 conversions for the oracle.  TEST INFRASTRUCTURE ONLY.

bfloat16 values travel as raw uint16 bit patterns (numpy has no bf16 type).
Decoding is exact (a bf16 is the top half of a binary32).  Encoding rounds to
nearest, ties to even, once, from the exact input value; this is the output
rounding of the forward and activation-gradient GEMMs, whose result the
benchmark configurations ask for in bf16 after FP32 accumulation.
"""

import numpy as np


def bf16_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16_rne(v):
    """Round float64 values to the nearest bf16 (ties to even); return uint16 bits.

    The bf16 grid in the binade [2^(e-1), 2^e) has step 2^(e-8) (8 significant
    bits); below 2^-126 the step is fixed at 2^-133 (bf16 subnormals).  The
    value is divided by its step (exact: a power of two), rounded half-to-even
    with ``np.rint``, and scaled back; the result is a bf16 value held exactly
    in float64 and float32.  Finite values inside the bf16 range only.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("f64_to_bf16_rne: non-finite input")
    _, e = np.frexp(v)                      # |v| in [2^(e-1), 2^e)
    q_exp = np.maximum(e - 8, -133)
    k = np.rint(np.ldexp(v, -q_exp))        # exact scaling, then half-to-even
    r = np.ldexp(k, q_exp)
    r32 = r.astype(np.float32)              # exact: r is on the bf16 grid
    if not np.all(np.isfinite(r32)):
        raise ValueError("f64_to_bf16_rne: value outside the bf16 range")
    assert np.array_equal(r32.astype(np.float64), r)
    return (r32.view(np.uint32) >> 16).astype(np.uint16)


def f32_to_bf16_rne(v):
    """Round float32 values to bf16 (RNE); float32 -> float64 is exact."""
    return f64_to_bf16_rne(np.asarray(v, dtype=np.float32).astype(np.float64))
