"""OCP E4M3 ("fn") 8-bit float: exact decode and round-to-nearest-even encode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say the GEMM inputs are FP8 but do not name the format
("DeepSeek-V3 技术报告深度解读", section 3).  The reading used throughout is
OCP E4M3 in its "fn" form: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
bits, no infinities, NaN only at S.1111.111, largest finite 448.

Code layout ``s eeee mmm``:
  * e == 0      : value = (-1)^s * m * 2^-9           (subnormals, m = 0 gives +-0)
  * 1 <= e <= 15: value = (-1)^s * (1 + m/8) * 2^(e-7)
  * e == 15, m == 7 (0x7F, 0xFF): NaN

Encoding of a binary32 value v (reading of "RNE with saturation"):
  * the sign of v is kept, also when the magnitude rounds to zero;
  * the magnitude is rounded once, from its exact binary32 value, to the
    nearest E4M3 magnitude; a tie goes to the code with an even mantissa;
  * magnitudes that would round above 448 (the 480 slot is NaN, so anything
    >= 464) give 448.
The encoder below does this with integer arithmetic on the binary32 bit
pattern, so there is exactly one rounding step.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode_table():
    """Return the 256 E4M3 values as float64 (NaN at 0x7F and 0xFF)."""
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            table[code] = np.nan
        elif exp == 0:
            table[code] = sign * man * 2.0 ** -9
        else:
            table[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return table


_TABLE = e4m3_decode_table()


def e4m3_decode(codes):
    """Decode an array of uint8 codes to float64 (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLE[codes]


def e4m3_encode(v):
    """Encode finite binary32 values to E4M3 codes (RNE, saturating, signed zero).

    ``v`` is converted to float32 first; the caller is expected to pass values
    that already are binary32 (the quantizer passes the binary32 quotient).
    """
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input (precondition: finite values)")
    bits = v.view(np.uint32).astype(np.int64)
    sign = (bits >> 31) & 1
    mag = bits & 0x7FFFFFFF
    bexp = mag >> 23                        # biased binary32 exponent
    frac = mag & 0x7FFFFF

    code = np.zeros(bits.shape, dtype=np.int64)
    normal = bexp > 0                       # binary32 subnormals are < 2^-126, far below 2^-10
    if np.any(normal):
        be = bexp[normal]
        sig = (1 << 23) | frac[normal]      # |v| = sig * 2^(be - 150), sig has 24 bits
        e = be - 127                        # |v| in [2^e, 2^(e+1))
        # quantum of the E4M3 grid around |v|: 2^(e-3) in a normal binade,
        # 2^-9 in the subnormal range (below 2^-6)
        q_exp = np.maximum(e, -6) - 3
        shift = q_exp - (be - 150)          # >= 20
        big = shift >= 62
        shift_c = np.minimum(shift, 62)
        k = sig >> shift_c
        rem = sig & ((np.int64(1) << shift_c) - 1)
        half = np.int64(1) << (shift_c - 1)
        round_up = (rem > half) | ((rem == half) & ((k & 1) == 1))
        k = k + round_up.astype(np.int64)
        k = np.where(big, 0, k)             # magnitude far below the smallest subnormal
        # |v| rounded = k * 2^q_exp.  In the subnormal range the code is k itself
        # (k == 8 is the smallest normal, code 0x08).  In binade e the code is
        # ((e + 7) << 3) + (k - 8); k == 16 carries into the next binade.
        c = np.where(q_exp == -9, k, ((e + 7) << 3) + k - 8)
        c = np.minimum(c, 0x7E)             # saturate: 0x7F is NaN, nothing above 448
        code[normal] = c
    code = code | (sign << 7)
    return code.astype(np.uint8)
