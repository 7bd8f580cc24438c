"""The HIP quantizers evaluate x / s with a per-tile reciprocal split in two
parts, r = fl32(1/s) and rl = fl32(fma(-s, r, 1) * r), and one FMA per element,
q = fma(x, r, x * rl), instead of a full division (tiles with a tiny amax run
the same two operations on values and divisor scaled by 2^64).  This CPU test
proves that both forms give the E4M3 code of the IEEE quotient for every pair
of bf16 inputs (all amax, every |x| <= amax), by exhaustive enumeration in C
(gcc, IEEE fmaf)."""

import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host", "recip_division_check.c")
COMMON_H = os.path.join(os.path.dirname(HERE), "fp8_fine_grained_act_amd", "csrc", "common.h")


def kernel_threshold():
    text = open(COMMON_H, encoding="utf-8").read()
    m = re.search(r"kTinyAmaxBits\s*=\s*(0x[0-9A-Fa-f]+)u", text)
    assert m, "threshold constant not found in the kernel header"
    return int(m.group(1), 16)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_reciprocal_correction_matches_ieee_division_exhaustively(tmp_path):
    exe = tmp_path / "recip_division_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), SRC, "-lm"], check=True)
    thr = kernel_threshold()
    out = subprocess.run([str(exe), hex(thr)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.count("mismatches=0") == 2, out.stdout


REQUANT_SRC = os.path.join(HERE, "host", "requant_division_check.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_retiling_quotient_matches_ieee_division_near_every_boundary(tmp_path):
    """The re-tiling kernel divides arbitrary binary32 values (s * dec(q)), which the
    exhaustive bf16 enumeration does not cover: check its quotient sequence against the
    IEEE quotient for numerators within 6 ulps of every E4M3 rounding boundary, for
    divisors spread over every binary32 binade (normal and subnormal)."""
    exe = tmp_path / "requant_division_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), REQUANT_SRC, "-lm"], check=True)
    out = subprocess.run([str(exe), "96"], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "mismatches=0" in out.stdout, out.stdout
