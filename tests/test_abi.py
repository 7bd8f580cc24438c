"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host with the documented status codes (no kernel is launched
on any of these paths, so they run without a GPU)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")

OK, ENULL, ESHAPE, EALIGN, EFLAG = 0, -1, -2, -3, -4
P = 0x100000          # a 16-byte aligned stand-in pointer, never dereferenced on these paths
P_ODD = P + 4


@pytest.fixture(scope="module")
def raw():
    from fp8_fine_grained_act_amd import lib

    return lib.raw


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"\b(fp8bs_\w+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("fp8bs_quantize_act_1x128", "fp8bs_quantize_w_128x128", "fp8bs_gemm", "fp8bs_grouped_gemm",
              "fp8bs_gemm_wgrad", "fp8bs_status_string", "fp8bs_moe_max_rows", "fp8bs_moe_route",
              "fp8bs_requantize_act_1x128_t",
              "fp8bs_moe_permute_quantize", "fp8bs_moe_combine"):
        assert n in names


def test_library_exports_every_declared_symbol(raw):
    for name in declared_functions():
        assert hasattr(raw, name), name
        assert isinstance(getattr(raw, name), ctypes._CFuncPtr)


def test_status_strings(raw):
    from fp8_fine_grained_act_amd import lib

    assert lib.status_string(OK) == "ok"
    for s in (ENULL, ESHAPE, EALIGN, EFLAG, -5, -6):
        assert lib.status_string(s) not in ("ok", "unknown status")
    assert lib.status_string(123) == "unknown status"


def test_quantize_act_validation(raw):
    f = raw.fp8bs_quantize_act_1x128
    assert f(None, 4, 128, 128, 0, P, 128, P, None) == ENULL
    assert f(P, 4, 128, 128, 2, P, 128, P, None) == EFLAG
    assert f(P, 4, 100, 128, 0, P, 128, P, None) == ESHAPE          # cols % 128
    assert f(P, 0, 128, 128, 0, P, 128, P, None) == ESHAPE
    assert f(P, 4, 128, 64, 0, P, 128, P, None) == ESHAPE           # ldx < cols
    assert f(P_ODD, 4, 128, 128, 0, P, 128, P, None) == EALIGN
    assert f(P, 4, 128, 130, 0, P, 128, P, None) == EALIGN          # ldx % 8
    assert f(P, 4, 128, 128, 0, P, 136, P, None) == EALIGN          # ldq % 16
    assert f(P, 100, 64, 64, 1, P, 112, P, None) == ESHAPE          # transposed: rows % 128
    assert f(P, 128, 60, 64, 1, P, 128, P, None) == ESHAPE          # transposed: cols % 8
    assert f(P, 128, 64, 64, 1, P, 64, P, None) == ESHAPE           # transposed: ldq < rows


def test_quantize_act_routed_validation(raw):
    f = raw.fp8bs_quantize_act_1x128_routed
    assert f(P, 4, 128, 128, None, P, 128, P, None) == ENULL         # row map required
    assert f(None, 4, 128, 128, P, P, 128, P, None) == ENULL
    assert f(P, 4, 100, 128, P, P, 128, P, None) == ESHAPE           # cols % 128
    assert f(P, 0, 128, 128, P, P, 128, P, None) == ESHAPE
    assert f(P, 4, 128, 64, P, P, 128, P, None) == ESHAPE            # ldx < cols
    assert f(P, 4, 128, 128, P, P, 64, P, None) == ESHAPE            # ldq < cols
    assert f(P_ODD, 4, 128, 128, P, P, 128, P, None) == EALIGN
    assert f(P, 4, 128, 128, P + 2, P, 128, P, None) == EALIGN       # row map 4-byte aligned
    assert f(P, 4, 128, 130, P, P, 128, P, None) == EALIGN           # ldx % 8


def test_quantize_act_dual_validation(raw):
    f = raw.fp8bs_quantize_act_1x128_dual
    assert f(P, 128, 128, 128, P, 128, P, None, 128, P, None) == ENULL
    assert f(P, 100, 128, 128, P, 128, P, P, 112, P, None) == ESHAPE   # rows % 128
    assert f(P, 128, 64, 64, P, 64, P, P, 128, P, None) == ESHAPE      # cols % 128
    assert f(P, 0, 128, 128, P, 128, P, P, 128, P, None) == ESHAPE
    assert f(P, 128, 128, 64, P, 128, P, P, 128, P, None) == ESHAPE    # ldx < cols
    assert f(P, 256, 128, 128, P, 128, P, P, 128, P, None) == ESHAPE   # ldqt < rows
    assert f(P, 128, 128, 132, P, 128, P, P, 128, P, None) == EALIGN   # ldx % 8
    assert f(P_ODD, 128, 128, 128, P, 128, P, P, 128, P, None) == EALIGN
    assert f(P, 128, 128, 128, P, 136, P, P, 128, P, None) == EALIGN   # ldq % 16
    assert f(P, 128, 128, 128, P, 128, P, P, 136, P, None) == EALIGN   # ldqt % 16


def test_quantize_w_validation(raw):
    f = raw.fp8bs_quantize_w_128x128
    assert f(P, 128, 128, 128, None, 128, P, None) == ENULL
    assert f(P, 100, 128, 128, P, 128, P, None) == ESHAPE
    assert f(P, 128, 200, 200, P, 208, P, None) == ESHAPE
    assert f(P, 128, 128, 128, P_ODD, 128, P, None) == EALIGN


def test_gemm_validation(raw):
    f = raw.fp8bs_gemm
    assert f(P, P, P, None, 4, 128, 128, 0, P, 128, None) == ENULL
    assert f(P, P, P, P, 4, 128, 128, 3, P, 128, None) == EFLAG
    assert f(P, P, P, P, 4, 100, 128, 0, P, 128, None) == ESHAPE    # n % 128
    assert f(P, P, P, P, 4, 128, 100, 0, P, 128, None) == ESHAPE    # k % 128
    assert f(P, P, P, P, 0, 128, 128, 0, P, 128, None) == ESHAPE
    assert f(P, P, P, P, 4, 128, 128, 0, P, 64, None) == ESHAPE     # ldc < n
    assert f(P, P, P_ODD, P, 4, 128, 128, 0, P, 128, None) == EALIGN
    assert f(P, P, P, P, 4, 128, 128, 0, P, 132, None) == EALIGN    # ldc % 8


def test_grouped_validation(raw):
    f = raw.fp8bs_grouped_gemm
    assert f(P, P, None, None, 4, 512, P, P, 128, 128, P, None) == ENULL
    assert f(P, P, P, None, 4, 512, P, P, 128, 128, None, None) == ENULL
    assert f(P, P, P, None, 0, 512, P, P, 128, 128, P, None) == ESHAPE
    assert f(P, P, P, None, 4, 500, P, P, 128, 128, P, None) == ESHAPE    # total_rows % 128
    assert f(P, P, P, None, 4, 512, P, P, 128, 100, P, None) == ESHAPE
    assert f(P, P, P + 2, None, 4, 512, P, P, 128, 128, P, None) == EALIGN
    assert f(P, P, P, P + 2, 4, 512, P, P, 128, 128, P, None) == EALIGN  # row_token


def test_grouped_bf16w_validation(raw):
    f = raw.fp8bs_grouped_gemm_bf16w
    assert f(P, P, P, None, 4, 512, None, 256, 128, P, None, None, 0, None) == ENULL      # w
    assert f(P, P, P, None, 4, 512, P, 256, 128, P, P, None, 0, None) == ENULL           # qw without sw
    assert f(P, P, P, None, 4, 512, P, 256, 128, P, None, None, 1, None) == ENULL        # keep without qw
    assert f(P, P, P, None, 4, 512, P, 256, 128, P, P, P, 2, None) == EFLAG              # keep_codes
    assert f(P, P, P, None, 4, 512, P, 128, 128, P, None, None, 0, None) == ESHAPE       # n % 256
    assert f(P, P, P, None, 4, 500, P, 256, 128, P, None, None, 0, None) == ESHAPE       # total_rows % 128
    assert f(P, P, P, None, 4, 512, P, 256, 100, P, None, None, 0, None) == ESHAPE       # k % 128
    assert f(P, P, P, None, 4, 512, P + 2, 256, 128, P, None, None, 0, None) == EALIGN   # w
    assert f(P, P, P, None, 4, 512, P, 256, 128, P, P + 8, P, 1, None) == EALIGN         # qw


def test_wgrad_validation(raw):
    f = raw.fp8bs_gemm_wgrad
    assert f(P, P, P, P, 8, 8, 128, None, 8, 0, None) == ENULL
    assert f(P, P, P, P, 8, 8, 128, P, 8, 2, None) == EFLAG
    assert f(P, P, P, P, 8, 8, 100, P, 8, 0, None) == ESHAPE         # t % 128
    assert f(P, P, P, P, 8, 6, 128, P, 8, 0, None) == ESHAPE         # n % 4
    assert f(P, P, P, P, 8, 8, 128, P, 4, 0, None) == ESHAPE         # ldc < n
    assert f(P, P, P, P, 8, 8, 128, P, 10, 0, None) == EALIGN        # ldc % 4


def test_binding_has_the_c_names():
    from fp8_fine_grained_act_amd import lib

    for name in declared_functions():
        if name != "fp8bs_status_string":
            assert callable(getattr(lib, name)), name


def test_moe_max_rows(raw):
    f = raw.fp8bs_moe_max_rows
    assert f(4096, 8, 256) == (32768 + 127 * 256) // 128 * 128
    assert f(4, 2, 3) == 384 and f(2, 1, 1000) == 256 and f(0, 8, 256) == 0
    assert f(-1, 8, 256) == ESHAPE and f(10, 0, 4) == ESHAPE and f(10, 65, 4) == ESHAPE
    assert f(10, 8, 0) == ESHAPE and f(10, 8, 65537) == ESHAPE
    assert f(1 << 28, 8, 256) == ESHAPE                             # rows past int32


def test_moe_route_validation(raw):
    f = raw.fp8bs_moe_route
    cap = raw.fp8bs_moe_max_rows(100, 8, 256)
    assert f(P, 100, 8, 256, P, P, None, cap, None) == ENULL
    assert f(P, 100, 8, 256, P, P, P, cap - 128, None) == ESHAPE     # capacity below the bound
    assert f(P, 100, 8, 513, P, P, P, 1 << 20, None) == ESHAPE       # more experts than one workgroup sorts
    assert f(P, 100, 0, 256, P, P, P, cap, None) == ESHAPE
    assert f(P, -1, 8, 256, P, P, P, cap, None) == ESHAPE
    assert f(P + 2, 100, 8, 256, P, P, P, cap, None) == EALIGN


def test_moe_permute_quantize_validation(raw):
    f = raw.fp8bs_moe_permute_quantize
    assert f(P, 100, 7168, 7168, P, 8, P, P, 256, None, 7168, P, 4096, None) == ENULL
    assert f(P, 100, 7100, 7168, P, 8, P, P, 256, P, 7168, P, 4096, None) == ESHAPE   # hidden % 128
    assert f(P, 100, 7168, 7040, P, 8, P, P, 256, P, 7168, P, 4096, None) == ESHAPE   # ldx < hidden
    assert f(P, 100, 7168, 7168, P, 8, P, P, 256, P, 7040, P, 4096, None) == ESHAPE   # ldq < hidden
    assert f(P, 100, 7168, 7168, P, 65, P, P, 256, P, 7168, P, 4096, None) == ESHAPE  # topk
    assert f(P, 100, 7168, 7168, P, 8, P, P, 256, P, 7168, P, -1, None) == ESHAPE     # capacity
    assert f(P, 100, 7168, 7172, P, 8, P, P, 256, P, 7168, P, 4096, None) == EALIGN   # ldx % 8
    assert f(P, 100, 7168, 7168, P, 8, P, P, 256, P, 7176, P, 4096, None) == EALIGN   # ldq % 16
    assert f(P_ODD, 100, 7168, 7168, P, 8, P, P, 256, P, 7168, P, 4096, None) == EALIGN


def test_moe_combine_validation(raw):
    f = raw.fp8bs_moe_combine
    assert f(P, 7168, 4096, P, None, 100, 8, 7168, P, 7168, None) == ENULL
    assert f(P, 7168, 4096, P, P, 100, 8, 7164, P, 7168, None) == ESHAPE      # n % 8
    assert f(P, 7160, 4096, P, P, 100, 8, 7168, P, 7168, None) == ESHAPE      # ldy < n
    assert f(P, 7168, 4096, P, P, 100, 0, 7168, P, 7168, None) == ESHAPE      # topk
    assert f(P, 7168, 4096, P, P, -1, 8, 7168, P, 7168, None) == ESHAPE
    assert f(P, 7172, 4096, P, P, 100, 8, 7168, P, 7168, None) == EALIGN      # ldy % 8
    assert f(P_ODD, 7168, 4096, P, P, 100, 8, 7168, P, 7168, None) == EALIGN
    assert f(P, 7168, 4096, P, P, 0, 8, 7168, P, 7168, None) == OK            # no tokens: nothing to do


def test_requantize_act_t_validation(raw):
    f = raw.fp8bs_requantize_act_1x128_t
    assert f(P, None, 256, 256, 256, P, 256, P, None) == ENULL
    assert f(P, P, 200, 256, 256, P, 256, P, None) == ESHAPE          # rows % 128
    assert f(P, P, 256, 200, 208, P, 256, P, None) == ESHAPE          # cols % 128
    assert f(P, P, 256, 256, 128, P, 256, P, None) == ESHAPE          # ldq < cols
    assert f(P, P, 256, 256, 256, P, 128, P, None) == ESHAPE          # ldqt < rows
    assert f(P, P, 256, 256, 264, P, 256, P, None) == EALIGN          # ldq % 16
    assert f(P_ODD, P, 256, 256, 256, P, 256, P, None) == EALIGN
    assert f(P, P, 0, 256, 256, P, 256, P, None) == ESHAPE


def test_moe_max_rows_matches_the_oracle_bound(raw):
    from oracle import moe_max_rows

    rng = np.random.default_rng(3)
    for _ in range(200):
        t, k, e = int(rng.integers(0, 20000)), int(rng.integers(1, 65)), int(rng.integers(1, 65537))
        assert raw.fp8bs_moe_max_rows(t, k, e) == moe_max_rows(t, k, e), (t, k, e)
