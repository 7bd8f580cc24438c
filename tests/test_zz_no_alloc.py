"""fp8bs_gemm_noalloc against fp8bs_gemm, through the C ABI (GPU).

The no-allocation call keeps a split GEMM's FP32 partials in the library's
fixed device array instead of a stream-ordered allocation; everything else is
the same launch.  Two calls in a row, the second with a smaller input, on
dgrad and on forward shapes that split the contraction (the only path that
touches the array; each first call fills all 32 MiB of it), then shapes that
do not split.
Each result must equal fp8bs_gemm's bit for bit, and meet the GEMM bar
(normwise <= 2e-3 against the float64 oracle, with the element-level
diagnostics) on sampled output rows.
"""

import numpy as np
import pytest
import torch

from oracle import gemm_dgrad, gemm_fprop
from tests.gpu_util import assert_gemm_parity, bf16_values_host, magnitude_codes, random_codes, random_scales, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def _rows(m, rng):
    return np.unique(np.concatenate([[0, m - 1], rng.choice(m, size=min(m, 12), replace=False)]))


def _dgrad_case(lib, rng, m, n, k, label):
    """dgrad C [m, n] = A [m, k] B [k, n]; returns nothing, asserts the bar."""
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (k, n))
    sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (k // 128, n // 128))
    dqa, dsa, dqb, dsb = to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)
    print(f"[noalloc] {label}: dgrad {m}x{n} over {k}", flush=True)
    c_ref = lib.fp8bs_gemm(dqa, dsa, dqb, dsb, b_layout=1)
    c_na = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    lib.fp8bs_gemm_noalloc(dqa, dsa, dqb, dsb, b_layout=1, c=c_na)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(c_na), _bits(c_ref)), f"{label}: differs from fp8bs_gemm"
    rows = _rows(m, rng)
    got = bf16_values_host(c_na)[rows]
    c64 = gemm_dgrad(qa[rows], sa[rows], qb, sb)
    mag = gemm_dgrad(magnitude_codes(qa[rows]), sa[rows], magnitude_codes(qb), sb)
    assert_gemm_parity(got, c64, mag, label=f"noalloc {label}")


def test_noalloc_split_dgrad_twice_then_smaller(gpu_lib):
    rng = np.random.default_rng(7070)
    # 4096 x 512 over 32768 (the kv-up layer's dgrad): 64 tiles of 256x128,
    # split 4 on 256 CUs, 32 MiB of partials -- the whole fixed array
    _dgrad_case(gpu_lib, rng, 4096, 512, 32768, "first call, split, 32 MiB of partials")
    # smaller, ragged rows: 8 tiles, split 4, 4 MB of partials over stale data
    _dgrad_case(gpu_lib, rng, 1000, 256, 8192, "second call, smaller split")


def _fprop_case(lib, rng, m, n, k, label):
    """forward C [m, n] = A [m, k] B [n, k]^T; returns nothing, asserts the bar."""
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (n // 128, k // 128))
    dqa, dsa, dqb, dsb = to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)
    print(f"[noalloc] {label}: forward {m}x{n} over {k}", flush=True)
    c_ref = lib.fp8bs_gemm(dqa, dsa, dqb, dsb)
    c_na = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    lib.fp8bs_gemm_noalloc(dqa, dsa, dqb, dsb, c=c_na)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(c_na), _bits(c_ref)), f"{label}: differs from fp8bs_gemm"
    rows = _rows(m, rng)
    got = bf16_values_host(c_na)[rows]
    c64 = gemm_fprop(qa[rows], sa[rows], qb, sb)
    mag = gemm_fprop(magnitude_codes(qa[rows]), sa[rows], magnitude_codes(qb), sb)
    assert_gemm_parity(got, c64, mag, label=f"noalloc {label}")


def test_noalloc_split_forward_twice_then_smaller(gpu_lib):
    rng = np.random.default_rng(7072)
    # 4096 x 512 over 16384: 64 tiles of 256x128, split 4, 32 MiB of partials
    _fprop_case(gpu_lib, rng, 4096, 512, 16384, "first call, split, 32 MiB of partials")
    # smaller, ragged rows: 8 tiles, split 4, 4 MB of partials over stale data
    _fprop_case(gpu_lib, rng, 1000, 256, 8192, "second call, smaller split")


def test_noalloc_unsplit_calls(gpu_lib):
    rng = np.random.default_rng(7071)
    _dgrad_case(gpu_lib, rng, 512, 1024, 1024, "dgrad without split")
    m, n, k = 300, 384, 640
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (n // 128, k // 128))
    dqa, dsa, dqb, dsb = to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)
    c_ref = gpu_lib.fp8bs_gemm(dqa, dsa, dqb, dsb)
    c_na = gpu_lib.fp8bs_gemm_noalloc(dqa, dsa, dqb, dsb)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(c_na), _bits(c_ref))
    c64 = gemm_fprop(qa, sa, qb, sb)
    mag = gemm_fprop(magnitude_codes(qa), sa, magnitude_codes(qb), sb)
    assert_gemm_parity(bf16_values_host(c_na), c64, mag, label="noalloc forward 300x384x640")


def test_noalloc_argument_errors(gpu_lib):
    f = gpu_lib.raw.fp8bs_gemm_noalloc
    p = 0x100000
    assert f(None, p, p, p, 4, 128, 128, 0, p, 128, None) == -1
    assert f(p, p, p, p, 4, 128, 128, 2, p, 128, None) == -4
    assert f(p, p, p, p, 4, 100, 128, 0, p, 128, None) == -2
