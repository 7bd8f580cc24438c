"""The fine-grained path on the GPU, measured against the unquantized product.

Same inputs as the oracle's error study (c2 layer, 512 tokens, 72 outlier
channels x50): the GPU's quantize + forward GEMM must land on the oracle's
fine-grained error (the two differ only by the GEMM's own rounding, about
1.7e-3 normwise against the oracle's result) and below the per-tensor error.
"""

import numpy as np
import pytest

from oracle import bf16_to_f32, e4m3_decode, quantize_per_tensor
from tests.gpu_util import bf16_values_host, to_dev_bf16
from tests.test_oracle_error_study import _study
from workloads import gemm_inputs

pytestmark = pytest.mark.gpu


def test_gpu_error_matches_the_oracle_study(gpu_lib):
    d = gemm_inputs("c2")
    a_bits, b_bits = d["a"][:512], d["b"]
    qa, sa = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(a_bits))
    qb, sb = gpu_lib.fp8bs_quantize_w_128x128(to_dev_bf16(b_bits))
    got = bf16_values_host(gpu_lib.fp8bs_gemm(qa, sa, qb, sb))
    a, b = bf16_to_f32(a_bits).astype(np.float64), bf16_to_f32(b_bits).astype(np.float64)
    exact = a @ b.T
    err_gpu = np.linalg.norm(got - exact) / np.linalg.norm(exact)
    r = _study(outliers=True)
    print(f"[error study] GPU fine-grained {err_gpu:.4e}, oracle fine-grained {r['gemm_fine']:.4e}, "
          f"oracle per-tensor {r['gemm_tensor']:.4e}")
    assert abs(err_gpu - r["gemm_fine"]) < 2e-3
    assert err_gpu < r["gemm_tensor"]
