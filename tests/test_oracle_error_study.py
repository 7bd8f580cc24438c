"""Quantization error of the fine-grained scheme against one scale per tensor.

The pages give the 1x128 / 128x128 groups as the replacement for per-tensor
scaling, whose single scale is set by the largest element and so leaves the
other values few significant bits when activations have outlier channels
(qqstock.cn page, FP8 section; "DeepSeek-V3 技术报告深度解读", section 3).
This study measures both on the same inputs: the c2 layer's activations (1% of
the channels x50) and weights, 512 tokens, against the unquantized float64
product of the bf16 values.

Pins of ``quantize_per_tensor`` (independent of its code): a 1x128 tensor is a
single tile (the pinned tile quantizer); power-of-two scaling invariance; the
amax element encodes to +-448.
"""

import numpy as np

from oracle import (bf16_to_f32, e4m3_decode, gemm_fprop, quantize_act_1x128, quantize_per_tensor,
                    quantize_w_128x128)
from workloads import f32_to_bf16_bits, gemm_inputs


def test_per_tensor_pins():
    rng = np.random.default_rng(1)
    x = f32_to_bf16_bits(rng.standard_normal((1, 128)).astype(np.float32) * np.float32(5))
    q, s = quantize_per_tensor(x)
    qt, st = quantize_act_1x128(x)
    assert np.array_equal(q, qt) and s == st[0, 0]
    y = f32_to_bf16_bits(rng.standard_normal((64, 300)).astype(np.float32))
    q1, s1 = quantize_per_tensor(y)
    q2, s2 = quantize_per_tensor(f32_to_bf16_bits(bf16_to_f32(y) * np.float32(2.0 ** -9)))
    assert np.array_equal(q1, q2) and s2 == s1 * np.float32(2.0 ** -9)
    assert np.max(e4m3_decode(q1 & 0x7F)) == 448.0


def _study(tokens=512, outliers=True):
    d = gemm_inputs("c2", n_outlier_cols=72 if outliers else 0)
    a_bits, b_bits = d["a"][:tokens], d["b"]
    a, b = bf16_to_f32(a_bits).astype(np.float64), bf16_to_f32(b_bits).astype(np.float64)
    exact = a @ b.T
    nrm = np.linalg.norm(exact)
    qa, sa = quantize_act_1x128(a_bits)
    qb, sb = quantize_w_128x128(b_bits)
    fine = gemm_fprop(qa, sa, qb, sb)
    ta, tsa = quantize_per_tensor(a_bits)
    tb, tsb = quantize_per_tensor(b_bits)
    tensor = (e4m3_decode(ta) * float(tsa)) @ (e4m3_decode(tb) * float(tsb)).T
    rec_fine = e4m3_decode(qa) * np.repeat(sa.astype(np.float64), 128, axis=1)
    rec_tensor = e4m3_decode(ta) * float(tsa)
    na = np.linalg.norm(a)
    return dict(gemm_fine=np.linalg.norm(fine - exact) / nrm, gemm_tensor=np.linalg.norm(tensor - exact) / nrm,
                act_fine=np.linalg.norm(rec_fine - a) / na, act_tensor=np.linalg.norm(rec_tensor - a) / na,
                underflow_tensor=float(np.mean((ta & 0x7F) == 0) - np.mean(a == 0)))


def test_fine_grained_beats_per_tensor_on_outlier_activations():
    r = _study(outliers=True)
    print("[error study] c2 sample, 72 outlier channels x50: " + ", ".join(f"{k} {v:.3e}" for k, v in r.items()))
    assert r["gemm_fine"] < r["gemm_tensor"] and r["act_fine"] < 0.5 * r["act_tensor"]
    assert r["gemm_fine"] < 0.04


def test_gap_narrows_without_outliers():
    r0 = _study(outliers=False)
    r1 = _study(outliers=True)
    print("[error study] c2 sample, no outliers: " + ", ".join(f"{k} {v:.3e}" for k, v in r0.items()))
    # the per-tensor activation error is what the outliers inflate
    assert r1["act_tensor"] / r1["act_fine"] > r0["act_tensor"] / r0["act_fine"]
