"""GPU parity of the re-tiling of a cached FP8 activation (tiles along the tokens).

Codes and scales are compared bit for bit with the oracle's
``requantize_act_1x128_t`` (x_hat = fl32(s * dec(q)), then the transposed tile
rules on binary32 values).  Inputs: the GPU's own 1x128 tiles of bf16
activations (already bit-exact with the oracle's), and random codes and scales
fed to both sides (every code class: +-0, subnormals, +-448; zero, subnormal
and huge scales).  At the full layer sizes the launch is the full-size one and
the oracle evaluates sampled 128-channel blocks (an output row depends only on
its own channel).
"""

import numpy as np
import pytest
import torch

from oracle import quantize_act_1x128, quantize_act_1x128_t, requantize_act_1x128_t
from tests.gpu_util import to_dev, to_dev_bf16
from workloads import config_by_name, f32_to_bf16_bits, gemm_inputs, wgrad_inputs

pytestmark = pytest.mark.gpu


def _same(label, q, s, q_ref, s_ref):
    assert q.shape == q_ref.shape and s.shape == s_ref.shape, label
    bad_s = np.argwhere(s.view(np.uint32) != s_ref.view(np.uint32))
    assert bad_s.size == 0, f"{label}: {len(bad_s)} scales differ, first at {tuple(bad_s[0])}"
    bad_q = np.argwhere(q != q_ref)
    assert bad_q.size == 0, (f"{label}: {len(bad_q)} codes differ, first at {tuple(bad_q[0])}: "
                             f"{q[tuple(bad_q[0])]:#x} vs {q_ref[tuple(bad_q[0])]:#x}")


def _random_cache(rng, t, c):
    q = rng.integers(0, 256, size=(t, c)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] &= 0xFE                               # no NaN codes
    q[rng.random((t, c)) < 0.05] = 0x80                         # negative zeros
    s = np.exp(rng.uniform(np.log(1e-30), np.log(1e20), size=(t, c // 128))).astype(np.float32)
    s[rng.random(s.shape) < 0.05] = 0.0                         # all-zero forward tiles
    s[rng.random(s.shape) < 0.03] = np.float32(1e-42)           # subnormal scales
    return q, s


@pytest.mark.parametrize("t,c,seed", [(128, 128, 1), (256, 384, 2), (640, 256, 3)])
def test_random_codes_and_scales(gpu_lib, t, c, seed):
    rng = np.random.default_rng(seed)
    q, s = _random_cache(rng, t, c)
    qt, st = gpu_lib.fp8bs_requantize_act_1x128_t(to_dev(q), to_dev(s))
    torch.cuda.synchronize()
    q_ref, s_ref = requantize_act_1x128_t(q, s)
    _same(f"random {t}x{c}", qt.cpu().numpy(), st.cpu().numpy(), q_ref, s_ref)


def test_gpu_forward_tiles_then_retile_with_strides(gpu_lib):
    rng = np.random.default_rng(9)
    x = f32_to_bf16_bits((rng.standard_normal((384, 512)) * np.exp(rng.uniform(-12, 12, (384, 1)))).astype(np.float32))
    x[:, 130] *= 0                                              # a channel of zeros in every token tile
    x[200:, 300] = 0x8000                                       # negative zeros
    xd = to_dev_bf16(x)
    qbuf = torch.full((384, 640), 0x11, dtype=torch.uint8, device="cuda")
    q, s = gpu_lib.fp8bs_quantize_act_1x128(xd, q=qbuf[:, :512])
    qtbuf = torch.full((512, 528), 0x22, dtype=torch.uint8, device="cuda")
    qt, st = gpu_lib.fp8bs_requantize_act_1x128_t(q, s, qt=qtbuf[:, :384])
    torch.cuda.synchronize()
    oq, osc = quantize_act_1x128(x)
    q_ref, s_ref = requantize_act_1x128_t(oq, osc)
    _same("strided 384x512", qt.cpu().numpy(), st.cpu().numpy(), q_ref, s_ref)
    assert torch.all(qtbuf[:, 384:] == 0x22)                    # row padding of qt untouched


def test_lossless_tiles_match_the_transposed_quantizer(gpu_lib):
    """Power-of-two tile scales with values on the E4M3 grid: re-tiling the cache equals
    quantizing the original bf16 values along the tokens (GPU against GPU, bit for bit)."""
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 0x7F, size=(256, 256)).astype(np.uint8) | (rng.integers(0, 2, (256, 256)) << 7).astype(np.uint8)
    codes[:, ::128] = 0x7E
    s = np.ldexp(1.0, rng.integers(-20, 10, size=(256, 2))).astype(np.float32)
    from oracle import e4m3_decode
    x = f32_to_bf16_bits((e4m3_decode(codes) * np.repeat(s, 128, axis=1)).astype(np.float32))
    qt, st = gpu_lib.fp8bs_requantize_act_1x128_t(*gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(x)))
    qt2, st2 = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(x), transpose=1)
    assert torch.equal(qt, qt2) and torch.equal(st.view(torch.int32), st2.view(torch.int32))


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_full_layer_activation_sampled_channel_blocks(gpu_lib, name):
    """The cached X of a layer (c2: 4096 x 7168; c5: 16384 x 7168): full launch, oracle on
    sampled 128-channel blocks (first, last, two inner ones; c2 includes outlier channels)."""
    cfg = config_by_name(name)
    x = gemm_inputs(cfg)["a"] if name == "c2" else wgrad_inputs(cfg)["x"]
    q, s = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(x))
    qt, st = gpu_lib.fp8bs_requantize_act_1x128_t(q, s)
    torch.cuda.synchronize()
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    nb = x.shape[1] // 128
    for cb in sorted({0, nb - 1, nb // 3, (2 * nb) // 3}):
        q_ref, s_ref = requantize_act_1x128_t(qh[:, 128 * cb:128 * (cb + 1)], sh[:, cb:cb + 1])
        _same(f"{name} channel block {cb}", qt[128 * cb:128 * (cb + 1)].cpu().numpy(),
              st[128 * cb:128 * (cb + 1)].cpu().numpy(), q_ref, s_ref)
    # and the double rounding stays close to quantizing the bf16 values along the tokens directly
    qd, sd = quantize_act_1x128_t(x[:, :128])
    from oracle import e4m3_decode
    direct = e4m3_decode(qd) * np.repeat(sd, 128, axis=1)
    cached = e4m3_decode(qt[:128].cpu().numpy()) * np.repeat(st[:128].cpu().numpy(), 128, axis=1)
    rel = np.linalg.norm(cached - direct) / np.linalg.norm(direct)
    print(f"[requant] {name}: re-tiled cache vs direct transposed tiles, normwise {rel:.3e}")
    # three independent E4M3 roundings (forward tiles, re-tiling, direct tiles), each about
    # 2^-4/sqrt(3) relative RMS: about 0.047 together
    assert rel < 0.06


def test_tall_and_narrow_caches(gpu_lib):
    """65536 tokens x 128 channels (512 squares down one channel block) and 128 x 8192."""
    rng = np.random.default_rng(71)
    for t, c in ((65536, 128), (128, 8192)):
        q, s = _random_cache(rng, t, c)
        qt, st = gpu_lib.fp8bs_requantize_act_1x128_t(to_dev(q), to_dev(s))
        torch.cuda.synchronize()
        q_ref, s_ref = requantize_act_1x128_t(q, s)
        _same(f"{t}x{c}", qt.cpu().numpy(), st.cpu().numpy(), q_ref, s_ref)
