"""GPU parity of the block-scaled GEMMs against the float64 oracle.

Bar (``assert_gemm_parity``): normwise relative error <= 2e-3 vs the oracle
for every output; every element within r * |C64| + 2^-10 * mag of the oracle,
where r is one bf16 ulp (bf16 outputs) or 2^-20 (the weight gradient's f32
outputs) and mag is the sum over K blocks of |sa * sb| * sum |a * b| (the
matrix core's own summation inside a 128-long block is not exact, see
``gpu_util``); bf16 outputs also >= 90% equal to bf16(C64).  Two kinds of input: the configurations' bf16 data run through
GPU quantization (codes already proven bit-exact by the quantizer tests), and
random codes/scales fed identically to both sides (GEMM-only parity).  At full
configuration sizes the launch is the full-size one and the oracle evaluates
sampled output rows (each output row depends only on its own A row).
"""

import numpy as np
import pytest
import torch

from oracle import (gemm_dgrad, gemm_fprop, gemm_wgrad, grouped_gemm, quantize_act_1x128,
                    quantize_act_1x128_t, quantize_w_128x128)
from tests.gpu_util import (assert_gemm_parity, bf16_values_host, magnitude_codes, random_codes,
                            random_scales, to_dev, to_dev_bf16)
from workloads import (config_by_name, device_expert_weights, gemm_inputs, grouped_inputs_host,
                       normal_bf16, wgrad_inputs)

pytestmark = pytest.mark.gpu


def _sample_rows(m, count, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(m, min(count, m), replace=False).tolist())
    rows.update({0, m - 1, min(127, m - 1), min(128, m - 1)})
    return np.array(sorted(rows))


# ---------------------------------------------------------------- forward -----

def test_fprop_random_codes_ragged(gpu_lib):
    rng = np.random.default_rng(200)
    for m, n, k in [(1, 128, 128), (5, 256, 384), (130, 384, 256), (257, 128, 1024), (128, 512, 512)]:
        qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
        sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (n // 128, k // 128))
        c = gpu_lib.fp8bs_gemm(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb))
        got = bf16_values_host(c)
        c64 = gemm_fprop(qa, sa, qb, sb)
        mag = gemm_fprop(magnitude_codes(qa), sa, magnitude_codes(qb), sb)
        assert_gemm_parity(got, c64, mag, label=f"fprop random {m}x{n}x{k}")


def test_fprop_c1_end_to_end(gpu_lib):
    d = gemm_inputs("c1")
    qa, sa = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(d["a"]))
    qb, sb = gpu_lib.fp8bs_quantize_w_128x128(to_dev_bf16(d["b"]))
    c = gpu_lib.fp8bs_gemm(qa, sa, qb, sb)
    got = bf16_values_host(c)
    oqa, osa = quantize_act_1x128(d["a"])
    oqb, osb = quantize_w_128x128(d["b"])
    c64 = gemm_fprop(oqa, osa, oqb, osb)
    mag = gemm_fprop(magnitude_codes(oqa), osa, magnitude_codes(oqb), osb)
    assert_gemm_parity(got, c64, mag, label="c1")
    # per 128x128 output tile
    for i in range(0, 256, 128):
        for j in range(0, 256, 128):
            t64 = c64[i:i + 128, j:j + 128]
            e = np.linalg.norm(got[i:i + 128, j:j + 128] - t64) / np.linalg.norm(t64)
            assert e <= 2.2e-3, (i, j, e)


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_fprop_full_config_sampled_rows(gpu_lib, name):
    d = gemm_inputs(name)
    qa, sa = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(d["a"]))
    qb, sb = gpu_lib.fp8bs_quantize_w_128x128(to_dev_bf16(d["b"]))
    c = gpu_lib.fp8bs_gemm(qa, sa, qb, sb)
    torch.cuda.synchronize()
    rows = _sample_rows(d["a"].shape[0], 48 if name == "c2" else 24)
    got = bf16_values_host(c[torch.from_numpy(rows).cuda()])
    oqa, osa = quantize_act_1x128(d["a"][rows])
    oqb, osb = quantize_w_128x128(d["b"])
    c64 = gemm_fprop(oqa, osa, oqb, osb)
    mag = gemm_fprop(magnitude_codes(oqa), osa, magnitude_codes(oqb), osb)
    assert_gemm_parity(got, c64, mag, label=name)


def test_fprop_strided_output_and_determinism(gpu_lib):
    rng = np.random.default_rng(201)
    m, n, k = 200, 256, 512
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (n // 128, k // 128))
    big = torch.zeros((m, n + 64), dtype=torch.bfloat16, device="cuda")
    dqa, dsa, dqb, dsb = to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)
    gpu_lib.fp8bs_gemm(dqa, dsa, dqb, dsb, c=big[:, :n])
    again = gpu_lib.fp8bs_gemm(dqa, dsa, dqb, dsb)
    torch.cuda.synchronize()
    assert torch.equal(big[:, :n], again)
    assert torch.count_nonzero(big[:, n:]) == 0
    mag = gemm_fprop(magnitude_codes(qa), sa, magnitude_codes(qb), sb)
    assert_gemm_parity(bf16_values_host(again), gemm_fprop(qa, sa, qb, sb), mag, label="strided")


# ---------------------------------------------------------------- dgrad -------

def test_large_ragged_shapes_sampled(gpu_lib):
    """Shapes large enough for the 256 x 128 warp-specialized kernel, with ragged
    edges: M not a multiple of 256 (forward, dgrad, wgrad) and, for the weight
    gradient, N not a multiple of 128.  Random codes and scales fed to both
    sides; the oracle checks sampled rows (including the last ones)."""
    rng = np.random.default_rng(210)
    m, n, k = 4096 + 77, 1536 + 128, 1024
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (n // 128, k // 128))
    rows = _sample_rows(m, 24)
    got = bf16_values_host(gpu_lib.fp8bs_gemm(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)))[rows]
    c64 = gemm_fprop(qa[rows], sa[rows], qb, sb)
    mag = gemm_fprop(magnitude_codes(qa[rows]), sa[rows], magnitude_codes(qb), sb)
    assert_gemm_parity(got, c64, mag, label=f"fprop large ragged {m}x{n}x{k}")
    # dgrad with the [K, N] weight: contraction n, output [m, ko]
    ko = 2048
    qw, sw = random_codes(rng, (n, ko)), random_scales(rng, (n // 128, ko // 128))
    qd, sd = random_codes(rng, (m, n)), random_scales(rng, (m, n // 128))
    got = bf16_values_host(gpu_lib.fp8bs_gemm(to_dev(qd), to_dev(sd), to_dev(qw), to_dev(sw), b_layout=1))[rows]
    c64 = gemm_dgrad(qd[rows], sd[rows], qw, sw)
    mag = gemm_dgrad(magnitude_codes(qd[rows]), sd[rows], magnitude_codes(qw), sw)
    assert_gemm_parity(got, c64, mag, label=f"dgrad large ragged {m}x{ko}x{n}")
    # wgrad: C f32 [mw, nw] over t tokens, nw % 128 != 0
    mw, nw, t = 1536 + 64, 7168 + 36, 1024
    qa2, qb2 = random_codes(rng, (mw, t)), random_codes(rng, (nw, t))
    sa2, sb2 = random_scales(rng, (mw, t // 128)), random_scales(rng, (nw, t // 128))
    out = gpu_lib.fp8bs_gemm_wgrad(to_dev(qa2), to_dev(sa2), to_dev(qb2), to_dev(sb2))
    torch.cuda.synchronize()
    wr = _sample_rows(mw, 12)
    cols = np.unique(np.concatenate([_sample_rows(nw, 64, seed=3), np.arange(nw - 40, nw)]))
    got = out.cpu().numpy()[np.ix_(wr, cols)].astype(np.float64)
    c64 = gemm_wgrad(qa2[wr], sa2[wr], qb2[cols], sb2[cols])
    mag = gemm_wgrad(magnitude_codes(qa2[wr]), sa2[wr], magnitude_codes(qb2[cols]), sb2[cols])
    assert_gemm_parity(got, c64, mag, out_bf16=False, label=f"wgrad large ragged {mw}x{nw}x{t}")


def test_xcd_banded_tile_order_full_outputs(gpu_lib):
    """Shapes whose operands outweigh half their output, so the launch walks the
    tiles in the XCD-aware banded order: tile counts that do not split evenly
    over 8 XCDs (221, 399) and bands whose last one is shorter (17 m-tiles in
    bands of 5), on both GEMM kernels.  The output is filled with NaN first and
    every element is compared with the oracle, so a tile mapped twice or never
    fails."""
    rng = np.random.default_rng(211)

    def nan_bf16(m, n):
        return torch.full((m, n), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)

    for m, n, k in [(4173, 1664, 1280), (1000, 640, 2048)]:
        qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
        sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (n // 128, k // 128))
        c = nan_bf16(m, n)
        gpu_lib.fp8bs_gemm(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), c=c)
        got = bf16_values_host(c)
        c64 = gemm_fprop(qa, sa, qb, sb)
        mag = gemm_fprop(magnitude_codes(qa), sa, magnitude_codes(qb), sb)
        assert_gemm_parity(got, c64, mag, label=f"fprop banded order {m}x{n}x{k}")
    m, kc, ko = 1000, 1536, 768           # dgrad: contraction kc, output [m, ko]
    qd, sd = random_codes(rng, (m, kc)), random_scales(rng, (m, kc // 128))
    qw, sw = random_codes(rng, (kc, ko)), random_scales(rng, (kc // 128, ko // 128))
    c = nan_bf16(m, ko)
    gpu_lib.fp8bs_gemm(to_dev(qd), to_dev(sd), to_dev(qw), to_dev(sw), b_layout=1, c=c)
    got = bf16_values_host(c)
    c64 = gemm_dgrad(qd, sd, qw, sw)
    mag = gemm_dgrad(magnitude_codes(qd), sd, magnitude_codes(qw), sw)
    assert_gemm_parity(got, c64, mag, label=f"dgrad banded order {m}x{ko}x{kc}")
    mw, nw, t = 1600, 7204, 4096
    qa2, qb2 = random_codes(rng, (mw, t)), random_codes(rng, (nw, t))
    sa2, sb2 = random_scales(rng, (mw, t // 128)), random_scales(rng, (nw, t // 128))
    out = torch.full((mw, nw), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.fp8bs_gemm_wgrad(to_dev(qa2), to_dev(sa2), to_dev(qb2), to_dev(sb2), c=out)
    got = out.cpu().numpy().astype(np.float64)
    c64 = gemm_wgrad(qa2, sa2, qb2, sb2)
    mag = gemm_wgrad(magnitude_codes(qa2), sa2, magnitude_codes(qb2), sb2)
    assert_gemm_parity(got, c64, mag, out_bf16=False, label=f"wgrad banded order {mw}x{nw}x{t}")


def test_persistent_tiles_full_outputs(gpu_lib):
    """Shapes with more 256x128 (or 192x128) tiles than CUs, so each workgroup
    of the warp-specialized kernel walks several tiles and the LDS ring runs
    across tile boundaries: forward 8200x1664x1024 (429 tiles), dgrad
    4173x2304 over 1536 (396 tiles of 192 rows), weight gradient 1100x7204 over 1024
    tokens (342 tiles of 192 rows).  Ragged M (and N for the weight gradient);
    NaN-filled outputs compared element by element with the oracle."""
    rng = np.random.default_rng(212)

    def nan_bf16(m, n):
        return torch.full((m, n), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)

    m, n, k = 8200, 1664, 1024
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (n // 128, k // 128))
    c = nan_bf16(m, n)
    gpu_lib.fp8bs_gemm(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), c=c)
    mag = gemm_fprop(magnitude_codes(qa), sa, magnitude_codes(qb), sb)
    assert_gemm_parity(bf16_values_host(c), gemm_fprop(qa, sa, qb, sb), mag, label=f"fprop persistent {m}x{n}x{k}")
    m, kc, ko = 4173, 1536, 2304
    qd, sd = random_codes(rng, (m, kc)), random_scales(rng, (m, kc // 128))
    qw, sw = random_codes(rng, (kc, ko)), random_scales(rng, (kc // 128, ko // 128))
    c = nan_bf16(m, ko)
    gpu_lib.fp8bs_gemm(to_dev(qd), to_dev(sd), to_dev(qw), to_dev(sw), b_layout=1, c=c)
    mag = gemm_dgrad(magnitude_codes(qd), sd, magnitude_codes(qw), sw)
    assert_gemm_parity(bf16_values_host(c), gemm_dgrad(qd, sd, qw, sw), mag, label=f"dgrad persistent {m}x{ko}x{kc}")
    mw, nw, t = 1100, 7204, 1024
    qa2, qb2 = random_codes(rng, (mw, t)), random_codes(rng, (nw, t))
    sa2, sb2 = random_scales(rng, (mw, t // 128)), random_scales(rng, (nw, t // 128))
    out = torch.full((mw, nw), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.fp8bs_gemm_wgrad(to_dev(qa2), to_dev(sa2), to_dev(qb2), to_dev(sb2), c=out)
    got = out.cpu().numpy().astype(np.float64)
    mag = gemm_wgrad(magnitude_codes(qa2), sa2, magnitude_codes(qb2), sb2)
    assert_gemm_parity(got, gemm_wgrad(qa2, sa2, qb2, sb2), mag, out_bf16=False,
                       label=f"wgrad persistent {mw}x{nw}x{t}")


def test_wide_forward_tiles_full_output(gpu_lib):
    """A forward shape whose 256x128 tiles would leave CUs idle (198 tiles),
    so the launch takes 128x192 tiles (255 of them): ragged M (2113) and a
    last tile column 128 wide (2816 = 14 x 192 + 128); the 48-column wave
    patches straddle 128-column weight blocks, so each 16-column MFMA tile
    takes its own weight scale."""
    rng = np.random.default_rng(213)
    m, n, k = 2113, 2816, 1024
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (n // 128, k // 128))
    c = torch.full((m, n), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    gpu_lib.fp8bs_gemm(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), c=c)
    mag = gemm_fprop(magnitude_codes(qa), sa, magnitude_codes(qb), sb)
    assert_gemm_parity(bf16_values_host(c), gemm_fprop(qa, sa, qb, sb), mag, label=f"fprop wide {m}x{n}x{k}")


def test_mid_size_full_outputs(gpu_lib):
    """Mid-size problems (about 2048x2048: 192x128 tiles for 0.7 of the CUs, fewer
    256x128 tiles than three quarters of them) run the warp-specialized kernel on
    one round of tiles: forward, dgrad and weight gradient, ragged M for the
    forward, every element compared with the oracle."""
    rng = np.random.default_rng(214)
    m, n, k = 2000, 2048, 512
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (n // 128, k // 128))
    got = bf16_values_host(gpu_lib.fp8bs_gemm(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)))
    mag = gemm_fprop(magnitude_codes(qa), sa, magnitude_codes(qb), sb)
    assert_gemm_parity(got, gemm_fprop(qa, sa, qb, sb), mag, label=f"fprop mid {m}x{n}x{k}")
    m, kc, ko = 2048, 512, 2048
    qd, sd = random_codes(rng, (m, kc)), random_scales(rng, (m, kc // 128))
    qw, sw = random_codes(rng, (kc, ko)), random_scales(rng, (kc // 128, ko // 128))
    got = bf16_values_host(gpu_lib.fp8bs_gemm(to_dev(qd), to_dev(sd), to_dev(qw), to_dev(sw), b_layout=1))
    mag = gemm_dgrad(magnitude_codes(qd), sd, magnitude_codes(qw), sw)
    assert_gemm_parity(got, gemm_dgrad(qd, sd, qw, sw), mag, label=f"dgrad mid {m}x{ko}x{kc}")
    mw, nw, t = 2048, 2048, 512
    qa2, qb2 = random_codes(rng, (mw, t)), random_codes(rng, (nw, t))
    sa2, sb2 = random_scales(rng, (mw, t // 128)), random_scales(rng, (nw, t // 128))
    out = gpu_lib.fp8bs_gemm_wgrad(to_dev(qa2), to_dev(sa2), to_dev(qb2), to_dev(sb2))
    got = out.cpu().numpy().astype(np.float64)
    mag = gemm_wgrad(magnitude_codes(qa2), sa2, magnitude_codes(qb2), sb2)
    assert_gemm_parity(got, gemm_wgrad(qa2, sa2, qb2, sb2), mag, out_bf16=False, label=f"wgrad mid {mw}x{nw}x{t}")


def test_dgrad_random_codes(gpu_lib):
    rng = np.random.default_rng(202)
    for m, k, n in [(3, 128, 128), (130, 256, 384), (256, 384, 256)]:      # contraction k, output n
        qa, qw = random_codes(rng, (m, k)), random_codes(rng, (k, n))
        sa, sw = random_scales(rng, (m, k // 128)), random_scales(rng, (k // 128, n // 128))
        c = gpu_lib.fp8bs_gemm(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw), b_layout=1)
        got = bf16_values_host(c)
        c64 = gemm_dgrad(qa, sa, qw, sw)
        mag = gemm_dgrad(magnitude_codes(qa), sa, magnitude_codes(qw), sw)
        assert_gemm_parity(got, c64, mag, label=f"dgrad {m}x{k}x{n}")


def test_dgrad_mla_shape_sampled_rows(gpu_lib):
    """dX [4096, 7168] = dY [4096, 1536] W [1536, 7168] with the forward weight as stored."""
    cfg = config_by_name("c2")
    d = gemm_inputs("c2")
    rng = np.random.default_rng(203)
    dy = (rng.standard_normal((cfg["M"], cfg["N"])) * 1e-3).astype(np.float32)
    from workloads import f32_to_bf16_bits
    dy_bits = f32_to_bf16_bits(dy)
    qdy, sdy = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(dy_bits))
    qw, sw = gpu_lib.fp8bs_quantize_w_128x128(to_dev_bf16(d["b"]))
    dx = gpu_lib.fp8bs_gemm(qdy, sdy, qw, sw, b_layout=1)
    torch.cuda.synchronize()
    rows = _sample_rows(cfg["M"], 24)
    got = bf16_values_host(dx[torch.from_numpy(rows).cuda()])
    oq, os_ = quantize_act_1x128(dy_bits[rows])
    oqw, osw = quantize_w_128x128(d["b"])
    c64 = gemm_dgrad(oq, os_, oqw, osw)
    mag = gemm_dgrad(magnitude_codes(oq), os_, magnitude_codes(oqw), osw)
    assert_gemm_parity(got, c64, mag, label="dgrad mla")


# ---------------------------------------------------------------- wgrad -------

def test_wgrad_random_codes_ragged_and_accumulate(gpu_lib):
    rng = np.random.default_rng(204)
    for m, n, t in [(1, 4, 128), (130, 136, 384), (256, 260, 256)]:
        qa, qb = random_codes(rng, (m, t)), random_codes(rng, (n, t))
        sa, sb = random_scales(rng, (m, t // 128)), random_scales(rng, (n, t // 128))
        args = (to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb))
        c = gpu_lib.fp8bs_gemm_wgrad(*args)
        c64 = gemm_wgrad(qa, sa, qb, sb)
        mag = gemm_wgrad(magnitude_codes(qa), sa, magnitude_codes(qb), sb)
        assert_gemm_parity(c.cpu().numpy(), c64, mag, out_bf16=False, label=f"wgrad {m}x{n}x{t}")
        gpu_lib.fp8bs_gemm_wgrad(*args, c=c, accumulate=1)
        assert_gemm_parity(c.cpu().numpy(), 2 * c64, 2 * mag, out_bf16=False, label="wgrad accumulate")


def test_wgrad_split_contraction(gpu_lib):
    """Weight gradients whose output tiles fill at most half the CUs and whose token
    contraction is long split it (FP32 partials summed in split order, then added
    to C with accumulate): ragged M and N, splits of 2 to 4, overwrite then
    accumulate into a strided output whose padding columns keep their sentinel."""
    rng = np.random.default_rng(243)
    for m, n, t in [(300, 1000, 8192), (512, 2048, 4096), (256, 7168, 16384)]:
        qa, qb = random_codes(rng, (m, t)), random_codes(rng, (n, t))
        sa, sb = random_scales(rng, (m, t // 128)), random_scales(rng, (n, t // 128))
        args = (to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb))
        big = torch.full((m, n + 8), -7.0, dtype=torch.float32, device="cuda")
        gpu_lib.fp8bs_gemm_wgrad(*args, c=big[:, :n])
        torch.cuda.synchronize()
        assert bool((big[:, n:] == -7.0).all())
        rows = _sample_rows(m, 48, seed=t) if m * n * t > 2 ** 33 else np.arange(m)
        c64 = gemm_wgrad(qa[rows], sa[rows], qb, sb)
        mag = gemm_wgrad(magnitude_codes(qa[rows]), sa[rows], magnitude_codes(qb), sb)
        assert_gemm_parity(big[:, :n].cpu().numpy()[rows], c64, mag, out_bf16=False, label=f"wgrad split {m}x{n}x{t}")
        gpu_lib.fp8bs_gemm_wgrad(*args, c=big[:, :n], accumulate=1)
        torch.cuda.synchronize()
        assert bool((big[:, n:] == -7.0).all())
        assert_gemm_parity(big[:, :n].cpu().numpy()[rows], 2 * c64, 2 * mag, out_bf16=False,
                           label=f"wgrad split accumulate {m}x{n}x{t}")


def test_wgrad_split_is_deterministic(gpu_lib):
    """The split's partials are summed in a fixed order: two runs agree bit for bit."""
    rng = np.random.default_rng(244)
    m, n, t = 384, 1536, 16384
    qa, qb = random_codes(rng, (m, t)), random_codes(rng, (n, t))
    sa, sb = random_scales(rng, (m, t // 128)), random_scales(rng, (n, t // 128))
    args = (to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb))
    c1 = gpu_lib.fp8bs_gemm_wgrad(*args)
    c2 = gpu_lib.fp8bs_gemm_wgrad(*args)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


def test_wgrad_c5_sampled_block(gpu_lib):
    """Full-size launch; the oracle checks sampled rows x sampled columns of dW.

    dW[i, j] depends only on dY channel i and X channel j, so the oracle quantizes
    just those channels (transposed tiles along the 16384 tokens)."""
    d = wgrad_inputs("c5")
    qdy, sdy = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(d["dy"]), transpose=1)   # [1536, 16384]
    qx, sx = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(d["x"]), transpose=1)      # [7168, 16384]
    dw = gpu_lib.fp8bs_gemm_wgrad(qdy, sdy, qx, sx)
    torch.cuda.synchronize()
    rows = _sample_rows(qdy.shape[0], 12)
    cols = _sample_rows(qx.shape[0], 192, seed=1)
    got = dw[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy()
    oqdy, osdy = quantize_act_1x128_t(np.ascontiguousarray(d["dy"][:, rows]))
    oqx, osx = quantize_act_1x128_t(np.ascontiguousarray(d["x"][:, cols]))
    c64 = gemm_wgrad(oqdy, osdy, oqx, osx)
    mag = gemm_wgrad(magnitude_codes(oqdy), osdy, magnitude_codes(oqx), osx)
    assert_gemm_parity(got, c64, mag, out_bf16=False, label="c5")


# ---------------------------------------------------------------- grouped -----

def _grouped_host_small():
    cfg = dict(kind="grouped", seed=9, tokens=160, topk=4, experts=7, N=256, K=384, zipf_s=1.1,
               a_std=1.0, b_std=0.02)
    return cfg, grouped_inputs_host(cfg)


def test_grouped_small_end_to_end(gpu_lib):
    cfg, g = _grouped_host_small()
    off = g["offsets"]
    qa, sa = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(g["x"]))
    qb, sb = gpu_lib.fp8bs_quantize_w_128x128(to_dev_bf16(g["w"]))
    c = gpu_lib.fp8bs_grouped_gemm(qa, sa, to_dev(off.astype(np.int32)), qb, sb)
    got = bf16_values_host(c)
    oqa, osa = quantize_act_1x128(g["x"])
    ws = [quantize_w_128x128(g["w"][e]) for e in range(cfg["experts"])]
    oqb, osb = np.stack([w[0] for w in ws]), np.stack([w[1] for w in ws])
    c64 = grouped_gemm(oqa, osa, off, oqb, osb)
    real = np.ones(off[-1], bool)
    for e in range(cfg["experts"]):
        real[off[e] + g["counts"][e]:off[e + 1]] = False
    mag = grouped_gemm(magnitude_codes(oqa), osa, off, magnitude_codes(oqb), osb)
    assert_gemm_parity(got[real], c64[real], mag[real], label="grouped small")
    assert np.all(got[~real] == 0)
    # equals per-expert plain GEMM calls on the same codes, bit for bit
    for e in range(cfg["experts"]):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            ce = gpu_lib.fp8bs_gemm(qa[lo:hi].contiguous(), sa[lo:hi].contiguous(), qb[e].contiguous(),
                                    sb[e].contiguous())
            assert torch.equal(ce, c[lo:hi])


def test_grouped_empty_and_single_expert(gpu_lib):
    """Empty segments, one expert owning every row; n = 128 runs the 128 x 128
    kernel, n = 512 the 128 x 256 warp-specialized one."""
    rng = np.random.default_rng(205)
    k = 256
    qa, sa = random_codes(rng, (384, k)), random_scales(rng, (384, k // 128))
    for n in (128, 512):
        qb, sb = random_codes(rng, (4, n, k)), random_scales(rng, (4, n // 128, k // 128))
        for off in ([0, 0, 384, 384, 384], [0, 128, 128, 256, 384], [0, 384, 384, 384, 384]):
            off = np.array(off)
            c = gpu_lib.fp8bs_grouped_gemm(to_dev(qa), to_dev(sa), to_dev(off.astype(np.int32)), to_dev(qb),
                                           to_dev(sb))
            c64 = grouped_gemm(qa, sa, off, qb, sb)
            mag = grouped_gemm(magnitude_codes(qa), sa, off, magnitude_codes(qb), sb)
            assert_gemm_parity(bf16_values_host(c), c64, mag, label=f"grouped n={n} offsets {off.tolist()}")


def test_grouped_row_token_clips_padding(gpu_lib):
    """With the row map, each 128-row tile reads its rows only up to its last
    routed row (row_token >= 0).  Tiles with 128, 1, 2, 127, 64 and 65 live
    rows, one routed row marked -1 inside the live run (still read: only the
    trailing run is padding), and padding rows holding non-zero codes and
    scales, which must not be read.  Both grouped kernels (n = 128: 128 x 128
    tiles, n = 256: 128 x 256 warp-specialized); outputs against the oracle on
    the inputs with the padding zeroed, and bit for bit against the call
    without the row map on those zeroed inputs."""
    rng = np.random.default_rng(233)
    k, live = 384, [128, 1, 2, 127, 64, 65]
    off = np.array([0, 256, 512, 768])                  # three experts of two tiles each
    rows = 128 * len(live)
    rt = np.full(rows, -1, np.int32)
    for t, nl in enumerate(live):
        rt[128 * t:128 * t + nl] = np.arange(nl, dtype=np.int32)
    rt[128 * 3 + 50] = -1                                # inside tile 3's live run
    pad = rt < 0
    pad[128 * 3 + 50] = False
    qa, sa = random_codes(rng, (rows, k)), random_scales(rng, (rows, k // 128))
    qa0, sa0 = qa.copy(), sa.copy()
    qa0[pad], sa0[pad] = 0, 0.0
    for n in (128, 256):
        qb, sb = random_codes(rng, (3, n, k)), random_scales(rng, (3, n // 128, k // 128))
        seg = to_dev(off.astype(np.int32))
        c_rt = gpu_lib.fp8bs_grouped_gemm(to_dev(qa), to_dev(sa), seg, to_dev(qb), to_dev(sb),
                                          row_token=to_dev(rt))
        c_zero = gpu_lib.fp8bs_grouped_gemm(to_dev(qa0), to_dev(sa0), seg, to_dev(qb), to_dev(sb))
        assert torch.equal(c_rt.view(torch.int16), c_zero.view(torch.int16)), f"n={n}"
        got = bf16_values_host(c_rt)
        c64 = grouped_gemm(qa0, sa0, off, qb, sb)
        mag = grouped_gemm(magnitude_codes(qa0), sa0, off, magnitude_codes(qb), sb)
        assert_gemm_parity(got[~pad], c64[~pad], mag[~pad], label=f"row map n={n}")
        assert np.all(bf16_values_host(c_rt)[pad] == 0)
        assert np.all(c_rt.view(torch.int16).cpu().numpy()[pad] == 0)   # +0, not -0


def test_grouped_c4_full_launch_sampled_experts(gpu_lib):
    cfg = config_by_name("c4")
    g = grouped_inputs_host(cfg, with_weights=False)
    off, counts = g["offsets"], g["counts"]
    w = device_expert_weights(cfg)                                 # [256, 4096, 7168] bf16 on the GPU
    qa, sa = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(g["x"]))
    qb, sb = gpu_lib.fp8bs_quantize_w_128x128(w)
    seg = to_dev(off.astype(np.int32))
    c = gpu_lib.fp8bs_grouped_gemm(qa, sa, seg, qb, sb)
    # with the row map (the bench's launch): the same bits over every row
    rt = np.full(int(off[-1]), -1, np.int32)
    for e in range(len(counts)):
        rt[off[e]:off[e] + counts[e]] = np.arange(counts[e], dtype=np.int32)
    c_rt = gpu_lib.fp8bs_grouped_gemm(qa, sa, seg, qb, sb, row_token=to_dev(rt))
    assert torch.equal(c_rt.view(torch.int16), c.view(torch.int16))
    del c_rt
    torch.cuda.synchronize()
    order = np.argsort(counts)
    experts = sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2]), 17})
    for e in experts:
        lo, hi, cnt = int(off[e]), int(off[e + 1]), int(counts[e])
        rows = np.arange(lo, hi)
        if hi - lo > 160:
            rows = np.unique(np.concatenate([rows[:64], rows[-64:], [lo + cnt - 1]]))
        got = bf16_values_host(c[torch.from_numpy(rows).cuda()])
        w_bits = w[e].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        oqb, osb = quantize_w_128x128(w_bits)
        assert np.array_equal(oqb, qb[e].cpu().numpy()) and np.array_equal(osb, sb[e].cpu().numpy())
        oqa, osa = quantize_act_1x128(g["x"][rows])
        c64 = gemm_fprop(oqa, osa, oqb, osb)
        realm = rows < lo + cnt
        mag = gemm_fprop(magnitude_codes(oqa), osa, magnitude_codes(oqb), osb)
        assert_gemm_parity(got[realm], c64[realm], mag[realm], label=f"c4 expert {e}")
        assert np.all(got[~realm] == 0)
    del w


def test_warp_specialized_strided_outputs(gpu_lib):
    """Outputs whose row stride runs past their columns (ldc > n) on the
    warp-specialized kernels: the 128x192 forward tiles (two adjacent MFMA
    tiles stored together, an odd third one alone), the persistent dgrad
    kernel and the weight gradient with accumulate.  Full outputs against the
    oracle; the columns between n and ldc keep their sentinel."""
    rng = np.random.default_rng(231)

    m, n, k = 2113, 2816, 256                      # 198 tiles of 256x128: 128x192 tiles instead
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (n // 128, k // 128))
    big = torch.full((m, n + 64), -1, dtype=torch.int16, device="cuda")
    gpu_lib.fp8bs_gemm(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), c=big.view(torch.bfloat16)[:, :n])
    torch.cuda.synchronize()
    assert bool((big[:, n:] == -1).all())
    mag = gemm_fprop(magnitude_codes(qa), sa, magnitude_codes(qb), sb)
    assert_gemm_parity(bf16_values_host(big.view(torch.bfloat16)[:, :n]), gemm_fprop(qa, sa, qb, sb), mag,
                       label=f"fprop strided {m}x{n}x{k}")

    mo, ko, kc = 2304, 4096, 256                   # dX [mo, ko] = dY [mo, kc] W [kc, ko]: more tiles than CUs
    qd, sd = random_codes(rng, (mo, kc)), random_scales(rng, (mo, kc // 128))
    qw, sw = random_codes(rng, (kc, ko)), random_scales(rng, (kc // 128, ko // 128))
    big = torch.full((mo, ko + 128), -1, dtype=torch.int16, device="cuda")
    gpu_lib.fp8bs_gemm(to_dev(qd), to_dev(sd), to_dev(qw), to_dev(sw), b_layout=1,
                       c=big.view(torch.bfloat16)[:, :ko])
    torch.cuda.synchronize()
    assert bool((big[:, ko:] == -1).all())
    mag = gemm_dgrad(magnitude_codes(qd), sd, magnitude_codes(qw), sw)
    assert_gemm_parity(bf16_values_host(big.view(torch.bfloat16)[:, :ko]), gemm_dgrad(qd, sd, qw, sw), mag,
                       label=f"dgrad strided {mo}x{ko}x{kc}")

    mw, nw, t = 1536, 4608, 256
    qa2, qb2 = random_codes(rng, (mw, t)), random_codes(rng, (nw, t))
    sa2, sb2 = random_scales(rng, (mw, t // 128)), random_scales(rng, (nw, t // 128))
    args = (to_dev(qa2), to_dev(sa2), to_dev(qb2), to_dev(sb2))
    big = torch.full((mw, nw + 32), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.fp8bs_gemm_wgrad(*args, c=big[:, :nw])
    c64 = gemm_wgrad(qa2, sa2, qb2, sb2)
    mag = gemm_wgrad(magnitude_codes(qa2), sa2, magnitude_codes(qb2), sb2)
    assert_gemm_parity(big[:, :nw].cpu().numpy(), c64, mag, out_bf16=False, label=f"wgrad strided {mw}x{nw}x{t}")
    gpu_lib.fp8bs_gemm_wgrad(*args, c=big[:, :nw], accumulate=1)
    assert_gemm_parity(big[:, :nw].cpu().numpy(), 2 * c64, 2 * mag, out_bf16=False, label="wgrad strided accumulate")
    assert bool(torch.isnan(big[:, nw:]).all())


def test_dgrad_split_contraction(gpu_lib):
    """Activation gradients whose 256x128 tiles fill at most half the CUs and
    whose contraction is long split the contraction over workgroups (FP32
    partials summed in split order, one rounding to bf16): ragged M, splits of
    4 and 2, a strided output whose padding columns keep their sentinel."""
    rng = np.random.default_rng(241)
    for mo, ko, kc in [(1000, 256, 8192), (300, 512, 4096), (4096, 512, 32768)]:
        qd, sd = random_codes(rng, (mo, kc)), random_scales(rng, (mo, kc // 128))
        qw, sw = random_codes(rng, (kc, ko)), random_scales(rng, (kc // 128, ko // 128))
        big = torch.full((mo, ko + 64), -1, dtype=torch.int16, device="cuda")
        gpu_lib.fp8bs_gemm(to_dev(qd), to_dev(sd), to_dev(qw), to_dev(sw), b_layout=1,
                           c=big.view(torch.bfloat16)[:, :ko])
        torch.cuda.synchronize()
        assert bool((big[:, ko:] == -1).all())
        got = bf16_values_host(big.view(torch.bfloat16)[:, :ko])
        rows = _sample_rows(mo, 96, seed=kc) if mo * kc > 2 ** 26 else np.arange(mo)
        mag = gemm_dgrad(magnitude_codes(qd[rows]), sd[rows], magnitude_codes(qw), sw)
        assert_gemm_parity(got[rows], gemm_dgrad(qd[rows], sd[rows], qw, sw), mag,
                           label=f"dgrad split {mo}x{ko}x{kc}")


def test_forward_split_contraction(gpu_lib):
    """Forward GEMMs too small for the warp-specialized kernel (192x128 tiles for
    fewer than half the CUs) with a long contraction split it like the dgrad:
    ragged M, the MLA latent projection 4096x640x7168 (split 2), splits of 4,
    a strided output whose padding columns keep their sentinel."""
    rng = np.random.default_rng(242)
    for m, n, k in [(1000, 256, 8192), (4096, 640, 7168), (4096, 512, 16384), (300, 512, 4096)]:
        qa, sa = random_codes(rng, (m, k)), random_scales(rng, (m, k // 128))
        qb, sb = random_codes(rng, (n, k)), random_scales(rng, (n // 128, k // 128))
        big = torch.full((m, n + 64), -1, dtype=torch.int16, device="cuda")
        gpu_lib.fp8bs_gemm(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), c=big.view(torch.bfloat16)[:, :n])
        torch.cuda.synchronize()
        assert bool((big[:, n:] == -1).all())
        got = bf16_values_host(big.view(torch.bfloat16)[:, :n])
        rows = _sample_rows(m, 96, seed=k) if m * k > 2 ** 26 else np.arange(m)
        mag = gemm_fprop(magnitude_codes(qa[rows]), sa[rows], magnitude_codes(qb), sb)
        assert_gemm_parity(got[rows], gemm_fprop(qa[rows], sa[rows], qb, sb), mag,
                           label=f"fprop split {m}x{n}x{k}")


# --------------------------------------------------------- random shape sweep -----

def _sweep_shapes(seed, count):
    """Seeded shapes that cross the launch choices (small, 128x128, warp-specialized,
    persistent, 128x192): M ragged, N and K multiples of 128."""
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(count):
        m = int(rng.choice([rng.integers(1, 300), rng.integers(300, 3000), rng.integers(3000, 9000)]))
        n = 128 * int(rng.integers(1, 64))
        k = 128 * int(rng.integers(1, 24))
        shapes.append((m, n, k))
    return shapes


@pytest.mark.parametrize("m,n,k", _sweep_shapes(301, 14))
def test_forward_and_dgrad_shape_sweep(gpu_lib, m, n, k):
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    rows = _sample_rows(m, 6)
    qa, sa = random_codes(rng, (m, k)), random_scales(rng, (m, k // 128))
    qb, sb = random_codes(rng, (n, k)), random_scales(rng, (n // 128, k // 128))
    got = bf16_values_host(gpu_lib.fp8bs_gemm(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)))[rows]
    c64 = gemm_fprop(qa[rows], sa[rows], qb, sb)
    mag = gemm_fprop(magnitude_codes(qa[rows]), sa[rows], magnitude_codes(qb), sb)
    assert_gemm_parity(got, c64, mag, label=f"fprop sweep {m}x{n}x{k}")
    # dgrad: contraction n (as k here), weight stored [k_contr, n_out]
    qw, sw = random_codes(rng, (k, n)), random_scales(rng, (k // 128, n // 128))
    got = bf16_values_host(gpu_lib.fp8bs_gemm(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw), b_layout=1))[rows]
    c64 = gemm_dgrad(qa[rows], sa[rows], qw, sw)
    mag = gemm_dgrad(magnitude_codes(qa[rows]), sa[rows], magnitude_codes(qw), sw)
    assert_gemm_parity(got, c64, mag, label=f"dgrad sweep {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,t", [(s[0] % 2500 + 1, s[1] + 4 * (s[2] // 128 % 5), s[2]) for s in _sweep_shapes(302, 8)])
def test_wgrad_shape_sweep(gpu_lib, m, n, t):
    rng = np.random.default_rng(m + 11 * n + t)
    qa, sa = random_codes(rng, (m, t)), random_scales(rng, (m, t // 128))
    qb, sb = random_codes(rng, (n, t)), random_scales(rng, (n, t // 128))
    out = gpu_lib.fp8bs_gemm_wgrad(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb))
    torch.cuda.synchronize()
    wr = _sample_rows(m, 6)
    cols = np.unique(np.concatenate([_sample_rows(n, 48, seed=5), np.arange(max(0, n - 8), n)]))
    got = out.cpu().numpy()[np.ix_(wr, cols)].astype(np.float64)
    c64 = gemm_wgrad(qa[wr], sa[wr], qb[cols], sb[cols])
    mag = gemm_wgrad(magnitude_codes(qa[wr]), sa[wr], magnitude_codes(qb[cols]), sb[cols])
    assert_gemm_parity(got, c64, mag, out_bf16=False, label=f"wgrad sweep {m}x{n}x{t}")


# ------------------------------------------------ grouped, bf16 weights -----

def _special_weights(rng, num_e, n, k):
    """bf16 expert weights N(0, 0.02) with special 128x128 blocks: all zero,
    tiny (amax below 2^-64, with subnormals: the scaled coding path), and
    large (|w| up to ~3e4)."""
    w = normal_bf16(rng, (num_e, n, k), 0.02)
    w[0, :128, :128] = 0
    sign = rng.integers(0, 2, size=(128, 128)).astype(np.uint16) << 15
    exp = rng.integers(0, 58, size=(128, 128)).astype(np.uint16)          # <= 2^-70 (0: subnormal)
    w[num_e - 1, n - 128:, k - 128:] = sign | (exp << 7) | rng.integers(0, 128, size=(128, 128)).astype(np.uint16)
    big = rng.integers(0x4500, 0x46F0, size=(128, 128)).astype(np.uint16)  # 2048 .. ~30000
    w[num_e // 2, :128, k - 128:] = big | (rng.integers(0, 2, size=(128, 128)).astype(np.uint16) << 15)
    return w


def _routed_rows(counts):
    """Padded segment starts and the row map (-1 on padding) for the counts."""
    off = np.concatenate([[0], np.cumsum((np.asarray(counts) + 127) // 128 * 128)]).astype(np.int64)
    rt = np.full(int(off[-1]), -1, np.int32)
    for e, cnt in enumerate(counts):
        rt[off[e]:off[e] + cnt] = np.arange(cnt, dtype=np.int32)
    return off, rt


@pytest.mark.parametrize("k,counts", [(128, [130, 0, 1, 256, 77]), (256, [130, 0, 1, 256, 77]),
                                      (384, [130, 0, 1, 256, 77]), (512, [130, 0, 1, 256, 77]),
                                      (640, [130, 0, 1, 256, 77]), (768, [130, 0, 1, 256, 77]),
                                      (896, [130, 0, 1, 256, 77]), (384, [0, 5, 0, 300, 0]), (256, [200]),
                                      (1280, [300, 129])])
def test_grouped_bf16w_equals_quantize_then_grouped(gpu_lib, k, counts):
    """The fused call (weights coded in the GEMM's copy waves) against
    fp8bs_quantize_w_128x128 followed by fp8bs_grouped_gemm: C bit for bit,
    with and without the row map; the stored codes and scales equal the block
    quantizer's for every expert with rows and leave an expert without rows
    untouched.  K = 128 .. 1280 runs 1 to 7 and 10 slab units (the copy waves
    alternate two register buffers); the routings include empty first
    and last experts and a single expert.  The first and last experts' stored
    blocks (zero, tiny and large ones) are also checked against the oracle."""
    rng = np.random.default_rng(240 + k + len(counts))
    n = 256
    num_e = len(counts)
    off, rt = _routed_rows(counts)
    rows = int(off[-1])
    qa, sa = random_codes(rng, (rows, k)), random_scales(rng, (rows, k // 128))
    pad = rt < 0
    qa[pad], sa[pad] = 0, 0.0
    w_h = _special_weights(rng, num_e, n, k)
    w = to_dev_bf16(w_h)
    qa_d, sa_d, seg, rt_d = to_dev(qa), to_dev(sa), to_dev(off.astype(np.int32)), to_dev(rt)
    qw_ref, sw_ref = gpu_lib.fp8bs_quantize_w_128x128(w)
    c_ref = gpu_lib.fp8bs_grouped_gemm(qa_d, sa_d, seg, qw_ref, sw_ref, row_token=rt_d)
    qw = torch.full((num_e, n, k), 0x5A, dtype=torch.uint8, device="cuda")
    sw = torch.full((num_e, n // 128, k // 128), -1.0, dtype=torch.float32, device="cuda")
    c = gpu_lib.fp8bs_grouped_gemm_bf16w(qa_d, sa_d, seg, w, qw=qw, sw=sw, row_token=rt_d)
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16)), f"k={k}: C with the row map"
    c2 = gpu_lib.fp8bs_grouped_gemm_bf16w(qa_d, sa_d, seg, w)
    assert torch.equal(c2.view(torch.int16), c_ref.view(torch.int16)), f"k={k}: C without the map"
    for e, cnt in enumerate(counts):
        if cnt:
            assert torch.equal(qw[e], qw_ref[e]) and torch.equal(sw[e].view(torch.int32), sw_ref[e].view(torch.int32)), \
                f"k={k}: stored weights of expert {e}"
        else:
            assert bool((qw[e] == 0x5A).all()) and bool((sw[e] == -1.0).all()), f"k={k}: expert {e} has no rows"
    # keep_codes=False: qw / sw as the call's workspace, holding the codes of
    # the experts with more than one 128-row tile only
    qw3 = torch.full_like(qw, 0x5A)
    sw3 = torch.full_like(sw, -1.0)
    c3 = gpu_lib.fp8bs_grouped_gemm_bf16w(qa_d, sa_d, seg, w, qw=qw3, sw=sw3, row_token=rt_d, keep_codes=False)
    assert torch.equal(c3.view(torch.int16), c_ref.view(torch.int16)), f"k={k}: C, codes of multi-tile experts only"
    for e in range(num_e):
        if off[e + 1] - off[e] > 128:
            assert torch.equal(qw3[e], qw_ref[e]) and torch.equal(sw3[e].view(torch.int32), sw_ref[e].view(torch.int32)), \
                f"k={k}: workspace codes of expert {e}"
        else:
            assert bool((qw3[e] == 0x5A).all()) and bool((sw3[e] == -1.0).all()), f"k={k}: expert {e} not stored"
    for e in sorted({0, num_e - 1}):
        if not counts[e]:
            continue
        oq, os_ = quantize_w_128x128(w_h[e])
        assert np.array_equal(qw[e].cpu().numpy(), oq) and np.array_equal(sw[e].cpu().numpy(), os_), f"oracle, expert {e}"


def test_grouped_bf16w_c4_full_launch(gpu_lib):
    """c4 at full size: the fused call against the two calls, whole outputs
    bit for bit, and the stored weights of every expert with rows; then with
    keep_codes=False: the same output, codes stored for the experts with
    several 128-row tiles only."""
    cfg = config_by_name("c4")
    g = grouped_inputs_host(cfg, with_weights=False)
    off, counts = g["offsets"], g["counts"]
    _, rt = _routed_rows(counts)
    assert np.array_equal(_routed_rows(counts)[0], off)
    w = device_expert_weights(cfg)
    qa, sa = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(g["x"]))
    seg, rt_d = to_dev(off.astype(np.int32)), to_dev(rt)
    qw_ref, sw_ref = gpu_lib.fp8bs_quantize_w_128x128(w)
    c_ref = gpu_lib.fp8bs_grouped_gemm(qa, sa, seg, qw_ref, sw_ref, row_token=rt_d)
    qw, sw = torch.zeros_like(qw_ref), torch.zeros_like(sw_ref)
    c = gpu_lib.fp8bs_grouped_gemm_bf16w(qa, sa, seg, w, qw=qw, sw=sw, row_token=rt_d)
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))
    has = torch.from_numpy(np.asarray(counts) > 0).cuda()
    assert torch.equal(qw[has], qw_ref[has]) and torch.equal(sw[has], sw_ref[has])
    # the bench step's mode: codes stored only for experts with several tiles
    multi = torch.from_numpy(np.diff(off) > 128).cuda()
    qw.zero_()
    sw.zero_()
    c.zero_()
    c = gpu_lib.fp8bs_grouped_gemm_bf16w(qa, sa, seg, w, c=c, qw=qw, sw=sw, row_token=rt_d, keep_codes=False)
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))
    assert torch.equal(qw[multi], qw_ref[multi]) and torch.equal(sw[multi], sw_ref[multi])
    assert not bool(qw[~multi].any()) and not bool(sw[~multi].any())
    del w, qw_ref, qw
