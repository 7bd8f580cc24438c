"""GPU parity of the quantization kernels: codes and scales bit-exact vs the oracle.

Covers every configuration's operands at full size (sampled where the oracle
would be slow: tiles are independent, so sampled rows / channels / experts are
checked whole), ragged and minimal shapes, strided buffers, all-zero tiles,
signed zeros, tiny (subnormal-scale) and huge magnitudes, exact E4M3 ties, and
every finite bf16 value.
"""

import numpy as np
import pytest
import torch

from oracle import bf16_to_f32, quantize_act_1x128, quantize_act_1x128_t, quantize_w_128x128
from tests.gpu_util import to_dev_bf16
from workloads import (config_by_name, f32_to_bf16_bits, gemm_inputs, grouped_inputs_host,
                       wgrad_inputs)

pytestmark = pytest.mark.gpu


def _act(lib, bits, transpose=0):
    q, s = lib.fp8bs_quantize_act_1x128(to_dev_bf16(bits), transpose=transpose)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def _assert_same(label, q, s, q_ref, s_ref):
    assert q.shape == q_ref.shape and s.shape == s_ref.shape, label
    if not np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)):
        bad = np.argwhere(s.view(np.uint32) != s_ref.view(np.uint32))
        i = tuple(bad[0])
        raise AssertionError(f"{label}: {len(bad)} scales differ, first at {i}: {s[i]!r} vs {s_ref[i]!r}")
    if not np.array_equal(q, q_ref):
        bad = np.argwhere(q != q_ref)
        i = tuple(bad[0])
        raise AssertionError(f"{label}: {len(bad)} codes differ, first at {i}: {q[i]:#x} vs {q_ref[i]:#x}")


def _edge_matrix(rng, rows, cols):
    """bf16 rows exercising zeros, -0, tiny, huge, ties and mixed magnitudes."""
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp(rng.uniform(-30, 30, size=(rows, 1))).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    tiles = bits.reshape(rows, cols // 128, 128)
    nt = tiles.shape[1]
    if rows > 0:
        tiles[0, 0, :] = 0                                    # all +0
    if rows > 1:
        tiles[1, 0, :] = 0x8000                               # all -0
        tiles[1, 0, 7] = 0                                    # mixed signed zeros
    if rows > 2:
        tiles[2, :, :] = rng.integers(0x0001, 0x0080, size=(nt, 128))      # bf16 subnormals only
    if rows > 3:
        tiles[3, :, :] = rng.integers(0x7E00, 0x7F7F, size=(nt, 128))      # huge, up to bf16 max
    if rows > 4:
        # exact E4M3 ties after scaling: amax 56 -> s = 1/8, x = (odd midpoints) / 8
        t = np.zeros(128, np.float32)
        t[0] = 56.0
        t[1:20] = np.array([2.125, 2.375, -2.125, 1.0625 / 8, 3 * 2.0 ** -13, 2.0 ** -13, -2.0 ** -13,
                            0.1328125, 58.0 / 8, 1.1875, -1.1875, 0.0, -0.0, 7.5 * 2.0 ** -12,
                            2.0 ** -12, 29.0 / 8, 30.0, 54.0, -56.0], np.float32)
        tiles[4, 0, :] = f32_to_bf16_bits(t)
    if rows > 5:
        tiles[5, :, :] = rng.integers(0, 0x7F80, size=(nt, 128)) | (rng.integers(0, 2, (nt, 128)) << 15)
    if rows > 6:
        tiles[6, :, :] = rng.integers(0x0001, 0x0400, size=(nt, 128))      # tiny normals + subnormals
    return tiles.reshape(rows, cols)


def test_act_rows_small_and_edges(gpu_lib):
    rng = np.random.default_rng(100)
    for rows, cols in [(1, 128), (3, 256), (7, 384), (130, 512), (257, 1024), (33, 7168)]:
        bits = _edge_matrix(rng, rows, cols)
        q, s = _act(gpu_lib, bits)
        _assert_same(f"act {rows}x{cols}", q, s, *quantize_act_1x128(bits))


def test_act_rows_every_finite_bf16_value(gpu_lib):
    """Every finite bf16 bit pattern appears as x, against many different amax values."""
    rng = np.random.default_rng(101)
    pats = np.arange(0, 0x10000, dtype=np.uint32)
    finite = (pats & 0x7F80) != 0x7F80
    pats = pats[finite].astype(np.uint16)
    rng.shuffle(pats)
    n_tiles = ((pats.size + 126) // 127 + 7) // 8 * 8         # whole 1024-wide rows
    bits = np.zeros((n_tiles, 128), np.uint16)
    flat = np.zeros(n_tiles * 127, np.uint16)
    flat[:pats.size] = pats
    bits[:, 1:] = flat.reshape(n_tiles, 127)
    # element 0 of each tile: a random amax at least as large as every other element
    mags = bits[:, 1:] & 0x7FFF
    top = mags.max(axis=1)
    bump = rng.integers(0, 200, size=n_tiles).astype(np.uint32)
    bits[:, 0] = np.minimum(top.astype(np.uint32) + bump, 0x7F7F).astype(np.uint16)
    bits = bits.reshape(-1, 1024)
    q, s = _act(gpu_lib, bits)
    _assert_same("all bf16 values", q, s, *quantize_act_1x128(bits))


def test_act_rows_strided_buffers(gpu_lib):
    rng = np.random.default_rng(102)
    full = f32_to_bf16_bits(rng.standard_normal((64, 640)).astype(np.float32))
    x = to_dev_bf16(full)[:, 64:576]                       # ldx = 640, cols = 512
    q = torch.full((64, 528), 0xAB, dtype=torch.uint8, device="cuda")[:, :512]   # ldq = 528
    s = torch.empty((64, 4), dtype=torch.float32, device="cuda")
    gpu_lib.fp8bs_quantize_act_1x128(x, q=q, scales=s)
    torch.cuda.synchronize()
    q_ref, s_ref = quantize_act_1x128(np.ascontiguousarray(full[:, 64:576]))
    _assert_same("strided", q.cpu().numpy(), s.cpu().numpy(), q_ref, s_ref)
    base = q.as_strided((64, 528), (528, 1)).cpu().numpy()
    assert np.all(base[:, 512:] == 0xAB)                   # nothing written past cols


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_act_rows_configs(gpu_lib, name):
    bits = gemm_inputs(name)["a"]
    q, s = _act(gpu_lib, bits)
    if bits.shape[0] > 1024:                               # tiles are independent: check sampled rows
        rows = np.random.default_rng(0).choice(bits.shape[0], 256, replace=False)
        rows.sort()
        _assert_same(name, q[rows], s[rows], *quantize_act_1x128(bits[rows]))
    else:
        _assert_same(name, q, s, *quantize_act_1x128(bits))


def test_act_rows_moe_padded_input(gpu_lib):
    cfg = config_by_name("c4")
    g = grouped_inputs_host(cfg, with_weights=False)
    bits, off, counts = g["x"], g["offsets"], g["counts"]
    q, s = _act(gpu_lib, bits)
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([rng.choice(bits.shape[0], 512, replace=False),
                                     off[:-1] + counts, off[1:] - 1]))   # includes padding rows
    rows = rows[rows < bits.shape[0]]
    _assert_same("c4 X", q[rows], s[rows], *quantize_act_1x128(bits[rows]))
    pad = np.zeros(bits.shape[0], bool)
    for e in range(len(counts)):
        pad[off[e] + counts[e]:off[e + 1]] = True
    assert np.all(q[pad] == 0) and np.all(s[pad] == 0)


def test_act_routed_rows_small_and_edges(gpu_lib):
    """Only the rows with a row-map entry >= 0 are coded, bit-exactly as the
    plain call codes them (edge rows included); the other rows keep what the
    output buffers held."""
    rng = np.random.default_rng(77)
    bits = _edge_matrix(rng, 37, 384)
    rt = np.where(rng.random(37) < 0.6, np.arange(37), -1).astype(np.int32)
    rt[:7] = np.arange(7)                                         # every edge row is coded
    rt[-1] = -1
    q = torch.full((37, 384), 0x5A, dtype=torch.uint8, device="cuda")
    s = torch.full((37, 3), -2.0, dtype=torch.float32, device="cuda")
    gpu_lib.fp8bs_quantize_act_1x128_routed(to_dev_bf16(bits), torch.from_numpy(rt).cuda(), q=q, scales=s)
    torch.cuda.synchronize()
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    live = rt >= 0
    _assert_same("routed rows", qh[live], sh[live], *quantize_act_1x128(bits[live]))
    assert np.all(qh[~live] == 0x5A) and np.all(sh[~live] == -2.0)
    # strided input and codes (ldx = 512, ldq = 416): the same bits, the gaps untouched
    xw = torch.zeros((37, 512), dtype=torch.bfloat16, device="cuda")
    xw[:, :384] = to_dev_bf16(bits)
    qw_ = torch.full((37, 416), 0x33, dtype=torch.uint8, device="cuda")
    s2 = torch.full((37, 3), -2.0, dtype=torch.float32, device="cuda")
    gpu_lib.fp8bs_quantize_act_1x128_routed(xw[:, :384], torch.from_numpy(rt).cuda(), q=qw_[:, :384], scales=s2)
    torch.cuda.synchronize()
    q2 = qw_.cpu().numpy()
    assert np.array_equal(q2[live, :384], qh[live]) and np.array_equal(s2.cpu().numpy(), sh)
    assert np.all(q2[~live] == 0x33) and np.all(q2[:, 384:] == 0x33)


def test_act_routed_rows_c4(gpu_lib):
    """c4's padded expert-major X with the routing's row map: the routed rows
    equal the plain call's codes and scales, the padding rows are untouched."""
    cfg = config_by_name("c4")
    g = grouped_inputs_host(cfg, with_weights=False)
    bits, off, counts = g["x"], g["offsets"], g["counts"]
    rt = np.full(bits.shape[0], -1, np.int32)
    for e, cnt in enumerate(counts):
        rt[off[e]:off[e] + cnt] = np.arange(cnt, dtype=np.int32)
    x = to_dev_bf16(bits)
    q_ref, s_ref = gpu_lib.fp8bs_quantize_act_1x128(x)
    q = torch.full_like(q_ref, 0xA5)
    s = torch.full_like(s_ref, 3.0)
    gpu_lib.fp8bs_quantize_act_1x128_routed(x, torch.from_numpy(rt).cuda(), q=q, scales=s)
    live = torch.from_numpy(rt >= 0).cuda()
    assert torch.equal(q[live], q_ref[live]) and torch.equal(s[live].view(torch.int32), s_ref[live].view(torch.int32))
    assert bool((q[~live] == 0xA5).all()) and bool((s[~live] == 3.0).all())


def test_act_transposed_small_and_ragged(gpu_lib):
    rng = np.random.default_rng(103)
    for t, c in [(128, 8), (128, 72), (256, 200), (384, 64), (1024, 520)]:
        padded = ((c + 127) // 128) * 128
        bits = np.ascontiguousarray(_edge_matrix(rng, t, padded)[:, :c])
        q, s = _act(gpu_lib, bits, transpose=1)
        q_ref, s_ref = quantize_act_1x128_t(bits)
        _assert_same(f"transposed {t}x{c}", q, s, q_ref, s_ref)
        q2, s2 = _act(gpu_lib, np.ascontiguousarray(bits.T), transpose=0)
        assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))


def test_act_transposed_c5(gpu_lib):
    d = wgrad_inputs("c5")
    rng = np.random.default_rng(2)
    for key in ("dy", "x"):
        bits = d[key]
        q, s = _act(gpu_lib, bits, transpose=1)
        cols = np.sort(rng.choice(bits.shape[1], 96, replace=False))
        q_ref, s_ref = quantize_act_1x128_t(np.ascontiguousarray(bits[:, cols]))
        _assert_same(f"c5 {key}^T", q[cols], s[cols], q_ref, s_ref)


def _dual(lib, bits):
    q, s, qt, st = lib.fp8bs_quantize_act_1x128_dual(to_dev_bf16(bits))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy(), qt.cpu().numpy(), st.cpu().numpy()


def test_act_dual_small_and_edges(gpu_lib):
    rng = np.random.default_rng(106)
    for t, c in [(128, 128), (384, 256), (256, 1024), (640, 384), (128, 7168)]:
        bits = _edge_matrix(rng, t, c)
        # an edge column too: all -0 in one 128-token group, subnormals in another
        bits[:128, 5] = 0x8000
        if t > 128:
            bits[128:256, 9] = rng.integers(0x0001, 0x0080, size=128)
        q, s, qt, st = _dual(gpu_lib, bits)
        _assert_same(f"dual rows {t}x{c}", q, s, *quantize_act_1x128(bits))
        _assert_same(f"dual transposed {t}x{c}", qt, st, *quantize_act_1x128_t(bits))


@pytest.mark.parametrize("name,key", [("c2", "a"), ("c2", "dy"), ("c5", "dy"), ("c3", "dy")])
def test_act_dual_configs(gpu_lib, name, key):
    from workloads import layer_inputs

    # c3's dY (4096 x 32768, 268 MB) is above the streaming threshold: non-temporal loads
    bits = (layer_inputs(name) if name in ("c2", "c3") else wgrad_inputs(name))[key]
    q, s, qt, st = _dual(gpu_lib, bits)
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(bits.shape[0], 192, replace=False))
    _assert_same(f"{name} {key} dual rows", q[rows], s[rows], *quantize_act_1x128(bits[rows]))
    cols = np.sort(rng.choice(bits.shape[1], 64, replace=False))
    q_ref, s_ref = quantize_act_1x128_t(np.ascontiguousarray(bits[:, cols]))
    _assert_same(f"{name} {key} dual transposed", qt[cols], st[cols], q_ref, s_ref)
    # the two orientations equal the single-orientation entry point bit for bit
    q1, s1 = _act(gpu_lib, bits, transpose=0)
    q2, s2 = _act(gpu_lib, bits, transpose=1)
    assert np.array_equal(q, q1) and np.array_equal(s.view(np.uint32), s1.view(np.uint32))
    assert np.array_equal(qt, q2) and np.array_equal(st.view(np.uint32), s2.view(np.uint32))


def test_act_dual_strided_buffers(gpu_lib):
    rng = np.random.default_rng(107)
    full = f32_to_bf16_bits(rng.standard_normal((384, 520)).astype(np.float32))
    x = to_dev_bf16(full)[:, 8:520]                                   # ldx = 520, cols = 512
    q = torch.full((384, 528), 0xAB, dtype=torch.uint8, device="cuda")[:, :512]
    qt = torch.full((512, 400), 0xCD, dtype=torch.uint8, device="cuda")[:, :384]
    s = torch.empty((384, 4), dtype=torch.float32, device="cuda")
    st = torch.empty((512, 3), dtype=torch.float32, device="cuda")
    gpu_lib.fp8bs_quantize_act_1x128_dual(x, q=q, scales=s, qt=qt, scales_t=st)
    torch.cuda.synchronize()
    sub = np.ascontiguousarray(full[:, 8:520])
    _assert_same("dual strided rows", q.cpu().numpy(), s.cpu().numpy(), *quantize_act_1x128(sub))
    _assert_same("dual strided transposed", qt.cpu().numpy(), st.cpu().numpy(), *quantize_act_1x128_t(sub))
    assert np.all(q.as_strided((384, 528), (528, 1)).cpu().numpy()[:, 512:] == 0xAB)
    assert np.all(qt.as_strided((512, 400), (400, 1)).cpu().numpy()[:, 384:] == 0xCD)


def test_weight_blocks_small_and_edges(gpu_lib):
    rng = np.random.default_rng(104)
    for n, k in [(128, 128), (256, 384), (384, 1024)]:
        bits = _edge_matrix(rng, n, k)
        # one block made entirely of -0 and one entirely of subnormals
        bits[128 * (n // 128 - 1):, :128] = 0x8000
        q, s = gpu_lib.fp8bs_quantize_w_128x128(to_dev_bf16(bits))
        torch.cuda.synchronize()
        _assert_same(f"w {n}x{k}", q.cpu().numpy(), s.cpu().numpy(), *quantize_w_128x128(bits))


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_weight_blocks_configs(gpu_lib, name):
    bits = gemm_inputs(name)["b"]
    q, s = gpu_lib.fp8bs_quantize_w_128x128(to_dev_bf16(bits))
    torch.cuda.synchronize()
    _assert_same(name, q.cpu().numpy(), s.cpu().numpy(), *quantize_w_128x128(bits))


def test_weight_blocks_stacked_experts(gpu_lib):
    rng = np.random.default_rng(105)
    w = f32_to_bf16_bits((rng.standard_normal((5, 256, 384)) * 0.02).astype(np.float32))
    q, s = gpu_lib.fp8bs_quantize_w_128x128(to_dev_bf16(w))
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    assert q.shape == (5, 256, 384) and s.shape == (5, 2, 3)
    for e in range(5):
        _assert_same(f"expert {e}", q[e], s[e], *quantize_w_128x128(w[e]))


def test_determinism(gpu_lib):
    bits = gemm_inputs("c1")["a"]
    x = to_dev_bf16(bits)
    q1, s1 = gpu_lib.fp8bs_quantize_act_1x128(x)
    q2, s2 = gpu_lib.fp8bs_quantize_act_1x128(x)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    assert np.all(np.isfinite(bf16_to_f32(bits)))
