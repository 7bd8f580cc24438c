"""GPU parity of the MoE dispatch (routing layout, permute + quantize), the
grouped GEMM over a row capacity, and the combine, against the oracle.

Bars: the routing layout (segment starts, slot rows, row tokens) and the
dispatch payload (codes, scales, zero padding) are integer / byte work and are
compared bit for bit.  The combine's bf16 output must lie between the bf16
roundings of s - G and s + G, where s is the oracle's exact sum and
G = k * 2^-24 * sum_j |g_j y_j| bounds the FP32 fused multiply-add chain's
error (each of the k steps rounds once, by at most 2^-24 of a partial sum no
larger than sum_j |g_j y_j|); most elements must equal bf16(s) exactly.
Sizes: small cases that span several tiles and ragged tails, empty and
degenerate routings, and the MoE workload's full launch (4096 tokens, top-8 of
256 experts, hidden 7168) with the oracle on sampled tokens and rows.
"""

import numpy as np
import pytest
import torch

from oracle import f64_to_bf16_rne, grouped_gemm, quantize_act_1x128, quantize_w_128x128
from oracle.moe import moe_combine_exact, moe_max_rows, moe_permute_quantize, moe_route
from tests.gpu_util import (assert_gemm_parity, bf16_bits_host, bf16_values_host, magnitude_codes, to_dev,
                            to_dev_bf16)
from workloads import f32_to_bf16_bits, moe_dispatch_inputs, normal_bf16

pytestmark = pytest.mark.gpu


def _route_dev(lib, ids, num_e, cap=None):
    seg, slot, tok = lib.fp8bs_moe_route(to_dev(ids.astype(np.int32)), num_e, rows_cap=cap)
    torch.cuda.synchronize()
    return seg.cpu().numpy().astype(np.int64), slot.cpu().numpy().astype(np.int64), tok.cpu().numpy().astype(np.int64)


def _check_route(lib, ids, num_e, label):
    r = moe_route(ids, num_e)
    seg, slot, tok = _route_dev(lib, ids, num_e)
    print(f"[route] {label}: padded rows {int(r['seg_offsets'][-1])} of capacity {tok.shape[0]}")
    assert np.array_equal(seg, r["seg_offsets"]), label
    assert np.array_equal(slot, r["slot_rows"]), label
    assert np.array_equal(tok, r["row_token"]), label
    return r


@pytest.mark.parametrize("t,k,e,seed", [(1, 1, 1, 0), (37, 3, 5, 1), (300, 8, 256, 2), (2000, 2, 512, 3),
                                        (5, 64, 7, 4), (129, 1, 1, 5)])
def test_route_random_ids_with_dropped_pairs(gpu_lib, t, k, e, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-3, e + 3, size=(t, k))                  # ids outside [0, E) are dropped
    skew = rng.random((t, k)) < 0.5
    ids[skew] = rng.integers(0, max(1, e // 8), size=int(skew.sum()))
    _check_route(gpu_lib, ids, e, f"T={t} k={k} E={e}")


def test_route_empty_and_exact_multiple(gpu_lib):
    # no tokens: every segment empty, no row
    seg, slot, tok = _route_dev(gpu_lib, np.zeros((0, 8), np.int64), 16)
    assert seg.tolist() == [0] * 17 and slot.shape == (0, 8) and tok.shape == (0,)
    # one expert with exactly 256 pairs: no padding; capacity larger than the bound is allowed
    seg, slot, tok = _route_dev(gpu_lib, np.zeros((256, 1), np.int64), 1, cap=512)
    assert seg.tolist() == [0, 256] and np.array_equal(slot[:, 0], np.arange(256))
    assert np.array_equal(tok[:256], np.arange(256)) and np.all(tok[256:] == -1)
    # every id dropped
    seg, slot, tok = _route_dev(gpu_lib, np.full((50, 4), 9), 9)
    assert np.all(seg == 0) and np.all(slot == -1) and np.all(tok == -1)


def test_route_moe_workload(gpu_lib):
    d = moe_dispatch_inputs("c4", hidden=128)
    r = _check_route(gpu_lib, d["ids"], d["experts"], "4096 tokens, top-8 of 256")
    assert int(r["seg_offsets"][-1]) <= moe_max_rows(4096, 8, 256)


def _payload_case(lib, t, k, e, h, seed, tiny=False):
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (t, h), 2.0)
    x[t // 2, :128] = 0                                         # an all-zero tile
    x[t // 3, 128 % h:] = 0x8000                                # negative zeros
    if tiny:
        x[1] = f32_to_bf16_bits(rng.standard_normal(h).astype(np.float32) * np.float32(1e-30))
    ids = rng.integers(0, e, size=(t, k))
    ids[0, 0] = e                                               # a dropped pair
    r = moe_route(ids, e)
    total = int(r["seg_offsets"][-1])
    seg, slot, tok = (to_dev(v.astype(np.int32)) for v in (r["seg_offsets"], r["slot_rows"], r["row_token"]))
    cap = tok.numel()
    q = torch.full((cap, h), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((cap, h // 128), -7.0, dtype=torch.float32, device="cuda")
    lib.fp8bs_moe_permute_quantize(to_dev_bf16(x), slot, seg, tok, q=q, scales=s)
    torch.cuda.synchronize()
    oq, osc = moe_permute_quantize(x, r["row_token"], total)
    gq, gs = q.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(gq[:total], oq), (t, k, e, h)
    assert np.array_equal(gs[:total].view(np.uint32), osc.view(np.uint32)), (t, k, e, h)
    assert np.all(gq[total:] == 0xAB) and np.all(gs[total:] == -7.0)     # past the padded total: untouched
    return x, q, s, r


@pytest.mark.parametrize("t,k,e,h,seed", [(300, 4, 10, 384, 1), (57, 8, 256, 128, 2), (9, 64, 3, 1152, 3),
                                          (130, 1, 1, 2176, 4)])
def test_permute_quantize_small(gpu_lib, t, k, e, h, seed):
    _payload_case(gpu_lib, t, k, e, h, seed, tiny=(seed == 3))


def test_permute_quantize_equals_quantizer_rows(gpu_lib):
    """Row r of the payload is row row_token[r] of the 1x128 quantizer's output, bit for bit."""
    x, q, s, r = _payload_case(gpu_lib, 200, 6, 12, 1024, 7)
    qx, sx = gpu_lib.fp8bs_quantize_act_1x128(to_dev_bf16(x))
    tok = r["row_token"][:int(r["seg_offsets"][-1])]
    real = torch.from_numpy(np.nonzero(tok >= 0)[0]).cuda()
    src = torch.from_numpy(tok[tok >= 0]).cuda()
    assert torch.equal(q[real], qx[src]) and torch.equal(s[real].view(torch.int32), sx[src].view(torch.int32))


def test_permute_quantize_moe_workload_sampled(gpu_lib):
    """Full launch (4096 x 7168 tokens, top-8 of 256): layout in full, payload rows sampled."""
    d = moe_dispatch_inputs("c4")
    ids, x = d["ids"], d["x"]
    seg, slot, tok = gpu_lib.fp8bs_moe_route(to_dev(ids), 256)
    q, s = gpu_lib.fp8bs_moe_permute_quantize(to_dev_bf16(x), slot, seg, tok)
    torch.cuda.synchronize()
    r = moe_route(ids, 256)
    total = int(r["seg_offsets"][-1])
    assert np.array_equal(tok.cpu().numpy(), r["row_token"])
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.choice(total, 96, replace=False), [0, total - 1],
                                     r["seg_offsets"][1:9] - 1]))
    t_of = r["row_token"][rows]
    gathered = np.zeros((rows.size, x.shape[1]), np.uint16)
    gathered[t_of >= 0] = x[t_of[t_of >= 0]]
    oq, osc = quantize_act_1x128(gathered)
    ri = torch.from_numpy(rows).cuda()
    assert np.array_equal(q[ri].cpu().numpy(), oq)
    assert np.array_equal(s[ri].cpu().numpy().view(np.uint32), osc.view(np.uint32))
    print(f"[dispatch] 4096 tokens: {total} padded rows, {int(np.sum(t_of < 0))} padding rows among the sample")


def _check_combine(out_bits, y_bits, slot, g, label, min_exact=0.97):
    exact = moe_combine_exact(y_bits, slot, g)
    yv = (y_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    k = slot.shape[1]
    mag = np.zeros_like(exact)
    for j in range(k):
        live = slot[:, j] >= 0
        mag[live] += np.abs(g[live, j].astype(np.float64))[:, None] * np.abs(yv[slot[live, j]])
    gam = k * 2.0 ** -24 * mag
    as_f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    lo, hi = as_f(f64_to_bf16_rne(exact - gam)), as_f(f64_to_bf16_rne(exact + gam))
    got = as_f(out_bits)
    inside = (got >= lo) & (got <= hi)
    same = float(np.mean(out_bits == f64_to_bf16_rne(exact)))
    print(f"[combine] {label}: equal to bf16(exact) {same:.5f}, inside the bracket {np.mean(inside):.6f}")
    assert np.all(inside), label
    assert same >= min_exact, label


@pytest.mark.parametrize("t,k,n,rows,seed", [(300, 8, 200, 700, 1), (64, 3, 1024, 64, 2), (17, 64, 520, 90, 3),
                                             (1, 1, 8, 1, 4)])
def test_combine_small(gpu_lib, t, k, n, rows, seed):
    rng = np.random.default_rng(seed)
    y = normal_bf16(rng, (rows, n), 3.0)
    slot = rng.integers(0, rows, size=(t, k))
    slot[rng.random((t, k)) < 0.1] = -1                         # dropped pairs
    g = rng.uniform(0.0, 1.0, size=(t, k)).astype(np.float32)
    g[0, 0] = -0.5                                              # gates need not be positive
    out = gpu_lib.fp8bs_moe_combine(to_dev_bf16(y), to_dev(slot.astype(np.int32)), to_dev(g))
    _check_combine(bf16_bits_host(out), y, slot, g, f"T={t} k={k} n={n}")


def test_combine_one_hot_and_round_trip(gpu_lib):
    """One-hot gates move bf16 rows exactly; dispatching rows then combining with gates 1/k returns them."""
    d = moe_dispatch_inputs({"tokens": 300, "topk": 8, "experts": 24, "zipf_s": 1.1, "seed": 11, "K": 512})
    seg, slot, tok = gpu_lib.fp8bs_moe_route(to_dev(d["ids"]), 24)
    tok_h = tok.cpu().numpy().astype(np.int64)
    y = np.zeros((tok_h.shape[0], 512), np.uint16)
    y[tok_h >= 0] = d["x"][tok_h[tok_h >= 0]]
    yd = to_dev_bf16(y)
    out = gpu_lib.fp8bs_moe_combine(yd, slot, torch.full((300, 8), 0.125, device="cuda"))
    assert np.array_equal(bf16_bits_host(out), d["x"])
    g = np.zeros((300, 8), np.float32)
    g[:, 5] = 1.0
    out = gpu_lib.fp8bs_moe_combine(yd, slot, to_dev(g))
    assert np.array_equal(bf16_bits_host(out), d["x"])


def test_combine_moe_workload_sampled(gpu_lib):
    """Full launch: 4096 tokens x top-8, expert outputs [capacity, 7168] bf16; oracle on sampled tokens."""
    d = moe_dispatch_inputs("c4")
    seg, slot, tok = gpu_lib.fp8bs_moe_route(to_dev(d["ids"]), 256)
    cap = tok.numel()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(44)
    y = torch.randn((cap, 7168), generator=gen, device="cuda").to(torch.bfloat16)
    out = gpu_lib.fp8bs_moe_combine(y, slot, to_dev(d["gates"]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    toks = np.unique(np.concatenate([rng.choice(4096, 48, replace=False), [0, 4095]]))
    slot_h = slot.cpu().numpy().astype(np.int64)[toks]
    need = np.unique(slot_h[slot_h >= 0])
    y_rows = bf16_bits_host(y[torch.from_numpy(need).cuda()])
    remap = np.full(cap, -1, np.int64)
    remap[need] = np.arange(need.size)
    slot_l = np.where(slot_h >= 0, remap[np.maximum(slot_h, 0)], -1)
    _check_combine(bf16_bits_host(out[torch.from_numpy(toks).cuda()]), y_rows, slot_l, d["gates"][toks],
                   "4096 tokens x 7168, sampled tokens")


@pytest.mark.parametrize("n,fused", [(128, False), (256, False), (256, True)])
def test_dispatch_grouped_combine_chain(gpu_lib, n, fused):
    """Route -> payload -> grouped GEMM over the row capacity (with the route's row map) -> combine,
    against the oracle chain.

    The grouped GEMM runs over the capacity (no host read of the padded total):
    its rows past the padded total must stay untouched.  n = 128 runs the
    128 x 128 grouped kernel, n = 256 the 128 x 256 warp-specialized one, and
    fused the call that quantizes the bf16 expert weights itself."""
    cfg = dict(tokens=333, topk=6, experts=9, zipf_s=1.1, seed=21, K=512)
    d = moe_dispatch_inputs(cfg)
    k = 512
    rng = np.random.default_rng(22)
    w = normal_bf16(rng, (9, n, k), 0.02)
    seg, slot, tok = gpu_lib.fp8bs_moe_route(to_dev(d["ids"]), 9)
    q, s = gpu_lib.fp8bs_moe_permute_quantize(to_dev_bf16(d["x"]), slot, seg, tok)
    qw, sw = gpu_lib.fp8bs_quantize_w_128x128(to_dev_bf16(w))
    cap = tok.numel()
    y = torch.full((cap, n), 77.0, dtype=torch.bfloat16, device="cuda")
    if fused:                                  # weights coded inside the grouped GEMM
        gpu_lib.fp8bs_grouped_gemm_bf16w(q, s, seg, to_dev_bf16(w), c=y, row_token=tok)
    else:
        gpu_lib.fp8bs_grouped_gemm(q, s, seg, qw, sw, c=y, row_token=tok)
    out = gpu_lib.fp8bs_moe_combine(y, slot, to_dev(d["gates"]))
    torch.cuda.synchronize()
    r = moe_route(d["ids"], 9)
    off = r["seg_offsets"]
    total = int(off[-1])
    assert total < cap
    oq, osc = moe_permute_quantize(d["x"], r["row_token"], total)
    ws = [quantize_w_128x128(w[e]) for e in range(9)]
    oqb, osb = np.stack([a[0] for a in ws]), np.stack([a[1] for a in ws])
    c64 = grouped_gemm(oq, osc, off, oqb, osb)
    mag = grouped_gemm(magnitude_codes(oq), osc, off, magnitude_codes(oqb), osb)
    got = bf16_values_host(y)
    real = r["row_token"][:total] >= 0
    assert_gemm_parity(got[:total][real], c64[real], mag[real], label="chain: grouped over capacity")
    assert np.all(got[:total][~real] == 0) and np.all(got[total:] == 77.0)
    # the combine of the GPU's expert outputs against the oracle's combine of the same outputs
    _check_combine(bf16_bits_host(out), bf16_bits_host(y), r["slot_rows"], d["gates"], "chain: combine")


def test_route_large_batch_and_most_experts(gpu_lib):
    """16384 tokens x top-8 over 512 experts (131072 pairs: several 1024-pair batches per wave)."""
    d = moe_dispatch_inputs({"tokens": 16384, "topk": 8, "experts": 512, "zipf_s": 0.8, "seed": 41, "K": 128})
    _check_route(gpu_lib, d["ids"], 512, "16384 tokens, top-8 of 512")


def test_combine_token_with_every_slot_dropped_is_zero(gpu_lib):
    rng = np.random.default_rng(51)
    y = normal_bf16(rng, (64, 136), 1.0)
    slot = rng.integers(0, 64, size=(10, 4))
    slot[3] = -1                                               # token 3: no expert row at all
    slot[7, :2] = 1000                                         # rows past the capacity: dropped too
    g = rng.uniform(0.1, 1.0, size=(10, 4)).astype(np.float32)
    out = bf16_bits_host(gpu_lib.fp8bs_moe_combine(to_dev_bf16(y), to_dev(slot.astype(np.int32)), to_dev(g)))
    assert np.all(out[3] == 0)
    ref_slot = np.where(slot >= 64, -1, slot)
    _check_combine(out, y, ref_slot, g, "dropped slots")


def test_dispatch_wide_rows(gpu_lib):
    """hidden 14336 (112 tiles: 14 wave steps per token), top-2 of 3 experts."""
    _payload_case(gpu_lib, 40, 2, 3, 14336, 61)
