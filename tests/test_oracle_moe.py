"""Pins of the oracle's MoE dispatch (routing layout, permute + quantize) and combine.

Top-k routing to routed experts (deepseek.csdn.net page, section 一(二)), the
all-to-all dispatch before and combine after the expert MLP (qqstock.cn page,
section "DualPipe 流水線并行"), FP8 / BF16 payloads (deepseek.csdn.net page,
section 二(四)).  Pins that do not come from the oracle's own code:
  * the hand-worked layouts and sums in tests/golden/moe_route_worked.txt and
    tests/golden/moe_combine_worked.txt;
  * brute force on small routings: each pair's row from counting earlier pairs
    of its expert one by one, and segment starts from per-expert loops;
  * the padded-row bound is reached by a routing built to reach it, and never
    exceeded;
  * dispatch commutes with the (already pinned) tile quantizer: quantizing the
    token rows first and moving whole code rows gives the same payload;
  * combine with one-hot gates moves bf16 rows exactly; dispatching bf16 rows
    and combining with gates 1/k gives back the token rows bit for bit; the
    combined value matches an exact-rational sum rounded to the nearest bf16
    by an independent search.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16_to_f32, quantize_act_1x128
from oracle.moe import moe_combine, moe_combine_exact, moe_max_rows, moe_permute_quantize, moe_route
from workloads import f32_to_bf16_bits, moe_dispatch_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    fields = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            fields[key] = rest
    return fields


def _matrix(text, dtype):
    return np.array([[float(v) for v in row.split()] for row in text.split("/")]).astype(dtype)


def test_golden_route_layout():
    f = _read_golden("moe_route_worked.txt")
    ids = _matrix(f["ids"], np.int64)
    r = moe_route(ids, int(f["experts"]))
    assert np.array_equal(r["counts"], np.array(f["counts"].split(), dtype=np.int64))
    assert np.array_equal(r["seg_offsets"], np.array(f["seg_offsets"].split(), dtype=np.int64))
    assert np.array_equal(r["slot_rows"], _matrix(f["slot_rows"], np.int64))
    cap = int(f["rows_cap"])
    assert moe_max_rows(ids.shape[0], ids.shape[1], int(f["experts"])) == cap
    want = np.full(cap, -1, dtype=np.int64)
    for item in f["row_token"].split():
        row, tok = item.split(":")
        want[int(row)] = int(tok)
    assert np.array_equal(r["row_token"], want)


def test_golden_combine_sums_and_ties():
    f = _read_golden("moe_combine_worked.txt")
    y = f32_to_bf16_bits(_matrix(f["y"], np.float32))
    rows = _matrix(f["slot_rows"], np.int64)
    g = _matrix(f["gates"], np.float32)
    out = bf16_to_f32(moe_combine(y, rows, g))
    assert np.array_equal(out, _matrix(f["out"], np.float32))


def _brute_route(ids, num_e):
    """Row of every pair by counting, one pair at a time (no sort, no cumsum)."""
    t, k = ids.shape
    pairs = [(tt, jj) for tt in range(t) for jj in range(k)]
    count = [0] * num_e
    for tt, jj in pairs:
        if 0 <= ids[tt, jj] < num_e:
            count[ids[tt, jj]] += 1
    start = [0] * (num_e + 1)
    for e in range(num_e):
        blocks = 0
        while blocks * 128 < count[e]:
            blocks += 1
        start[e + 1] = start[e] + 128 * blocks
    rows = np.full((t, k), -1, dtype=np.int64)
    for i, (tt, jj) in enumerate(pairs):
        e = ids[tt, jj]
        if not 0 <= e < num_e:
            continue
        earlier = sum(1 for (t2, j2) in pairs[:i] if ids[t2, j2] == e)
        rows[tt, jj] = start[e] + earlier
    return np.array(start, dtype=np.int64), rows


@pytest.mark.parametrize("t,k,e,seed", [(1, 1, 1, 0), (37, 3, 5, 1), (300, 2, 3, 2), (64, 8, 16, 3),
                                        (90, 4, 40, 4)])
def test_route_against_brute_force(t, k, e, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, e + 1, size=(t, k))       # includes dropped ids -1 and e
    r = moe_route(ids, e)
    start, rows = _brute_route(ids, e)
    assert np.array_equal(r["seg_offsets"], start)
    assert np.array_equal(r["slot_rows"], rows)
    # row_token is the inverse map; every other row of the capacity is -1
    tok = r["row_token"]
    live = rows >= 0
    assert np.array_equal(tok[rows[live]], np.nonzero(live)[0])
    assert np.count_nonzero(tok >= 0) == np.count_nonzero(live)
    assert start[-1] <= moe_max_rows(t, k, e) == tok.shape[0]


def test_route_bound_reached_and_top_k_order():
    # counts 1, 1, 1, 997 -> 1 + 1 + 1 + 8 blocks = 11 = (1000 + 127 * 4) // 128
    ids = np.concatenate([[0, 1, 2], np.full(997, 3)]).reshape(1000, 1)
    r = moe_route(ids, 4)
    assert r["seg_offsets"][-1] == moe_max_rows(1000, 1, 4) == 11 * 128
    # a single expert with a multiple of 128 pairs needs no padding at all
    r = moe_route(np.zeros((256, 1), dtype=np.int64), 1)
    assert r["seg_offsets"].tolist() == [0, 256] and np.array_equal(r["row_token"][:256], np.arange(256))
    # more experts than pairs: the bound counts only experts that can be busy
    assert moe_max_rows(2, 1, 1000) == (2 + 2 * 127) // 128 * 128


def test_route_of_the_moe_workload_is_stable_and_sorted():
    d = moe_dispatch_inputs({"tokens": 600, "topk": 8, "experts": 32, "zipf_s": 1.1, "seed": 9, "K": 128})
    r = moe_route(d["ids"], 32)
    seg, tok = r["seg_offsets"], r["row_token"]
    for e in range(32):
        real = tok[seg[e]:seg[e + 1]]
        n = int(r["counts"][e])
        assert np.all(real[:n] >= 0) and np.all(real[n:] == -1)
        assert np.all(np.diff(real[:n]) > 0)              # tokens ascending (distinct experts per token)
        assert np.all(np.any(d["ids"][real[:n]] == e, axis=1))   # each row's token chose e


def test_permute_quantize_commutes_with_tile_quantizer():
    rng = np.random.default_rng(5)
    t, k, e, h = 50, 3, 4, 384
    x = f32_to_bf16_bits(rng.standard_normal((t, h)).astype(np.float32) * np.float32(3.0))
    x[7, 128:256] = 0                                      # an all-zero tile
    ids = rng.integers(0, e, size=(t, k))
    r = moe_route(ids, e)
    total = int(r["seg_offsets"][-1])
    q, s = moe_permute_quantize(x, r["row_token"], total)
    qx, sx = quantize_act_1x128(x)                         # token order, then move whole rows
    for tt in range(t):
        for jj in range(k):
            row = r["slot_rows"][tt, jj]
            assert np.array_equal(q[row], qx[tt]) and np.array_equal(s[row], sx[tt])
    pad = r["row_token"][:total] < 0
    assert np.all(q[pad] == 0) and np.all(s[pad] == 0) and np.count_nonzero(pad) == total - t * k


def test_combine_one_hot_moves_rows_exactly():
    rng = np.random.default_rng(6)
    y = f32_to_bf16_bits(rng.standard_normal((40, 256)).astype(np.float32) * np.float32(1e3))
    rows = rng.integers(0, 40, size=(12, 4))
    rows[3, 2] = -1
    g = np.zeros((12, 4), np.float32)
    pick = rng.integers(0, 4, size=12)
    pick[3] = 0
    g[np.arange(12), pick] = 1.0
    g[3, 2] = 5.0                                          # gate of a dropped pair: ignored
    out = moe_combine(y, rows, g)
    assert np.array_equal(out, y[rows[np.arange(12), pick]])


def test_dispatch_then_combine_with_gates_one_over_k_is_identity():
    d = moe_dispatch_inputs({"tokens": 200, "topk": 8, "experts": 24, "zipf_s": 1.1, "seed": 11, "K": 256})
    r = moe_route(d["ids"], 24)
    tok = r["row_token"]
    y = np.zeros((tok.shape[0], 256), dtype=np.uint16)
    y[tok >= 0] = d["x"][tok[tok >= 0]]                    # expert outputs = dispatched token rows
    g = np.full((200, 8), 1.0 / 8, dtype=np.float32)
    assert np.array_equal(moe_combine(y, r["slot_rows"], g), d["x"])


def _nearest_bf16_exact(v):
    """Nearest bf16 to a Fraction by search over neighbouring bit patterns (ties: even)."""
    f = float(v)
    base = int(f32_to_bf16_bits(np.array([f], np.float32))[0])
    best = None
    for b in range(max(base - 2, 0) if f >= 0 else base - 2, base + 3):
        bits = b & 0xFFFF
        val = Fraction(float(bf16_to_f32(np.array([bits], np.uint16))[0]))
        if (val < 0) != (v < 0) and val != 0:
            continue
        d = abs(val - v)
        if best is None or d < best[0] or (d == best[0] and bits % 2 == 0):
            best = (d, bits)
    return best[1]


def test_combine_matches_exact_rational_sum():
    rng = np.random.default_rng(7)
    y = f32_to_bf16_bits(rng.standard_normal((30, 16)).astype(np.float32))
    rows = rng.integers(-1, 30, size=(10, 8))
    g = rng.uniform(0, 1, size=(10, 8)).astype(np.float32)
    out = moe_combine(y, rows, g)
    exact = moe_combine_exact(y, rows, g)
    yv = bf16_to_f32(y)
    for t in range(10):
        for c in range(16):
            s = sum((Fraction(float(g[t, j])) * Fraction(float(yv[rows[t, j], c])) for j in range(8)
                     if rows[t, j] >= 0), Fraction(0))
            assert Fraction(float(exact[t, c])) == s       # float64 sum of 8 such terms is exact here
            if s != 0:
                assert out[t, c] == _nearest_bf16_exact(s)
