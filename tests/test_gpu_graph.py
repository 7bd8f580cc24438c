"""HIP-graph capture of a whole training pass of a linear layer.

The library's calls are plain kernel launches on the caller's stream (no
memset, no host synchronisation; the one allocation, a split contraction's
workspace, is stream-ordered and recorded by the capture), so a
captured pass must replay to exactly the eager result.  The graph is replayed several times with
unrelated eager work and synchronisations between the replays; every replay
is compared bit for bit with the eager launches, and the eager result itself
is checked against the oracle.
"""

import numpy as np
import pytest
import torch

from oracle import gemm_fprop, quantize_act_1x128, quantize_w_128x128
from tests.gpu_util import assert_gemm_parity, bf16_values_host, magnitude_codes, to_dev_bf16
from workloads import gemm_inputs, layer_inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.uint8) if t.element_size() == 1 else t.view(
        torch.int16 if t.element_size() == 2 else torch.int32)


def test_layer_pass_graph_replays_match_eager(gpu_lib):
    d = layer_inputs("c1")
    x, w, dy = to_dev_bf16(d["a"]), to_dev_bf16(d["b"]), to_dev_bf16(d["dy"])
    m, k = x.shape
    n = w.shape[0]
    u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16
    e = lambda *s, dt: torch.empty(s, dtype=dt, device="cuda")  # noqa: E731
    qx, sx, qw, sw = e(m, k, dt=u8), e(m, k // 128, dt=f32), e(n, k, dt=u8), e(n // 128, k // 128, dt=f32)
    y, qdy, sdy, dx = e(m, n, dt=bf16), e(m, n, dt=u8), e(m, n // 128, dt=f32), e(m, k, dt=bf16)
    qdyt, sdyt, qxt, sxt = e(n, m, dt=u8), e(n, m // 128, dt=f32), e(k, m, dt=u8), e(k, m // 128, dt=f32)
    dw = e(n, k, dt=f32)
    outs = [qx, sx, qw, sw, y, qdy, sdy, dx, qdyt, sdyt, qxt, sxt, dw]

    def layer_pass():
        gpu_lib.fp8bs_quantize_act_1x128(x, q=qx, scales=sx)
        gpu_lib.fp8bs_quantize_w_128x128(w, q=qw, scales=sw)
        gpu_lib.fp8bs_gemm(qx, sx, qw, sw, c=y)
        gpu_lib.fp8bs_quantize_act_1x128(dy, q=qdy, scales=sdy)
        gpu_lib.fp8bs_gemm(qdy, sdy, qw, sw, b_layout=1, c=dx)
        gpu_lib.fp8bs_quantize_act_1x128(dy, transpose=1, q=qdyt, scales=sdyt)
        gpu_lib.fp8bs_quantize_act_1x128(x, transpose=1, q=qxt, scales=sxt)
        gpu_lib.fp8bs_gemm_wgrad(qdyt, sdyt, qxt, sxt, c=dw)

    layer_pass()
    torch.cuda.synchronize()
    ref = [_bits(t).clone() for t in outs]

    # the eager pass is right to begin with (forward output against the oracle)
    oqa, osa = quantize_act_1x128(d["a"])
    oqb, osb = quantize_w_128x128(d["b"])
    c64 = gemm_fprop(oqa, osa, oqb, osb)
    mag = gemm_fprop(magnitude_codes(oqa), osa, magnitude_codes(oqb), osb)
    assert_gemm_parity(bf16_values_host(y), c64, mag, label="graph test eager forward")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            layer_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    other = to_dev_bf16(gemm_inputs("c1", seed=77)["a"])
    for rep in range(4):
        for t in outs:
            t.view(torch.uint8).fill_(0xA5)
        # unrelated eager library work between replays
        gpu_lib.fp8bs_quantize_act_1x128(other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(_bits(t), r), f"replay {rep}: output {i} differs from the eager pass"
    print(f"[graph] {len(outs)} outputs bit-identical to eager on 4 replays", flush=True)
    assert np.isfinite(bf16_values_host(y)).all()


@pytest.mark.parametrize("mode", ["two_calls", "fused", "fused_workspace"])
def test_moe_forward_graph_replays_match_eager(gpu_lib, mode):
    """Route -> dispatch -> grouped GEMM over the row capacity -> combine, captured once.

    No call reads a size back to the host, so the whole MoE forward is one graph.
    The expert weights are quantized by their own call, or (fused) inside the
    grouped GEMM from bf16 with the codes stored (two launches), or with codes
    stored only for the experts whose other tiles read them back (qw/sw as the
    call's workspace, poisoned before every replay like the outputs).  The eager
    layout is checked against the oracle; replays with poisoned outputs and
    unrelated eager work in between must reproduce the eager bits (rows past
    the padded total are not defined outputs and are left out)."""
    from oracle.moe import moe_route
    from workloads import moe_dispatch_inputs, normal_bf16

    cfg = dict(tokens=300, topk=8, experts=16, zipf_s=1.1, seed=31, K=256)
    d = moe_dispatch_inputs(cfg)
    n = 256
    w = to_dev_bf16(normal_bf16(np.random.default_rng(32), (16, n, 256), 0.02))
    ids, gates, x = (torch.from_numpy(d["ids"]).cuda(), torch.from_numpy(d["gates"]).cuda(),
                     to_dev_bf16(d["x"]))
    cap = gpu_lib.fp8bs_moe_max_rows(300, 8, 16)
    i32, u8, f32, bf16 = torch.int32, torch.uint8, torch.float32, torch.bfloat16
    e = lambda *s, dt: torch.empty(s, dtype=dt, device="cuda")  # noqa: E731
    seg, slot, tok = e(17, dt=i32), e(300, 8, dt=i32), e(cap, dt=i32)
    q, s = e(cap, 256, dt=u8), e(cap, 2, dt=f32)
    qw, sw = e(16, n, 256, dt=u8), e(16, n // 128, 2, dt=f32)
    y, out = e(cap, n, dt=bf16), e(300, n, dt=bf16)

    def moe_pass():
        gpu_lib.fp8bs_moe_route(ids, 16, rows_cap=cap, seg_offsets=seg, slot_rows=slot, row_token=tok)
        gpu_lib.fp8bs_moe_permute_quantize(x, slot, seg, tok, q=q, scales=s)
        if mode != "two_calls":
            gpu_lib.fp8bs_grouped_gemm_bf16w(q, s, seg, w, c=y, qw=qw, sw=sw, row_token=tok,
                                             keep_codes=mode == "fused")
        else:
            gpu_lib.fp8bs_quantize_w_128x128(w, q=qw, scales=sw)
            gpu_lib.fp8bs_grouped_gemm(q, s, seg, qw, sw, c=y, row_token=tok)
        gpu_lib.fp8bs_moe_combine(y, slot, gates, out=out)

    moe_pass()
    torch.cuda.synchronize()
    r = moe_route(d["ids"], 16)
    total = int(r["seg_offsets"][-1])
    assert np.array_equal(seg.cpu().numpy(), r["seg_offsets"]) and np.array_equal(tok.cpu().numpy(), r["row_token"])
    # the fused call stores the weight codes of experts that have rows only, or
    # (workspace) of those with more than one 128-row tile
    rows_e = np.diff(r["seg_offsets"])
    used = {"two_calls": np.ones(16, bool), "fused": rows_e > 0, "fused_workspace": rows_e > 128}[mode]
    assert mode != "fused_workspace" or 0 < int(used.sum()) < 16, "the routing must mix one- and multi-tile experts"
    used_e = [int(e) for e in np.nonzero(used)[0]]
    outs = [seg, slot, tok, q[:total], s[:total], *[qw[e] for e in used_e], *[sw[e] for e in used_e],
            y[:total], out]
    ref = [_bits(t).clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            moe_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    other = to_dev_bf16(gemm_inputs("c1", seed=78)["a"])
    for rep in range(4):
        for t in (seg, slot, tok, q, s, qw, sw, y, out):
            t.view(torch.uint8).fill_(0x5A)
        gpu_lib.fp8bs_quantize_act_1x128(other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, rb) in enumerate(zip(outs, ref)):
            assert torch.equal(_bits(t), rb), f"replay {rep}: MoE output {i} differs from the eager pass"


def test_split_contraction_dgrad_graph_replays_match_eager(gpu_lib):
    """The split-contraction dgrad (few output tiles, long contraction) takes its
    FP32 partials from a stream-ordered allocation; captured in a graph, its
    replays reproduce the eager bits."""
    rng = np.random.default_rng(251)
    mo, ko, kc = 300, 512, 4096
    qd = torch.from_numpy(rng.integers(0, 0x7E, (mo, kc), dtype=np.uint8)).cuda()
    sd = torch.from_numpy(rng.uniform(0.5, 2.0, (mo, kc // 128)).astype(np.float32)).cuda()
    qw = torch.from_numpy(rng.integers(0, 0x7E, (kc, ko), dtype=np.uint8)).cuda()
    sw = torch.from_numpy(rng.uniform(0.5, 2.0, (kc // 128, ko // 128)).astype(np.float32)).cuda()
    out = torch.empty((mo, ko), dtype=torch.bfloat16, device="cuda")
    gpu_lib.fp8bs_gemm(qd, sd, qw, sw, b_layout=1, c=out)
    torch.cuda.synchronize()
    ref = _bits(out).clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            gpu_lib.fp8bs_gemm(qd, sd, qw, sw, b_layout=1, c=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        out.view(torch.int16).fill_(-1)
        gpu_lib.fp8bs_gemm(qd, sd, qw, sw, b_layout=1)      # unrelated eager work of the same kind
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), ref), f"replay {rep} differs from the eager result"


def test_split_forward_and_wgrad_graph_replays_match_eager(gpu_lib):
    """The forward and the weight gradient split their contraction the same way
    (a stream-ordered workspace for the FP32 partials; the weight gradient's
    summing kernel adds into C when accumulating).  Captured together, with the
    weight gradient accumulating into a buffer reset before every replay, the
    replays reproduce the eager bits."""
    rng = np.random.default_rng(252)
    m, n, k = 1000, 256, 8192                          # forward: 8 tiles, split 4
    mw, nw, t = 512, 2048, 4096                        # wgrad: 32 tiles, split 2
    dev = lambda a: torch.from_numpy(a).cuda()        # noqa: E731
    qa = dev(rng.integers(0, 0x7E, (m, k), dtype=np.uint8))
    sa = dev(rng.uniform(0.5, 2.0, (m, k // 128)).astype(np.float32))
    qb = dev(rng.integers(0, 0x7E, (n, k), dtype=np.uint8))
    sb = dev(rng.uniform(0.5, 2.0, (n // 128, k // 128)).astype(np.float32))
    qg = dev(rng.integers(0, 0x7E, (mw, t), dtype=np.uint8))
    sg = dev(rng.uniform(0.5, 2.0, (mw, t // 128)).astype(np.float32))
    qx = dev(rng.integers(0, 0x7E, (nw, t), dtype=np.uint8))
    sx = dev(rng.uniform(0.5, 2.0, (nw, t // 128)).astype(np.float32))
    base = dev(rng.standard_normal((mw, nw)).astype(np.float32))
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    dw = base.clone()

    def calls():
        gpu_lib.fp8bs_gemm(qa, sa, qb, sb, c=y)
        gpu_lib.fp8bs_gemm_wgrad(qg, sg, qx, sx, c=dw, accumulate=1)

    calls()
    torch.cuda.synchronize()
    ref_y, ref_dw = _bits(y).clone(), _bits(dw).clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        y.view(torch.int16).fill_(-1)
        dw.copy_(base)
        gpu_lib.fp8bs_gemm_wgrad(qg, sg, qx, sx)          # unrelated eager work of the same kind
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), ref_y), f"replay {rep}: forward differs from the eager result"
        assert torch.equal(_bits(dw), ref_dw), f"replay {rep}: weight gradient differs from the eager result"
