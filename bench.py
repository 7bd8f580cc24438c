#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 GEMM path on one MI355X.

Default workload (``--config c4``, the largest configuration): the MoE routed-
expert grouped GEMM of 4096 tokens x top-8 of 256 experts (Zipf 1.1 counts,
each expert's rows padded to a multiple of 128), fused gate+up N = 4096,
K = 7168.  One step runs the configuration's whole FP8 path:
    quantize X (1x128 tiles, the routed rows of the padded expert-major layout)
    quantize every expert's W (128x128 blocks, 256 x 4096 x 7168)
    grouped GEMM C = X W_e^T per expert segment (bf16 out)
``value`` = the grouped GEMM's FLOPs over the routed (real) rows,
2 * 32768 * 4096 * 7168, divided by the step time, in TFLOP/s.  The MoE
routing, dispatch (permute + quantize from token order) and combine around it
are timed on their own and reported under ``moe_kernels`` (not in ``value``).

Other configurations print their own line: ``--config c2|c3`` one FP8
training pass of a linear layer (quantize X, W, dY; forward, dgrad and wgrad
GEMMs), ``--config c5`` the weight gradient over 16384 tokens (both operands
transpose-quantized).

Inputs are resident in HBM before timing; small configurations rotate over
several input copies (>= 512 MB in total) so the 256 MB Infinity Cache cannot
hold them between steps (c4's 15 GB of expert weights need no rotation).  The
timed steps are eager launches on one stream, bracketed by device
synchronizations; ``--graph`` times one captured graph per step instead (each
replay is first checked bit for bit against the eager launches).  Per-kernel
durations come from a second timed region: each call is captured
``--kernel-reps`` times in a row into a graph of its own (rotating over the
input copies) and timed with HIP events on the stream it is launched on.

Each call carries its own roofline bound: the larger of its FLOPs at the FP8
dense peak (5 PFLOP/s) and its algorithmic bytes at the HBM peak (8 TB/s).
``roofline`` is the call with the largest time, ``roofline_gemm`` the GEMM of
the step with the largest time.  ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same workload on the host cores.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-scaled FP8 GEMM TFLOP/s and % of MI355X FP8 dense MFMA peak (1 GPU)"
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the sources behind each kernel family's launches (the kernel file, the device
# helpers, the launch constants): traffic counters taken on other sources are stale
_SHARED = ["fp8_fine_grained_act_amd/csrc/common.h", "fp8_fine_grained_act_amd/csrc/launch.h"]
KERNEL_SOURCES = {
    "gemm": ["fp8_fine_grained_act_amd/csrc/gemm.hip"] + _SHARED,
    "quant": ["fp8_fine_grained_act_amd/csrc/quantize.hip"] + _SHARED,
    "moe": ["fp8_fine_grained_act_amd/csrc/moe.hip"] + _SHARED,
    "requant": ["fp8_fine_grained_act_amd/csrc/requant.hip"] + _SHARED,
}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    # the GPU reaches its steady clock only after ~10 ms of back-to-back work
    # (c2 steps measured 245 -> 223 -> 217 us over three runs of 50): the
    # default warm-up covers that, and the timed steps last ~50 ms
    # (c4's step lasts ~6 ms, so any warm-up settles it; the layer
    # configurations take the longer defaults below when none is given)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--config", default="c4", choices=["c2", "c3", "c4", "c5"])
    p.add_argument("--rotate", type=int, default=0, help="input copies to rotate over (0 = automatic)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="the CPU oracle repeats its sample until this much host time has passed")
    p.add_argument("--kernel-reps", type=int, default=None,
                   help="launches per per-kernel timing graph (default 24; 6 for c4)")
    p.add_argument("--graph", action="store_true",
                   help="time one HIP graph replay per step instead of eager launches")
    p.add_argument("--eager", action="store_true", help="eager launches (the default; kept for old command lines)")
    p.add_argument("--separate-quant", action="store_true",
                   help="quantize each activation orientation with its own call instead of the fused call")
    p.add_argument("--act-cache", action="store_true",
                   help="FP8 activation caching (c2, c3, c5): X is kept as its forward 1x128 tiles and the "
                        "weight gradient's tiles along the tokens are re-tiled from them")
    p.add_argument("--c4-two-calls", action="store_true",
                   help="c4: quantize the expert weights and run the grouped GEMM as two calls instead of the "
                        "grouped GEMM that quantizes its bf16 weights itself")
    p.add_argument("--c4-keep-codes", action="store_true",
                   help="c4: the fused grouped GEMM also stores the FP8 codes and scales of every expert "
                        "(kept for later GEMMs such as a backward's dgrad), not only those its own tiles "
                        "read back")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run plain 512 MiB device-to-device copies (reference for HBM byte counters)")
    a = p.parse_args()
    small = a.config != "c4"
    if a.steps is None:
        a.steps = 200 if small else 20
    if a.warmup is None:
        a.warmup = 50 if small else 5
    if a.kernel_reps is None:
        a.kernel_reps = 24 if small else 6
    return a


def source_hash(kind):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def dev_bf16(bits):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class Call:
    def __init__(self, name, kind, fn, flops=0.0, nbytes=0.0, outs=()):
        self.name, self.kind, self.fn, self.flops, self.nbytes = name, kind, fn, flops, nbytes
        self.outs = list(outs)
        self.times_ms = []


def build_layer_step(lib, cfg_name, rotate, dual=True, act_cache=False):
    """Calls of one training pass of a linear layer (configs c2 / c3 shapes).

    With ``dual`` (default) X and dY are each quantized once into both
    orientations (1x128 tiles along the features for forward / dgrad, along
    the tokens for wgrad); otherwise each orientation is its own call.
    """
    import torch

    from workloads import config_by_name, layer_inputs

    cfg = config_by_name(cfg_name)
    m, n, k = cfg["M"], cfg["N"], cfg["K"]
    d = layer_inputs(cfg)
    x0, w0, dy0 = dev_bf16(d["a"]), dev_bf16(d["b"]), dev_bf16(d["dy"])
    per_set = (x0.numel() + w0.numel() + dy0.numel()) * 2
    if rotate <= 0:
        rotate = max(2, -(-512 * 2 ** 20 // per_set))
    sets = [(x0, w0, dy0)] + [(x0.clone(), w0.clone(), dy0.clone()) for _ in range(rotate - 1)]
    u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16
    e = lambda *s, dt: torch.empty(s, dtype=dt, device="cuda")  # noqa: E731
    qx, sx = e(m, k, dt=u8), e(m, k // 128, dt=f32)
    qw, sw = e(n, k, dt=u8), e(n // 128, k // 128, dt=f32)
    y = e(m, n, dt=bf16)
    qdy, sdy = e(m, n, dt=u8), e(m, n // 128, dt=f32)
    dx = e(m, k, dt=bf16)
    qdyt, sdyt = e(n, m, dt=u8), e(n, m // 128, dt=f32)
    qxt, sxt = e(k, m, dt=u8), e(k, m // 128, dt=f32)
    dw = e(n, k, dt=f32)
    state = {"i": 0}

    def cur():
        return sets[state["i"] % rotate]

    act_bytes = lambda r, c: r * c * 3 + r * c // 128 * 4  # noqa: E731
    # compulsory GEMM bytes: both operands' codes and scales, the output
    wsc = (n // 128) * (k // 128) * 4
    fprop_bytes = m * k + m * (k // 128) * 4 + n * k + wsc + m * n * 2
    dgrad_bytes = m * n + m * (n // 128) * 4 + n * k + wsc + m * k * 2
    wgrad_bytes = (n + k) * m + (n + k) * (m // 128) * 4 + n * k * 4
    dual_bytes = lambda r, c: r * c * 4 + 2 * (r * c // 128) * 4  # noqa: E731
    requant_bytes = lambda r, c: r * c * 2 + 2 * (r * c // 128) * 4  # noqa: E731
    if act_cache:
        calls = [
            Call("quant_act_x", "quant", lambda: lib.fp8bs_quantize_act_1x128(cur()[0], q=qx, scales=sx),
                 nbytes=act_bytes(m, k), outs=(qx, sx)),
            Call("quant_w", "quant", lambda: lib.fp8bs_quantize_w_128x128(cur()[1], q=qw, scales=sw),
                 nbytes=n * k * 3 + (n // 128) * (k // 128) * 4, outs=(qw, sw)),
            Call("gemm_fprop", "gemm", lambda: lib.fp8bs_gemm(qx, sx, qw, sw, c=y), flops=2.0 * m * n * k, nbytes=fprop_bytes,
                 outs=(y,)),
            Call("quant_act_dy_dual", "quant",
                 lambda: lib.fp8bs_quantize_act_1x128_dual(cur()[2], q=qdy, scales=sdy, qt=qdyt, scales_t=sdyt),
                 nbytes=dual_bytes(m, n), outs=(qdy, sdy, qdyt, sdyt)),
            Call("gemm_dgrad", "gemm", lambda: lib.fp8bs_gemm(qdy, sdy, qw, sw, b_layout=1, c=dx),
                 flops=2.0 * m * n * k, nbytes=dgrad_bytes, outs=(dx,)),
            Call("requant_x_t", "requant",
                 lambda: lib.fp8bs_requantize_act_1x128_t(qx, sx, qt=qxt, scales_t=sxt),
                 nbytes=requant_bytes(m, k), outs=(qxt, sxt)),
            Call("gemm_wgrad", "gemm", lambda: lib.fp8bs_gemm_wgrad(qdyt, sdyt, qxt, sxt, c=dw),
                 flops=2.0 * m * n * k, nbytes=wgrad_bytes, outs=(dw,)),
        ]
    elif dual:
        calls = [
            Call("quant_act_x_dual", "quant",
                 lambda: lib.fp8bs_quantize_act_1x128_dual(cur()[0], q=qx, scales=sx, qt=qxt, scales_t=sxt),
                 nbytes=dual_bytes(m, k), outs=(qx, sx, qxt, sxt)),
            Call("quant_w", "quant", lambda: lib.fp8bs_quantize_w_128x128(cur()[1], q=qw, scales=sw),
                 nbytes=n * k * 3 + (n // 128) * (k // 128) * 4, outs=(qw, sw)),
            Call("gemm_fprop", "gemm", lambda: lib.fp8bs_gemm(qx, sx, qw, sw, c=y), flops=2.0 * m * n * k, nbytes=fprop_bytes,
                 outs=(y,)),
            Call("quant_act_dy_dual", "quant",
                 lambda: lib.fp8bs_quantize_act_1x128_dual(cur()[2], q=qdy, scales=sdy, qt=qdyt, scales_t=sdyt),
                 nbytes=dual_bytes(m, n), outs=(qdy, sdy, qdyt, sdyt)),
            Call("gemm_dgrad", "gemm", lambda: lib.fp8bs_gemm(qdy, sdy, qw, sw, b_layout=1, c=dx),
                 flops=2.0 * m * n * k, nbytes=dgrad_bytes, outs=(dx,)),
            Call("gemm_wgrad", "gemm", lambda: lib.fp8bs_gemm_wgrad(qdyt, sdyt, qxt, sxt, c=dw),
                 flops=2.0 * m * n * k, nbytes=wgrad_bytes, outs=(dw,)),
        ]
    else:
        calls = [
            Call("quant_act_x", "quant", lambda: lib.fp8bs_quantize_act_1x128(cur()[0], q=qx, scales=sx),
                 nbytes=act_bytes(m, k), outs=(qx, sx)),
            Call("quant_w", "quant", lambda: lib.fp8bs_quantize_w_128x128(cur()[1], q=qw, scales=sw),
                 nbytes=n * k * 3 + (n // 128) * (k // 128) * 4, outs=(qw, sw)),
            Call("gemm_fprop", "gemm", lambda: lib.fp8bs_gemm(qx, sx, qw, sw, c=y), flops=2.0 * m * n * k, nbytes=fprop_bytes,
                 outs=(y,)),
            Call("quant_act_dy", "quant", lambda: lib.fp8bs_quantize_act_1x128(cur()[2], q=qdy, scales=sdy),
                 nbytes=act_bytes(m, n), outs=(qdy, sdy)),
            Call("gemm_dgrad", "gemm", lambda: lib.fp8bs_gemm(qdy, sdy, qw, sw, b_layout=1, c=dx),
                 flops=2.0 * m * n * k, nbytes=dgrad_bytes, outs=(dx,)),
            Call("quant_act_dy_t", "quant",
                 lambda: lib.fp8bs_quantize_act_1x128(cur()[2], transpose=1, q=qdyt, scales=sdyt),
                 nbytes=act_bytes(m, n), outs=(qdyt, sdyt)),
            Call("quant_act_x_t", "quant",
                 lambda: lib.fp8bs_quantize_act_1x128(cur()[0], transpose=1, q=qxt, scales=sxt),
                 nbytes=act_bytes(m, k), outs=(qxt, sxt)),
            Call("gemm_wgrad", "gemm", lambda: lib.fp8bs_gemm_wgrad(qdyt, sdyt, qxt, sxt, c=dw),
                 flops=2.0 * m * n * k, nbytes=wgrad_bytes, outs=(dw,)),
        ]
    desc = dict(workload=f"{cfg_name}: one FP8 training pass (forward + dgrad + wgrad, all quantization "
                         f"included) of a linear layer, {cfg['desc']}",
                M_tokens=m, N_out=n, K_in=k, input_copies=rotate,
                activation_quantization=("X: forward 1x128 tiles kept as the FP8 cache, weight-gradient tiles "
                                         "re-tiled from it; dY: one call for both orientations") if act_cache
                else "one call per tensor for both orientations" if dual
                else "one call per tensor and orientation")
    return calls, state, desc, dict(d, kind="layer", cfg=cfg), []


def build_grouped_step(lib, rotate, fused=True, keep_codes=False):
    """Calls of configuration c4: the MoE expert grouped GEMM with its quantization.

    The step: quantize X (1x128 tiles over the routed rows of the padded
    expert-major layout; the padding rows, which the grouped GEMM does not read
    through the row map, are not coded) -> quantize every expert's weight (128x128 blocks,
    codes and scales stored) -> grouped GEMM over the padded total.  By
    default the last two are one call, fp8bs_grouped_gemm_bf16w, whose copy
    waves code each weight block where the GEMM reads it; it stores the codes
    of the experts with several 128-row tiles once, for their other tiles to
    read back (keep_codes: those of every expert, for later GEMMs); with
    fused=False they are fp8bs_quantize_w_128x128 and fp8bs_grouped_gemm
    (the same bits).  The MoE routing layout, the
    dispatch payload (permute + 1x128 quantize from token order) and the
    combine (gate-weighted sum of each token's k expert rows, [capacity, 7168]
    bf16 expert outputs drawn once on the device) are returned as extra calls:
    they are timed on their own, outside the step.  No call reads a size back
    to the host.
    """
    import numpy as np
    import torch

    from workloads import (config_by_name, device_expert_weights, grouped_inputs_host, moe_dispatch_inputs)

    cfg = config_by_name("c4")
    host = grouped_inputs_host(cfg, with_weights=False)
    counts, offsets = host["counts"], host["offsets"]
    total = int(offsets[-1])
    k, n, num_e = cfg["K"], cfg["N"], cfg["experts"]
    pairs = int(counts.sum())
    x = dev_bf16(host["x"])
    seg_pad = torch.from_numpy(offsets.astype(np.int32)).cuda()
    # the routing's row map of this layout: each expert's routed rows, then -1 on its padding
    rt_host = np.full(total, -1, np.int32)
    for ex in range(len(counts)):
        rt_host[offsets[ex]:offsets[ex] + counts[ex]] = np.arange(counts[ex], dtype=np.int32)
    row_token = torch.from_numpy(rt_host).cuda()
    w = device_expert_weights(cfg)
    i32, u8, f32, bf16 = torch.int32, torch.uint8, torch.float32, torch.bfloat16
    e = lambda *s, dt: torch.empty(s, dtype=dt, device="cuda")  # noqa: E731
    qx, sx = e(total, k, dt=u8), e(total, k // 128, dt=f32)
    qw, sw = e(num_e, n, k, dt=u8), e(num_e, n // 128, k // 128, dt=f32)
    y = e(total, n, dt=bf16)
    state = {"i": 0}
    kb = k // 128
    # algorithmic bytes: the X quantizer reads and writes the routed rows and reads the row map; the
    # grouped GEMM reads the routed rows of X (the row map clips the padding),
    # the row map, every expert weight once, and writes every padded output row
    x_bytes = pairs * (k * 3 + kb * 4) + total * 4
    w_bytes = num_e * n * k * 3 + num_e * (n // 128) * kb * 4
    gemm_bytes = pairs * (k + kb * 4) + total * 4 + num_e * (n * k + (n // 128) * kb * 4) + total * n * 2
    # fused: the bf16 weights read once, the routed rows of X and the row map
    # read, every padded output row written; with keep_codes also every
    # expert's codes and scales written once (outputs of the call).  Without
    # it the codes stored for the experts' other tiles are the call's own
    # workspace and are not counted.
    fused_bytes = (num_e * n * k * 2 + pairs * (k + kb * 4) + total * 4 + total * n * 2
                   + (num_e * n * k + num_e * (n // 128) * kb * 4 if keep_codes else 0))
    # X: only the routed rows are coded (the grouped GEMM reads no padding row through the row map)
    quant_x = Call("quant_act_x", "quant",
                   lambda: lib.fp8bs_quantize_act_1x128_routed(x, row_token, q=qx, scales=sx),
                   nbytes=x_bytes, outs=(qx, sx))
    if fused:
        calls = [
            quant_x,
            Call("gemm_grouped_bf16w_keep_codes" if keep_codes else "gemm_grouped_bf16w", "gemm",
                 lambda: lib.fp8bs_grouped_gemm_bf16w(qx, sx, seg_pad, w, c=y, qw=qw, sw=sw, row_token=row_token,
                                                      keep_codes=keep_codes),
                 flops=2.0 * pairs * n * k, nbytes=fused_bytes, outs=(y, qw, sw) if keep_codes else (y,)),
        ]
    else:
        calls = [
            quant_x,
            Call("quant_w_experts", "quant", lambda: lib.fp8bs_quantize_w_128x128(w, q=qw, scales=sw),
                 nbytes=w_bytes, outs=(qw, sw)),
            Call("gemm_grouped", "gemm",
                 lambda: lib.fp8bs_grouped_gemm(qx, sx, seg_pad, qw, sw, c=y, row_token=row_token),
                 flops=2.0 * pairs * n * k, nbytes=gemm_bytes, outs=(y,)),
        ]

    # the MoE kernels around the grouped GEMM (timed on their own)
    d = moe_dispatch_inputs(cfg)
    tokens, topk = d["ids"].shape
    cap = lib.fp8bs_moe_max_rows(tokens, topk, num_e)
    xt = dev_bf16(d["x"])
    ids = torch.from_numpy(d["ids"]).cuda()
    gates = torch.from_numpy(d["gates"]).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4004)
    y_down = torch.randn((cap, k), generator=gen, device="cuda").to(bf16)
    seg, slot, tok = e(num_e + 1, dt=i32), e(tokens, topk, dt=i32), e(cap, dt=i32)
    dq, ds = e(cap, k, dt=u8), e(cap, kb, dt=f32)
    out = e(tokens, k, dt=bf16)
    seg_rows = np.diff(offsets)
    scanned = int(np.minimum(seg_rows, 128).sum())          # row tokens read by the padding workgroups
    extras = [
        Call("moe_route", "moe", lambda: lib.fp8bs_moe_route(ids, num_e, rows_cap=cap, seg_offsets=seg,
                                                                slot_rows=slot, row_token=tok),
             nbytes=tokens * topk * 4 * 2 + cap * 4 + (num_e + 1) * 4, outs=(seg, slot, tok)),
        Call("moe_dispatch_x", "moe", lambda: lib.fp8bs_moe_permute_quantize(xt, slot, seg, tok, q=dq, scales=ds),
             nbytes=tokens * k * 2 + tokens * topk * 4 + scanned * 4 + total * (k + kb * 4), outs=(dq, ds)),
        Call("moe_combine", "moe", lambda: lib.fp8bs_moe_combine(y_down, slot, gates, out=out),
             nbytes=pairs * k * 2 + tokens * topk * 8 + tokens * k * 2, outs=(out,)),
    ]
    if not fused:
        step = "1x128 quantization of the routed rows + 128x128 quantization of all 256 expert weights + grouped GEMM"
    elif keep_codes:
        step = ("1x128 quantization of the routed rows + grouped GEMM from the bf16 expert weights, each 128x128 "
                "weight block quantized in the GEMM and its codes and scales stored once per expert")
    else:
        step = ("1x128 quantization of the routed rows + grouped GEMM from the bf16 expert weights, each 128x128 "
                "weight block quantized in the GEMM (codes stored once only for the experts with several "
                "128-row tiles, which read them back)")
    desc = dict(workload="c4: MoE expert grouped GEMM, 4096 tokens x top-8 of 256 experts (Zipf 1.1 counts, "
                         "rows padded to 128 per expert), fused gate+up N=4096, K=7168; step = " + step,
                routed_rows=pairs, padded_rows=total, experts=num_e, N=n, K=k,
                value_flops="grouped GEMM over the routed rows, 2*32768*4096*7168",
                bytes_counted="X quantizer: routed rows and the row map; grouped GEMM: routed rows of X, "
                              "padded output rows"
                              + (("; bf16 weights read once" + (", codes written once" if keep_codes else ""))
                                 if fused else ""))
    data = dict(kind="c4", x=host["x"], counts=counts, offsets=offsets, w_dev=w, cfg=cfg)
    return calls, state, desc, data, extras


def build_wgrad_step(lib, rotate, act_cache=False):
    import torch

    from workloads import config_by_name, wgrad_inputs

    cfg = config_by_name("c5")
    t, m, n = cfg["T"], cfg["M"], cfg["N"]
    d = wgrad_inputs(cfg)
    dy, x = dev_bf16(d["dy"]), dev_bf16(d["x"])
    qdy, sdy = torch.empty((m, t), dtype=torch.uint8, device="cuda"), torch.empty(
        (m, t // 128), dtype=torch.float32, device="cuda")
    qx, sx = torch.empty((n, t), dtype=torch.uint8, device="cuda"), torch.empty(
        (n, t // 128), dtype=torch.float32, device="cuda")
    dw = torch.empty((m, n), dtype=torch.float32, device="cuda")
    state = {"i": 0}
    if act_cache:
        # the cached forward tiles of X exist before the step (the forward pass made them)
        cx, csx = lib.fp8bs_quantize_act_1x128(x)
        x_call = Call("requant_x_t", "requant",
                      lambda: lib.fp8bs_requantize_act_1x128_t(cx, csx, qt=qx, scales_t=sx),
                      nbytes=t * n * 2 + 2 * (t * n // 128) * 4, outs=(qx, sx))
    else:
        x_call = Call("quant_act_x_t", "quant",
                      lambda: lib.fp8bs_quantize_act_1x128(x, transpose=1, q=qx, scales=sx),
                      nbytes=t * n * 3 + t * n // 128 * 4, outs=(qx, sx))
    calls = [
        Call("quant_act_dy_t", "quant", lambda: lib.fp8bs_quantize_act_1x128(dy, transpose=1, q=qdy, scales=sdy),
             nbytes=t * m * 3 + t * m // 128 * 4, outs=(qdy, sdy)),
        x_call,
        Call("gemm_wgrad", "gemm", lambda: lib.fp8bs_gemm_wgrad(qdy, sdy, qx, sx, c=dw), flops=2.0 * m * n * t,
             nbytes=(m + n) * t + (m + n) * (t // 128) * 4 + m * n * 4,
             outs=(dw,)),
    ]
    desc = dict(workload="c5: weight gradient dW[1536,7168] = dY^T X over 16384 tokens, " + (
                    "dY transpose-quantized along tokens, X re-tiled along tokens from its cached FP8 forward tiles"
                    if act_cache else "both operands transpose-quantized along tokens"), T=t, M=m, N=n)
    return calls, state, desc, dict(d, kind="wgrad", cfg=cfg), []


def run_steps(calls, state, steps):
    for _ in range(steps):
        for c in calls:
            c.fn()
        state["i"] += 1


def output_buffers(calls):
    """Every output tensor of the step, without duplicates."""
    seen, out = set(), []
    for c in calls:
        for v in c.outs:
            if v.data_ptr() not in seen:
                seen.add(v.data_ptr())
                out.append(v)
    return out


def capture_steps(calls, state, rotate):
    """One HIP graph per input copy, each holding one whole step."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(side):
        for i in range(rotate):
            state["i"] = i
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for c in calls:
                    c.fn()
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    state["i"] = 0
    return graphs


def replay_matches_eager(calls, state, graphs):
    """Run set 0 eagerly, then replay its graph over poisoned buffers: outputs must be bit-identical."""
    import torch

    bufs = output_buffers(calls)
    state["i"] = 0
    for c in calls:
        c.fn()
    torch.cuda.synchronize()
    ref = [b.clone() for b in bufs]
    for b in bufs:
        b.view(torch.uint8).fill_(0xAB)
    torch.cuda.synchronize()
    graphs[0].replay()
    torch.cuda.synchronize()

    def bits(t):
        return t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int16 if t.element_size() == 2
                                                                         else torch.int32)
    return all(torch.equal(bits(a), bits(b)) for a, b in zip(ref, bufs))


def time_kernels(calls, state, rotate, reps):
    """Average duration of each call: ``reps`` launches in one graph, HIP events around its replay."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = []
    with torch.cuda.stream(side):
        for c in calls:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for r in range(reps):
                    state["i"] = r % rotate
                    c.fn()
            g.replay()                       # warm
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(side)
            g.replay()
            b.record(side)
            b.synchronize()
            out.append(a.elapsed_time(b) / reps)
            del g
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    state["i"] = 0
    return out


def copy_rate_gbps(reps=8):
    """A plain 512 MiB device-to-device copy (reads and writes 512 MiB), timed
    with HIP events on the current stream: the HBM rate a streaming kernel can
    reach on this GPU, beside the 8 TB/s specification."""
    import torch

    n = 512 * 2 ** 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    b.synchronize()
    rate = 2 * n * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return rate


def host_threads():
    """Host threads the CPU oracle runs its matrix products on: the affinity
    mask, capped by OMP_NUM_THREADS where the environment sets it."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def cpu_model():
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def _oracle_sample_layer(data):
    """c2 / c3: the whole training pass over the first tokens (the full weight quantized each pass)."""
    from oracle import (gemm_dgrad, gemm_fprop, gemm_wgrad, quantize_act_1x128, quantize_act_1x128_t,
                        quantize_w_128x128)

    rows = 4096 if data["cfg"]["name"] == "c2" else 1024
    x, w, dy = data["a"][:rows], data["b"], data["dy"][:rows]
    m, k = x.shape
    n = w.shape[0]

    def one():
        qx, sx = quantize_act_1x128(x)
        qw, sw = quantize_w_128x128(w)
        gemm_fprop(qx, sx, qw, sw)
        qdy, sdy = quantize_act_1x128(dy)
        gemm_dgrad(qdy, sdy, qw, sw)
        qdyt, sdyt = quantize_act_1x128_t(dy)
        qxt, sxt = quantize_act_1x128_t(x)
        gemm_wgrad(qdyt, sdyt, qxt, sxt)

    text = (f"training pass over {m} of {data['a'].shape[0]} tokens: quantize X, dY (both orientations) and the "
            f"whole weight [{n},{k}], forward, dgrad and wgrad GEMMs; value = GEMM FLOPs / pass wall time")
    return one, 3 * 2.0 * m * n * k, text


def _oracle_sample_grouped(data, rows=512):
    """c4: the step's costs measured on a sample and scaled to the whole step.

    Every expert's weight has the same shape, so one expert's 128x128
    quantization stands for each of the 256; the 1x128 quantization and the
    GEMM cost in proportion to their rows, so ``rows`` routed rows of the
    largest expert (a GEMM of realistic height) stand for the routed rows
    (quantization and GEMM).  Returns the sample and a
    function that turns the sample's time into the whole step's time.
    """
    import numpy as np
    import torch

    from oracle import gemm_fprop, quantize_act_1x128, quantize_w_128x128

    counts, off, x = data["counts"], data["offsets"], data["x"]
    n, k = data["cfg"]["N"], data["cfg"]["K"]
    num_e, routed = len(counts), int(counts.sum())
    e0 = int(np.argmax(counts))
    rows = min(rows, int(counts[e0]))
    xs = x[off[e0]:off[e0] + rows]
    # the weights were drawn on the device (seeded torch generator); their bf16 bits come back unchanged
    w0 = data["w_dev"][e0].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    parts = {"w": 0.0, "x": 0.0, "gemm": 0.0}

    def one():
        t0 = time.perf_counter()
        qw, sw = quantize_w_128x128(w0)
        t1 = time.perf_counter()
        qx, sx = quantize_act_1x128(xs)
        t2 = time.perf_counter()
        gemm_fprop(qx, sx, qw, sw)
        t3 = time.perf_counter()
        parts["w"] += t1 - t0
        parts["x"] += t2 - t1
        parts["gemm"] += t3 - t2

    def step_seconds(reps):
        return (num_e * parts["w"] + routed / rows * (parts["x"] + parts["gemm"])) / reps

    text = (f"128x128 quantization of expert #{e0}'s weight [{n},{k}] (x{num_e} experts), 1x128 quantization of "
            f"{rows} of its routed rows and their GEMM (both x{routed / rows:.1f} for the {routed} routed rows); "
            f"value = the step's routed-row GEMM FLOPs / the step time so scaled")
    return one, 2.0 * routed * n * k, text, step_seconds


def _oracle_sample_wgrad(data, tokens=2048):
    """c5: the weight gradient over the first tokens (both operands transpose-quantized)."""
    from oracle import gemm_wgrad, quantize_act_1x128_t

    dy, x = data["dy"][:tokens], data["x"][:tokens]
    m, n = dy.shape[1], x.shape[1]

    def one():
        qa, sa = quantize_act_1x128_t(dy)
        qb, sb = quantize_act_1x128_t(x)
        gemm_wgrad(qa, sa, qb, sb)

    text = (f"weight gradient [{m},{n}] over the first {tokens} of {data['dy'].shape[0]} tokens: both operands "
            f"transpose-quantized, then the GEMM; value = GEMM FLOPs / wall time")
    return one, 2.0 * m * n * tokens, text


def cpu_baseline(data, min_seconds=10.0):
    """The oracle, as it stands, on a bounded sample of the configuration (host cores).

    The sample is repeated until ``min_seconds`` of host time have passed;
    value = the sample's GEMM FLOPs / mean wall time per repetition, in TFLOP/s.
    numpy's matrix products run on ``cores`` BLAS threads; its elementwise
    steps (decode, quantization) on one.
    """
    threads = host_threads()
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=threads, user_api="blas")
    except Exception:  # pragma: no cover - threadpoolctl missing
        limit = None
    try:
        kind = data["kind"]
        scale = None
        if kind == "c4":
            one, flops, text, scale = _oracle_sample_grouped(data)
        else:
            one, flops, text = _oracle_sample_layer(data) if kind == "layer" else _oracle_sample_wgrad(data)
        reps, t0 = 0, time.perf_counter()
        while True:
            one()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    finally:
        if limit is not None:
            limit.restore_original_limits()
    per_rep = scale(reps) if scale else dt / reps
    return {"value": round(flops / per_rep / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(), "seconds": round(dt, 3), "repetitions": reps,
            "sample": f"{data['cfg']['name']}: {text}; repeated {reps}x"}


def call_roofline(c, avg_s):
    """The bound of one call and how close its average duration comes to it.

    The bound is whichever takes longer at the MI355X peaks: the call's FLOPs
    at the dense FP8 MFMA rate, or its algorithmic bytes at the HBM rate.
    ``achieved`` is the same quantity (FLOPs or bytes) per second.
    """
    t_mfma = c.flops / (FP8_PEAK_TFLOPS * 1e12)
    t_hbm = c.nbytes / (HBM_PEAK_GBPS * 1e9)
    if c.flops > 0 and t_mfma >= t_hbm:
        ach = c.flops / avg_s / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / FP8_PEAK_TFLOPS, 4), "algorithmic": c.flops}
    ach = c.nbytes / avg_s / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBPS, 4), "algorithmic": c.nbytes}


def load_traffic(name, kind):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE, encoding="utf-8") as f:
        tab = json.load(f)
    ent = tab.get(name)
    if not ent or ent.get("source_sha") != source_hash(kind):
        return None
    return ent.get("bytes_per_launch")


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding of the path is described in the design notes, not run.", file=sys.stderr)
        sys.exit(2)
    import torch

    from fp8_fine_grained_act_amd import lib

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        # a plain copy of known size: reads and writes 512 MiB each per launch
        src = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel(), "launches": 4}), flush=True)
        return

    if args.config in ("c2", "c3"):
        calls, state, desc, data, extras = build_layer_step(lib, args.config, args.rotate,
                                                            dual=not args.separate_quant, act_cache=args.act_cache)
    elif args.config == "c4":
        calls, state, desc, data, extras = build_grouped_step(lib, args.rotate, fused=not args.c4_two_calls,
                                                              keep_codes=args.c4_keep_codes)
    else:
        calls, state, desc, data, extras = build_wgrad_step(lib, args.rotate, act_cache=args.act_cache)
    if args.act_cache:
        data = None                      # the CPU baseline times the plain pass only
    torch.cuda.synchronize()
    rotate = desc.get("input_copies", 1)
    run_steps(calls, state, 1)                       # first launches outside any capture
    torch.cuda.synchronize()
    graphs, replay_ok = None, None
    if args.graph and not args.eager:
        graphs = capture_steps(calls, state, rotate)
        replay_ok = replay_matches_eager(calls, state, graphs)
        if not replay_ok:
            print("bench.py: a graph replay of the step differs from its eager launches", file=sys.stderr)
            sys.exit(1)

    def steps(n):
        if graphs is None:
            run_steps(calls, state, n)
        else:
            for _ in range(n):
                graphs[state["i"] % rotate].replay()
                state["i"] += 1

    steps(args.warmup)
    # timed region: K steps back to back
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps(args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_per_step = wall * 1e3 / args.steps
    # the step's own roofline: per call, its FLOPs at the FP8 peak or its
    # algorithmic bytes at the HBM peak, whichever takes longer
    roof_step_us = sum(max(c.flops / (FP8_PEAK_TFLOPS * 1e12), c.nbytes / (HBM_PEAK_GBPS * 1e9))
                       for c in calls) * 1e6
    gemm_flops = sum(c.flops for c in calls)
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    # per-kernel durations (second timed region, same stream discipline);
    # --kernel-reps 0 skips it (profiler runs), leaving the step average per call
    timed = calls + extras
    if args.kernel_reps > 0:
        for c, ms in zip(timed, time_kernels(timed, state, rotate, args.kernel_reps)):
            c.times_ms.append(ms)
    else:
        for c in calls:
            c.times_ms.append(ms_per_step / len(calls))
        # profiler runs: launch the extra calls a few times so a kernel trace records them
        for _ in range(min(args.steps, 5)):
            for c in extras:
                c.fn()
        torch.cuda.synchronize()
        extras = []
    kernel_sum_us = sum(c.times_ms[0] for c in calls) * 1e3
    copy_gbps = copy_rate_gbps() if args.kernel_reps > 0 else None

    def entry(c):
        avg_s = sum(c.times_ms) / len(c.times_ms) * 1e-3
        ent = {"avg_us": round(avg_s * 1e6, 2)}
        ent.update(call_roofline(c, avg_s))
        if c.kind == "gemm":
            ent["frac_fp8_peak"] = round(c.flops / avg_s / 1e12 / FP8_PEAK_TFLOPS, 4)
        if ent["bound"] == "mfma":
            ent["algorithmic_bytes"] = c.nbytes
        if copy_gbps and ent["bound"] == "hbm":
            ent["frac_copy"] = round(c.nbytes / avg_s / 1e9 / copy_gbps, 4)
        ent["traffic"] = load_traffic(f"{args.config}:{c.name}", c.kind)
        return ent

    kernels = {c.name: entry(c) for c in calls}
    dom = max(calls, key=lambda c: sum(c.times_ms))
    roof = dict(kernels[dom.name], kernel=dom.name)
    roof.pop("avg_us", None)
    gemms = [c for c in calls if c.kind == "gemm"]
    roof_gemm = None
    if gemms:
        g = max(gemms, key=lambda c: sum(c.times_ms))
        roof_gemm = dict(kernels[g.name], kernel=g.name)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "pct_of_fp8_dense_peak": round(100 * value / FP8_PEAK_TFLOPS, 2),
        "step_roofline": {"us": round(roof_step_us, 1), "pct": round(100 * roof_step_us / (ms_per_step * 1e3), 1),
                          "note": "per call max(FLOPs / 5 PFLOP/s, algorithmic bytes / 8 TB/s), summed"},
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded, shapes and distributions of the configuration)",
        "config": desc,
        "roofline": roof,
        "roofline_gemm": roof_gemm,
        "kernels": kernels,
        "timing": {"step": "eager launches on one stream" if graphs is None else "one HIP graph per step "
                   "(replay checked bit-identical to eager launches)", "kernel_sum_us": round(kernel_sum_us, 1),
                   "kernel_reps": args.kernel_reps, "warmup_steps_untimed": args.warmup},
        "hbm_copy_gbps": None if copy_gbps is None else round(copy_gbps, 1),
    }
    if extras:
        out["moe_kernels"] = {c.name: entry(c) for c in extras}
    if not args.no_cpu_baseline and data is not None:
        out["cpu_baseline"] = cpu_baseline(data, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
