"""Seeded generators for the benchmark inputs (bf16 bit patterns as uint16)."""

import numpy as np

from .configs import config_by_name

GROUP = 128


def f32_to_bf16_bits(x):
    """Round finite float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _streams(seed, count=4):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(count)]


def normal_bf16(rng, shape, std):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def _n_outliers(dim):
    return int(round(0.01 * dim))


def gemm_inputs(name_or_cfg, **override):
    """Forward-GEMM inputs: A [M,K] (outlier columns) and B [N,K].

    Returns dict(a=uint16 [M,K], b=uint16 [N,K], outlier_cols=int array).
    """
    cfg = config_by_name(name_or_cfg) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(override)
    m, n, k = cfg["M"], cfg["N"], cfg["K"]
    rng_a, rng_b, rng_o, _ = _streams(cfg["seed"])
    a = rng_a.standard_normal(size=(m, k), dtype=np.float32)
    if cfg.get("a_std", 1.0) != 1.0:
        a *= np.float32(cfg["a_std"])
    n_out = cfg.get("n_outlier_cols")
    if n_out is None:
        n_out = _n_outliers(k)
    cols = np.sort(rng_o.choice(k, size=n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    a[:, cols] *= np.float32(cfg.get("outlier_scale", 1.0))
    a_bits = f32_to_bf16_bits(a)
    del a
    b_bits = normal_bf16(rng_b, (n, k), cfg.get("b_std", 0.02))
    return dict(a=a_bits, b=b_bits, outlier_cols=cols)


def layer_inputs(name_or_cfg, dy_std=1e-3, **override):
    """Forward-GEMM inputs plus an output gradient dY [M, N] ~ N(0, dy_std).

    For a training pass of one linear layer: forward Y = X W^T, activation
    gradient dX = dY W, weight gradient dW = dY^T X.  dY comes from a fifth
    stream of the same seed, so A and B are identical to ``gemm_inputs``.
    Returns dict(a=X [M,K], b=W [N,K], dy=[M,N]) as bf16 bits.
    """
    cfg = config_by_name(name_or_cfg) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(override)
    d = gemm_inputs(cfg)
    rng_dy = _streams(cfg["seed"], 5)[4]
    d["dy"] = normal_bf16(rng_dy, (cfg["M"], cfg["N"]), dy_std)
    return d


def wgrad_inputs(name_or_cfg, **override):
    """Weight-gradient inputs: dY [T,M] (outlier token rows) and X [T,N].

    Returns dict(dy=uint16 [T,M], x=uint16 [T,N], outlier_rows=int array).
    """
    cfg = config_by_name(name_or_cfg) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(override)
    t, m, n = cfg["T"], cfg["M"], cfg["N"]
    rng_a, rng_b, rng_o, _ = _streams(cfg["seed"])
    dy = rng_a.standard_normal(size=(t, m), dtype=np.float32)
    dy *= np.float32(cfg.get("dy_std", 1e-3))
    n_out = cfg.get("n_outlier_rows")
    if n_out is None:
        n_out = _n_outliers(t)
    rows = np.sort(rng_o.choice(t, size=n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    dy[rows, :] *= np.float32(cfg.get("outlier_scale", 1.0))
    dy_bits = f32_to_bf16_bits(dy)
    del dy
    x_bits = normal_bf16(rng_b, (t, n), cfg.get("x_std", 1.0))
    return dict(dy=dy_bits, x=x_bits, outlier_rows=rows)


def _topk_choice(cfg):
    """Seeded top-k expert choice: (ids [T, k] by descending key, keys [T, E], rng).

    Expert e has popularity p(e) proportional to (e+1)^(-s); a token's k
    distinct experts come from the Gumbel-top-k trick on log p (one Gumbel
    draw per token and expert), listed from the largest key down.
    """
    tokens, topk, num_e, s = cfg["tokens"], cfg["topk"], cfg["experts"], cfg["zipf_s"]
    rng = _streams(cfg["seed"])[3]
    logp = -s * np.log(np.arange(1, num_e + 1, dtype=np.float64))
    keys = logp[None, :] + rng.gumbel(size=(tokens, num_e))
    chosen = np.argpartition(-keys, topk - 1, axis=1)[:, :topk]
    order = np.argsort(-np.take_along_axis(keys, chosen, axis=1), axis=1, kind="stable")
    return np.take_along_axis(chosen, order, axis=1), keys, rng


def moe_dispatch_inputs(name_or_cfg, hidden=None, **override):
    """Token-order inputs of the MoE dispatch and combine.

    ids    int32 [T, k]   top-k expert ids (``_topk_choice``)
    gates  float32 [T, k] gate weights: uniform(0.05, 1) draws, divided by
           their per-token sum (positive, summing to about 1, like normalized
           router affinities of the chosen experts)
    x      bf16 bits [T, hidden] i.i.d. N(0, a_std) token activations
    hidden defaults to the configuration's K (the model width).
    """
    cfg = config_by_name(name_or_cfg) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(override)
    ids, _, rng = _topk_choice(cfg)
    tokens, topk = ids.shape
    g = rng.uniform(0.05, 1.0, size=(tokens, topk)).astype(np.float32)
    g /= g.sum(axis=1, keepdims=True, dtype=np.float32)
    h = int(cfg["K"] if hidden is None else hidden)
    x = normal_bf16(_streams(cfg["seed"])[0], (tokens, h), cfg.get("a_std", 1.0))
    return dict(ids=ids.astype(np.int32), gates=g.astype(np.float32), x=x, experts=int(cfg["experts"]))


def moe_routing(name_or_cfg, **override):
    """Per-expert routed-row counts for top-k routing with Zipf-skewed popularity.

    Each token picks ``topk`` distinct experts; expert e has popularity
    p(e) proportional to (e+1)^(-s).  Sampling without replacement is done by
    the Gumbel-top-k trick on log p (one seeded Gumbel draw per token/expert).
    Returns dict(counts [E], padded [E], offsets [E+1] (padded, multiples of 128)).
    """
    cfg = config_by_name(name_or_cfg) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(override)
    tokens, topk, num_e, s = cfg["tokens"], cfg["topk"], cfg["experts"], cfg["zipf_s"]
    chosen = _topk_choice(cfg)[0]
    counts = np.bincount(chosen.ravel(), minlength=num_e).astype(np.int64)
    padded = (counts + GROUP - 1) // GROUP * GROUP
    offsets = np.zeros(num_e + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    return dict(counts=counts, padded=padded, offsets=offsets)


def grouped_inputs_host(name_or_cfg, with_weights=True, **override):
    """Grouped-GEMM inputs drawn on the host.

    X: the routed rows, i.i.d. N(0, a_std), placed in expert order into the
    padded segments; padding rows are +0.0.  W: per-expert [E, N, K] from the
    weight stream (only when ``with_weights``; practical for small shapes).
    Returns dict(x [R_pad,K], w [E,N,K] or None, counts, offsets).
    """
    cfg = config_by_name(name_or_cfg) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(override)
    route = moe_routing(cfg)
    counts, offsets = route["counts"], route["offsets"]
    k, n, num_e = cfg["K"], cfg["N"], cfg["experts"]
    rng_a, rng_b, _, _ = _streams(cfg["seed"])
    real = rng_a.standard_normal(size=(int(counts.sum()), k), dtype=np.float32)
    if cfg.get("a_std", 1.0) != 1.0:
        real *= np.float32(cfg["a_std"])
    real_bits = f32_to_bf16_bits(real)
    del real
    x = np.zeros((int(offsets[-1]), k), dtype=np.uint16)
    src = 0
    for e in range(num_e):
        c = int(counts[e])
        x[offsets[e]:offsets[e] + c] = real_bits[src:src + c]
        src += c
    w = normal_bf16(rng_b, (num_e, n, k), cfg.get("b_std", 0.02)) if with_weights else None
    return dict(x=x, w=w, counts=counts, offsets=offsets)


def device_expert_weights(name_or_cfg, device="cuda", **override):
    """Expert weights [E, N, K] in bf16 drawn on the GPU (seeded torch generator)."""
    import torch

    cfg = config_by_name(name_or_cfg) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(override)
    num_e, n, k = cfg["experts"], cfg["N"], cfg["K"]
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 + int(cfg["seed"]))
    w = torch.empty((num_e, n, k), dtype=torch.bfloat16, device=device)
    std = float(cfg.get("b_std", 0.02))
    for e in range(num_e):
        t = torch.randn((n, k), generator=gen, device=device, dtype=torch.float32)
        w[e].copy_(t.mul_(std))
    return w
