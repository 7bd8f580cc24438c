"""The five benchmark configurations (shapes, distributions, seeds)."""

CONFIGS = {
    # plumbing case: small enough for the oracle to finish in well under a second
    "c1": dict(kind="gemm", seed=1, M=256, N=256, K=512,
               a_std=1.0, b_std=0.02, n_outlier_cols=4, outlier_scale=50.0,
               desc="tiny plumbing GEMM 256x256x512"),
    # MLA query down-projection, hidden 7168 -> query latent 1536
    "c2": dict(kind="gemm", seed=2, M=4096, N=1536, K=7168,
               a_std=1.0, b_std=0.02, n_outlier_cols=72, outlier_scale=50.0,
               desc="MLA q-down projection forward 4096x1536x7168"),
    # MLA KV up-projection from the 512-wide latent to 128 heads x (128 K + 128 V)
    "c3": dict(kind="gemm", seed=3, M=4096, N=32768, K=512,
               a_std=1.0, b_std=0.02, n_outlier_cols=5, outlier_scale=20.0,
               desc="MLA kv-up projection forward 4096x32768x512"),
    # MoE routed experts: 4096 tokens, top-8 of 256, fused gate+up (N=4096), K=7168
    "c4": dict(kind="grouped", seed=4, tokens=4096, topk=8, experts=256, N=4096, K=7168,
               zipf_s=1.1, a_std=1.0, b_std=0.02,
               desc="MoE grouped GEMM, 4096 tokens x top-8 of 256 experts, N=4096, K=7168"),
    # weight gradient dW = dY^T X over 16384 tokens
    "c5": dict(kind="wgrad", seed=5, T=16384, M=1536, N=7168,
               dy_std=1e-3, x_std=1.0, n_outlier_rows=164, outlier_scale=30.0,
               desc="weight-gradient GEMM 1536x7168 over 16384 tokens"),
}


def config_by_name(name):
    if name not in CONFIGS:
        raise KeyError(f"unknown configuration {name!r}; have {sorted(CONFIGS)}")
    return dict(CONFIGS[name], name=name)
