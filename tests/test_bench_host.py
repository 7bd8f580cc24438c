"""Host-side checks of bench.py (no GPU needed).

- It runs on one GPU only: a request for more exits with status 2 and says so.
- The per-kernel HBM traffic it reports comes from profiles/traffic.json; every
  entry must be well formed, carry the calibration of a plain device copy
  (FETCH_SIZE reads half the copied bytes, WRITE_SIZE all of them), and add up
  to its own counter readings.
"""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402  (imports torch lazily, inside its GPU paths)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_kernel_source_lists_exist_and_hash():
    for kind, files in bench.KERNEL_SOURCES.items():
        assert files, kind
        for rel in files:
            assert os.path.isfile(os.path.join(ROOT, rel)), rel
        h = bench.source_hash(kind)
        assert len(h) == 16 and int(h, 16) >= 0
        assert h == bench.source_hash(kind)


def test_traffic_table_entries():
    with open(bench.TRAFFIC_FILE, encoding="utf-8") as f:
        tab = json.load(f)
    assert tab
    for key, ent in tab.items():
        cfg, call = key.split(":")
        assert cfg in ("c2", "c3", "c4", "c5"), key
        assert call, key
        assert len(ent["source_sha"]) == 16 and int(ent["source_sha"], 16) >= 0, key
        assert abs(ent["fetch_factor"] - 2.0) < 0.05, key
        assert abs(ent["write_factor"] - 1.0) < 0.05, key
        total = 1024 * (ent["fetch_kib"] * ent["fetch_factor"] + ent["write_kib"] * ent["write_factor"])
        assert ent["bytes_per_launch"] > 0
        # the stored readings and factors are rounded (0.1 KiB, 4 decimals)
        assert abs(ent["bytes_per_launch"] - total) <= 1e-3 * total, key


def test_traffic_lookup_rejects_stale_sources(monkeypatch, tmp_path):
    fake = tmp_path / "traffic.json"
    fake.write_text(json.dumps({
        "c2:gemm_wgrad": {"source_sha": bench.source_hash("gemm"), "bytes_per_launch": 123},
        "c2:quant_w": {"source_sha": "0" * 16, "bytes_per_launch": 456},
    }))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(fake))
    assert bench.load_traffic("c2:gemm_wgrad", "gemm") == 123
    assert bench.load_traffic("c2:quant_w", "quant") is None
    assert bench.load_traffic("c2:missing", "gemm") is None


def test_call_roofline_picks_the_longer_bound():
    """A call's bound is whichever of its FLOPs at the dense FP8 peak and its
    algorithmic bytes at the HBM peak takes longer; `achieved` is that quantity
    per second of the measured duration."""
    # c4's fused grouped GEMM: 1.924 TFLOP over the routed rows, 15.72 GB moved
    flops, nbytes = 2.0 * 32768 * 4096 * 7168, 15_716_272_640
    c = bench.Call("gemm_grouped_bf16w", "gemm", None, flops=flops, nbytes=nbytes)
    r = bench.call_roofline(c, 5.58e-3)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["algorithmic"] == nbytes
    assert abs(r["achieved"] - nbytes / 5.58e-3 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / bench.HBM_PEAK_GBPS) < 1e-4
    # a square layer GEMM: 2 * 4096^2 * 7168 FLOP over ~100 MB is MFMA-bound
    c = bench.Call("gemm_fprop", "gemm", None, flops=2.0 * 4096 * 4096 * 7168, nbytes=100e6)
    r = bench.call_roofline(c, 100e-6)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["achieved"] - c.flops / 100e-6 / 1e12) < 0.1
    # a quantizer has no FLOPs: always HBM
    c = bench.Call("quant_w", "quant", None, nbytes=1e9)
    assert bench.call_roofline(c, 1e-3)["bound"] == "hbm"


def test_c4_two_calls_flag_parses():
    sys_argv = sys.argv
    try:
        sys.argv = ["bench.py", "--c4-two-calls"]
        a = bench.parse_args()
        assert a.c4_two_calls and a.config == "c4" and a.steps == 20 and a.warmup == 5
        sys.argv = ["bench.py"]
        a = bench.parse_args()
        assert not a.c4_two_calls and not a.c4_keep_codes
        sys.argv = ["bench.py", "--c4-keep-codes"]
        assert bench.parse_args().c4_keep_codes
    finally:
        sys.argv = sys_argv
