"""Host logic of bench.py: the one-GPU contract, the algorithmic bytes of the
roofline, and the counter summaries it reads (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from multiresolution_hash_grid_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_per_point():
    # x once (12 B), 8 corners x L x F table elements, the L*F outputs; the
    # backward reads the upstream row and makes 8 L F fp32 additions.
    w = I.WORKLOADS["standard"]
    assert bench.algorithmic_bytes_per_point(w, 4) == {"fwd": 12 + 8 * 16 * 2 * 4 + 16 * 2 * 4,
                                                       "bwd": 12 + 16 * 2 * 4 + 8 * 16 * 2 * 4}
    assert bench.algorithmic_bytes_per_point(w, 4)["fwd"] == 1164
    assert bench.algorithmic_bytes_per_point(I.WORKLOADS["large_f16"], 2)["fwd"] == 12 + 8 * 32 * 2 * 2 + 32 * 2 * 4


def test_l2_request_peak_is_the_chip_derivation():
    assert bench.L2_REQ_PEAK_PER_S == pytest.approx(8 * 16 * 2.4e9)


def test_counter_summaries_missing_or_stale(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.load_counters("standard") is None
    assert bench.load_traffic("backward") is None
    assert bench.counter_summary(None) is None
    (tmp_path / "counters_standard.json").write_text(
        '{"source_sha256": "0", "passes": {"backward": {"hbm_bytes": 1.0}}, "kernels": {}}')
    assert bench.load_counters("standard") is None       # taken on other library sources
    assert bench.load_traffic("backward") is None


def test_counter_summary_fields(tmp_path, monkeypatch):
    from multiresolution_hash_grid_amd import profile_summary as ps
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    p = {"hbm_bytes": 7.0, "hbm_GBps": 1.0, "hbm_frac": 0.1, "traffic_over_algorithmic": 2.0, "l2_hit_rate": 0.5,
         "l2_requests_per_s": 3.0, "l2_request_frac": 0.2, "time_us": 10.0}
    rec = {"source_sha256": ps.source_digest(), "passes": {"backward": p},
           "kernels": {"mlp_bwd_kernel": {"pass": "backward", "mfma_util_pct": 24.0, "mfma_fp16_tflops": 300.0}}}
    import json
    (tmp_path / "counters_standard.json").write_text(json.dumps(rec))
    assert bench.load_traffic("backward") == 7.0
    cs = bench.counter_summary(bench.load_counters("standard"))
    assert cs["backward"]["l2_hit_rate"] == 0.5 and cs["backward"]["mfma"]["mlp_bwd_kernel"]["util_pct"] == 24.0


def test_cpu_model_is_reported():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
