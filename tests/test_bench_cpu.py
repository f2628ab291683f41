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
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "absent.json"))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.load_counters() == (None, None)
    assert bench.load_traffic("backward") is None
    assert bench.cache_summary(None) is None
    stale = tmp_path / "stale.json"
    stale.write_text('{"source_sha256": "0", "mlp_source_sha256": "0", "l2": {"k": {}}, "mfma": {"m": {}},'
                     ' "passes": {"backward": {"hbm_bytes_per_launch": 1.0}}}')
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(stale))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.load_counters() == (None, None)       # taken on other kernel sources
    assert bench.load_traffic("backward") is None


def test_cpu_model_is_reported():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
