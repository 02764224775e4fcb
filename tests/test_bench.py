"""bench.py's contract: the one-GPU guard and the traffic summary parsing run on the CPU, the
JSON line's fields are checked on a GPU at the tiny sampling size."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rejection_sampling_verification_row_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_summary_needs_the_current_kernel_source(tmp_path, monkeypatch):
    good = tmp_path / "good.md"
    good.write_text("# x\n\n- traffic_bytes_per_launch: 1234\n- kernel_source_sha256: %s\n"
                    % bench.kernel_source_hash())
    stale = tmp_path / "stale.md"
    stale.write_text("- traffic_bytes_per_launch: 1234\n- kernel_source_sha256: %s\n" % ("0" * 64))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("good.md") == 1234
    assert bench.measured_traffic("stale.md") is None
    assert bench.measured_traffic(None) is None
    assert bench.measured_traffic("missing.md") is None


def test_cpu_baseline_reports_the_oracle_on_a_bounded_sample():
    w = synth.make_sampling(3, 2, 500, synth.F32, 1.0, 5, target_sigma=2.0)
    cb = bench.cpu_baseline(w, 0.2)
    assert cb["kind"] == "oracle" and cb["cores"] == 1
    assert cb["unit"] == "verified draft positions/s" and cb["value"] > 0
    assert "passes over the 3" in cb["sample"]


@pytest.mark.gpu
def test_bench_line_has_the_contract_fields():
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "c1",
                        "--steps", "16", "--warmup", "4", "--cpu-seconds", "0.5"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 16 and d["warmup"] == 4 and d["value"] > 0
    assert d["config"]["workload"].startswith("sampling verify B=1 K=4 V=1000")
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    assert rf["timed_launches"] == 2 and rf["timing_stride"] == 8   # steps 0 and 8 of 16
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
