"""bench.py's contract: the one-GPU guard and the traffic summary parsing run on the CPU, the
JSON line's fields are checked on a GPU at the tiny sampling size."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rejection_sampling_verification_row_amd import synth  # noqa: E402
import oracle  # noqa: E402


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
    cb, firsts = bench.cpu_baseline(w, 0.3, threads=2)
    assert cb["kind"] == "oracle" and cb["cores"] == 2
    assert cb["unit"] == "verified draft positions/s" and cb["value"] > 0
    assert cb["single_core_value"] > 0 and "on one thread" in cb["single_core_sample"]
    assert "passes over the 3" in cb["sample"] and "on 2 threads" in cb["sample"]
    assert sorted(firsts) == [0, 1, 2]          # every sequence at least once
    assert cb["cpu_model"] and cb["cpu_model"] == bench.cpu_model()
    assert 1 <= bench.host_threads() <= bench.CPU_SHARE


def test_timing_stride_keeps_about_25_timed_launches():
    assert bench.timing_stride(16) == 8 and bench.timing_stride(200) == 8
    assert bench.timing_stride(2000) == 80
    assert len(range(0, 2000, bench.timing_stride(2000))) == 25


def test_preheat_runs_calls_for_its_time_and_syncs_every_8():
    calls, syncs = [], []
    n = bench.preheat(calls.append, lambda: syncs.append(len(calls)), seconds=0.01)
    assert n == len(calls) >= 8 and n % 8 == 0
    assert calls == list(range(n))
    assert syncs == list(range(8, n + 1, 8))
    assert bench.preheat(calls.append, lambda: None, seconds=0.0) == 8   # at least one round


def test_percentiles_interpolate_like_numpy():
    xs = [5.0, 1.0, 4.0, 2.0, 3.0, 9.0, 7.0]
    got = bench.percentiles(xs)
    assert np.allclose([got["p10_ms"], got["median_ms"], got["p90_ms"]],
                       np.percentile(xs, [10, 50, 90]))
    assert bench.percentiles([])["median_ms"] is None


def test_run_calls_covers_the_first_items_however_short_the_time():
    seen = []
    n, dt, firsts = bench.run_calls(lambda i: seen.append(i) or i * i, 3, 0.0, 10)
    assert sorted(firsts) == list(range(10)) and firsts[7] == 49
    assert n == len(seen) >= 10


def _as_gpu(res, probs=True):
    g = {"acc": res.accepted_len.copy(), "out": res.out_tokens.copy()}
    if probs:
        g["probs"] = res.out_probs.astype(np.float32)
    return g


def test_oracle_check_counts_agreement_and_catches_a_planted_mismatch():
    w = synth.make_sampling(6, 3, 400, synth.F32, 1.0, 7, target_sigma=2.0)
    whole = oracle.run_workload(w)                      # stands in for the GPU's outputs
    firsts = {b: oracle.run_workload(w.subset([b])) for b in range(w.B)}
    g = _as_gpu(whole)
    chk = bench.oracle_check(w, g, firsts)
    assert chk["mismatched"] == 0 and chk["bit_exact"] + chk["low_margin"] == w.B
    b = next(i for i in range(w.B) if firsts[i].margin[0] >= oracle.LOW_MARGIN)
    L = int(g["acc"][b])                                # plant a wrong draw in sequence b
    g["out"][b, L] = (g["out"][b, L] + 1) % w.V
    assert bench.oracle_check(w, g, firsts)["mismatched"] == 1
    g = _as_gpu(whole)
    g["probs"][1, 0, 0] *= 1.001                        # a probability off by 1e-3
    assert bench.oracle_check(w, g, firsts)["mismatched"] == 1


def test_oracle_check_greedy_is_exact():
    w = synth.make_greedy(5, 4, 300, synth.BF16, 11)
    whole = oracle.run_workload(w)
    firsts = {b: oracle.run_workload(w.subset([b])) for b in range(w.B)}
    g = _as_gpu(whole, probs=False)
    assert bench.oracle_check(w, g, firsts) | {"rule": ""} == {
        "items": 5, "bit_exact": 5, "low_margin": 0, "mismatched": 0, "rule": ""}
    g["acc"][2] = (g["acc"][2] + 1) % (w.K + 1)
    assert bench.oracle_check(w, g, firsts)["mismatched"] == 1


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
    # the dominant kernel timed in a pass of its own: at least 25 launches, even for 16 steps
    assert rf["timed_launches"] == 25 and rf["timing_stride"] == 8
    assert 0 < rf["p10_ms"] <= rf["median_ms"] <= rf["p90_ms"]
    pc = d["per_call_ms"]                       # per-call percentiles from their own pass
    assert pc["calls"] == 100 and 0 < pc["p10_ms"] <= pc["median_ms"] <= pc["p90_ms"]
    # the breakdown is taken after a preheat: its kernels fit inside the step, up to the
    # completion signalling an event-timed dispatch adds (about 1 us each: this call is 11 us)
    assert sum(d["kernels_ms_per_step"].values()) <= d["ms_per_step"] * 1.05 + 0.003
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    chk = d["oracle_check"]
    assert chk["items"] == 1 and chk["mismatched"] == 0
