#!/usr/bin/env python3
"""Benchmark of the sampling verify-and-accept step on one MI355X.

Workload: B=256 sequences, K=8 draft tokens, V=128256, bfloat16 logits, T=0.7 (target
~N(0,4^2) plus +8 at 20 distinct ids per row, draft = target + N(0,1.5^2)), seeded and
synthetic.  One step = one specverify_run_sampling call over the whole batch (row
statistics, then accept + first-reject scan + residual/bonus draw).  Inputs sit in HBM
before timing starts and alternate between two copies so that no step reads logits the
previous one left in the 256 MB last-level cache.

Prints one JSON line: verified draft positions/s (B*K per step), the row-statistics
kernel's bytes/s against the 8 TB/s HBM peak (timed with HIP events on the call's stream),
and the fp64 CPU oracle timed on a bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified draft positions/s + HBM GB/s vs peak at B=256 K=8 V=128256 bf16"
HBM_PEAK_GBPS = 8000.0
B, K, V, T, SEED = 256, 8, 128256, 0.7, 1003
KERNEL_SRC = os.path.join(ROOT, "rejection_sampling_verification_row_amd", "csrc", "sv_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "row_stats_bf16_B256_K8_V128256_traffic.md")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per launch of the row-statistics kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        line = line.strip().lstrip("-* ")
        if ":" in line and line.startswith(("traffic_bytes_per_launch", "kernel_source_sha256")):
            k, v = line.split(":", 1)
            vals[k.strip().strip("`")] = v.strip().strip("` ")
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, seconds: float):
    """The oracle, single-threaded, on the first sequences of the batch until `seconds`."""
    import oracle
    oracle.build(force=False)
    done, t0 = 0, time.perf_counter()
    while done < w.B and time.perf_counter() - t0 < seconds:
        oracle.run_workload(w.subset([done]))
        done += 1
    dt = time.perf_counter() - t0
    return {"value": done * w.K / dt, "unit": "verified draft positions/s", "cores": 1,
            "kind": "oracle",
            "sample": "first %d of the %d sequences of the same batch, one at a time, %.1f s "
                      "single-threaded fp64 C" % (done, w.B, dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU work for the oracle baseline sample (0 disables it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, copy a 1 GiB buffer once (a known-size kernel for "
                         "scaling the HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the verify step shards over sequences with no exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from rejection_sampling_verification_row_amd import binding as sv
    from rejection_sampling_verification_row_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    log("generating the workload (seed %d)" % SEED)
    w = synth.c3_sampling_large_vocab(B=B, seed=SEED)
    log("uploading %.2f GB of logits x2" % (w.logit_bytes / 1e9))

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")

    copies = []
    for _ in range(2):
        copies.append((up(w.target), up(w.draft)))
    toks, unif = up(w.tokens), up(w.uniforms)
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    probs = torch.empty((B, K, 2), dtype=torch.float32, device="cuda")
    ctx = sv.specverify_create(0, B, K, V)
    stream = torch.cuda.current_stream()

    def step(i):
        tg, dr = copies[i & 1]
        sv.specverify_run_sampling(ctx, stream, synth.BF16, B, K, V, w.temperature, tg, dr, toks,
                                   unif, acc, out, probs)

    log("warmup %d" % args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    # HIP events around the row-statistics kernel only, on the call's stream
    sv.specverify_profile_begin(ctx, args.steps, ["row_stats"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kms, kn = sv.specverify_profile_end(ctx)
    mean_L = float(acc.float().mean().item())
    # per-kernel breakdown from a separate, untimed pass with events around every kernel
    nb = min(args.steps, 20)
    sv.specverify_profile_begin(ctx, nb)
    for i in range(nb):
        step(i)
    torch.cuda.synchronize()
    bms, bn = sv.specverify_profile_end(ctx)
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d bytes once for counter calibration" % src.nbytes)
    sv.specverify_destroy(ctx)

    ms_step = (t1 - t0) * 1e3 / args.steps
    positions = B * K / (ms_step * 1e-3)
    stats_ms = kms["row_stats"] / max(kn["row_stats"], 1)
    logit_bytes = w.logit_bytes                      # one read of every logit row
    call_bytes = logit_bytes + w.tokens.nbytes + w.uniforms.nbytes + acc.nbytes + out.nbytes
    achieved = logit_bytes / (stats_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": positions,
        "unit": "verified draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "sampling verify B=256 K=8 V=128256 bf16 logits T=0.7",
                   "B": B, "K": K, "V": V, "logits": "bf16", "temperature": T, "seed": SEED},
        "hbm_gbps_per_call": call_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac_of_peak_per_call": call_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(),
                     "kernel": "k_stats_sampling<bf16>", "algorithmic_bytes": logit_bytes,
                     "avg_ms": stats_ms},
        "kernels_ms_per_step": {k: bms[k] / bn[k] for k in bms if bn[k]},
        "mean_accepted_len": mean_L,
    }
    if args.cpu_seconds > 0:
        log("CPU oracle baseline (~%.0f s)" % args.cpu_seconds)
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
