#!/usr/bin/env python3
"""Benchmark of the batched verify-and-accept step on one MI355X.

Default workload (the headline): sampling verify, B=256 sequences, K=8 draft tokens,
V=128256, bfloat16 logits, T=0.7 (target ~N(0,4^2) plus +8 at 20 distinct ids per row,
draft = target + N(0,1.5^2)), seeded and synthetic.  One step = one specverify_run_sampling
call over the whole batch (row statistics, then accept + first-reject scan + residual/bonus
draw).  Inputs sit in HBM before timing starts and alternate between two copies so that no
step reads logits the previous one left in the 256 MB last-level cache.

Prints one JSON line: verified draft positions/s (B*K per step, from the wall clock over
back-to-back calls with no events in them), per-call p10 / median / p90 (HIP events around
each call, in a pass of its own), the dominant kernel's bytes/s against the 8 TB/s HBM peak
(HIP events attached to that kernel's dispatch on the call's stream, at least 25 launches in
a pass of their own: every 40th of 1000 calls by default),
the fp64 CPU oracle timed on a bounded sample of the same batch (on one thread, then on all
host threads up to 16), and a check of the GPU's outputs for the whole batch against that
oracle run.

--workload names one of the other synthetic workloads (the tiny and mid-size sampling ones,
greedy blockwise, contrastive, and the operations next to the verify step: the draft-token
sampler, greedy verify with the next block's proposals, the alpha-quantile cut) to measure
its path the same way; the default is the one the headline metric is quoted on.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "rejection_sampling_verification_row_amd", "csrc", "sv_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")

# workload key -> (description, timed kernel kind, its kernel name, traffic summary file)
WORKLOADS = {
    "c3": ("sampling verify B=256 K=8 V=128256 bf16 logits T=0.7", "row_stats",
           "k_stats_sampling<bf16>", "row_stats_bf16_B256_K8_V128256_traffic.md"),
    "c1": ("sampling verify B=1 K=4 V=1000 f32 logits T=1", "row_stats",
           "k_stats_sampling<f32>", "row_stats_f32_B1_K4_V1000_traffic.md"),
    "c2": ("sampling verify B=64 K=5 V=32000 f32 logits T=1", "row_stats",
           "k_stats_sampling<f32>", "row_stats_f32_B64_K5_V32000_traffic.md"),
    "c4": ("greedy blockwise verify B=512 K=8 V=32000 bf16 logits", "row_argmax",
           "k_argmax<bf16>", "row_argmax_bf16_B512_K8_V32000_traffic.md"),
    "c5": ("contrastive verify B=128 K=4 V=152064 bf16 logits tau=1", "row_stats",
           "k_stats_contrastive<bf16>", "contrastive_stats_bf16_B128_K4_V152064_traffic.md"),
    "sample": ("draft-token sampler N=256 V=128256 bf16 logits T=0.7", "row_stats",
               "k_stats_sampling<bf16>", "sampler_stats_bf16_N256_V128256_traffic.md"),
    "heads": ("greedy verify with next-block proposals B=512 K=4 H=4 V=32000 bf16 logits",
              "row_argmax", "k_argmax<bf16> (head 0 rows)",
              "head0_argmax_bf16_B512_K4_H4_V32000_traffic.md"),
    "cut": ("alpha-quantile cut P=128 N=1000 alpha=0.5 f32 scores", "quantile_cut",
            "k_quantile_cut", None),
    "early": ("sampling verify with early exit B=256 K=8 V=128256 bf16 logits T=0.7",
              "row_stats", "k_stats_prefix<bf16> (positions 0-1 of every sequence)",
              "prefix_stats_bf16_B256_K8_V128256_traffic.md"),
    "early_c4": ("greedy blockwise verify with early exit B=512 K=8 V=32000 bf16 logits",
                 "row_argmax", "k_argmax_prefix<bf16> (positions 0-2 of every sequence)",
                 "prefix_argmax_bf16_B512_K8_V32000_traffic.md"),
    "early_c5": ("contrastive verify with early exit B=128 K=4 V=152064 bf16 logits tau=1",
                 "row_stats", "k_pairs_prefix<bf16> (row pairs 0-1 of every sequence)",
                 "prefix_pairs_bf16_B128_K4_V152064_traffic.md"),
}
TIMING_STRIDE = 8   # the dominant kernel is timed in calls 0, 8, 16, ... of its pass
TIMED_LAUNCHES = 25  # ... at least this many launches (spread further in longer runs)


def timing_stride(steps: int) -> int:
    """Time every stride-th step: every 8th, or fewer so that about 25 launches are timed.
    A timed dispatch costs the call several microseconds more (its completion signalling),
    which is negligible for a 200 us call but not for a 5 us one, so longer runs of short
    calls time proportionally fewer of them."""
    return max(TIMING_STRIDE, steps // TIMED_LAUNCHES)
METRIC = "verified draft positions/s + HBM GB/s vs peak at B=256 K=8 V=128256 bf16"


PREHEAT_SECONDS = 0.03  # untimed calls before the warm-up steps, by wall time
# The first few thousand kernel launches of a process enqueue slowly (about 25 us per call of
# the sampler against 7-8 us later, through the binding or bare ctypes alike), which made a
# small workload's loop host-bound; the first preheat therefore also makes this many calls.
PREHEAT_FIRST_CALLS = 3000


def preheat(step, sync, seconds: float = PREHEAT_SECONDS, calls: int = 0) -> int:
    """Untimed calls for about `seconds` of wall time and at least `calls` calls, synchronising
    every 8 calls so that the host does not run ahead of the GPU.  The GPU raises its clocks
    only after ~12 ms of continuous work, whatever the call size; running this before the
    warm-up steps keeps a short --warmup from leaving the first timed steps in that ramp.
    Returns the calls made."""
    t_end = time.perf_counter() + seconds
    n = 0
    while True:
        for _ in range(8):
            step(n)
            n += 1
        sync()
        if time.perf_counter() >= t_end and n >= calls:
            return n


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence


def hip_runtime():
    """The HIP runtime library this process (torch) has loaded."""
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                return ctypes.CDLL(line.split()[-1])
    raise RuntimeError("libamdhip64.so is not loaded in this process")


def call_times(step, n, torch):
    """Milliseconds of each of n calls, from a pair of HIP events recorded around it on the
    current stream.  The events are created with hipEventDisableSystemFence: they serve
    timing only, so recording them writes back and invalidates no cache (torch's events do,
    which adds that cost to the call being timed)."""
    hip = hip_runtime()
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    evs = [ctypes.c_void_p() for _ in range(2 * n)]

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError("%s failed with HIP error %d" % (what, rc))
    try:
        for e in evs:
            ok(hip.hipEventCreateWithFlags(ctypes.byref(e),
                                           ctypes.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE)),
               "hipEventCreateWithFlags")
        for i in range(n):
            ok(hip.hipEventRecord(evs[2 * i], sh), "hipEventRecord")
            step(i)
            ok(hip.hipEventRecord(evs[2 * i + 1], sh), "hipEventRecord")
        torch.cuda.synchronize()
        ms = []
        for i in range(n):
            t = ctypes.c_float()
            ok(hip.hipEventElapsedTime(ctypes.byref(t), evs[2 * i], evs[2 * i + 1]),
               "hipEventElapsedTime")
            ms.append(t.value)
        return ms
    finally:
        for e in evs:
            if e.value:
                hip.hipEventDestroy(e)


def timed_passes(args, step, ctx, kind, sv, torch):
    """The passes after the wall-clock loop, each after a preheat that brings the clocks back
    up from the idle wait at the end of the previous one:
    - the dominant kernel's durations: HIP events attached to its dispatch, on the call's
      stream, in every stride-th of max(steps, 25 * stride) calls (at least 25 launches; a
      timed dispatch costs the call a few microseconds, so the events stay out of the
      wall-clock loop);
    - per-call times: a pair of HIP events around each of max(steps, 100) calls (their marker
      packets sit between calls, not between a call's kernels), for p10 / median / p90;
      the events are created without the system-scope fence (`call_times`);
    - the per-kernel breakdown: every kernel of every 8th of 160 calls.
    Returns (dominant-kernel durations ms, per-kind sums ms, per-kind counts, stride,
    per-call ms, breakdown sums ms, breakdown counts)."""
    stride = timing_stride(args.steps)
    n_k = max(args.steps, TIMED_LAUNCHES * stride)
    preheat(step, torch.cuda.synchronize)
    sv.specverify_profile_begin(ctx, n_k, [kind], stride=stride)
    for i in range(n_k):
        step(i)
    torch.cuda.synchronize()
    kdur = sv.specverify_profile_launches(ctx, kind)
    kms, kn = sv.specverify_profile_end(ctx)

    n_c = max(args.steps, 100)
    preheat(step, torch.cuda.synchronize)
    call_ms = call_times(step, n_c, torch)

    nb = 20 * TIMING_STRIDE
    preheat(step, torch.cuda.synchronize)
    sv.specverify_profile_begin(ctx, (nb + TIMING_STRIDE - 1) // TIMING_STRIDE,
                                stride=TIMING_STRIDE)
    for i in range(nb):
        step(i)
    torch.cuda.synchronize()
    bms, bn = sv.specverify_profile_end(ctx)
    return kdur, kms, kn, stride, call_ms, bms, bn


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(name):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary, if there is one and it was taken on the current kernel source; else None."""
    if not name:
        return None
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
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


def percentiles(ms: list) -> dict:
    """p10, median and p90 of durations (ms), by linear interpolation."""
    if not ms:
        return {"p10_ms": None, "median_ms": None, "p90_ms": None}
    xs = sorted(ms)

    def q(f):
        x = f * (len(xs) - 1)
        i = int(x)
        j = min(i + 1, len(xs) - 1)
        return xs[i] + (xs[j] - xs[i]) * (x - i)

    return {"p10_ms": q(0.1), "median_ms": q(0.5), "p90_ms": q(0.9)}


CPU_SHARE = 16   # host threads that go with one GPU


def host_threads() -> int:
    """Threads for the oracle's parallel leg: the CPUs this process may run on, at most the
    host share of one GPU."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(CPU_SHARE, n))


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or 'unknown'."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_calls(work, threads: int, seconds: float, first: int):
    """Call work(i) for i = 0, 1, 2, ... on `threads` threads until `seconds` of wall time
    have passed and every i < first has been called.  ctypes releases the GIL inside the
    oracle's C functions, so the threads run side by side.  Returns (calls finished, wall
    seconds, {i: work(i) for i < first})."""
    import itertools
    import threading
    ids, lock, firsts, done = itertools.count(), threading.Lock(), {}, [0]
    t0 = time.perf_counter()

    def loop():
        while True:
            with lock:
                i = next(ids)
            if i >= first and time.perf_counter() - t0 >= seconds:
                return
            r = work(i)
            with lock:
                done[0] += 1
                if i < first:
                    firsts[i] = r

    pool = [threading.Thread(target=loop) for _ in range(threads)]
    for t in pool:
        t.start()
    for t in pool:
        t.join()
    return done[0], time.perf_counter() - t0, firsts


def cpu_baseline(w, seconds: float, threads: int = 0):
    """The oracle (fp64 C), one sequence per call in batch order, starting over at the end of
    the batch: a single-threaded leg for a third of `seconds`, then `threads` threads (all the
    host threads, up to the share of one GPU) for about two thirds of `seconds` of CPU work,
    and never less than one pass over the batch.  Returns the baseline (the parallel leg's
    rate) and the parallel leg's first result for every sequence, for oracle_check."""
    import oracle
    oracle.build(force=False)
    threads = threads or host_threads()

    def work(i):
        return oracle.run_workload(w.subset([i % w.B]))

    n1, dt1, _ = run_calls(work, 1, seconds / 3, 0)
    n, dt, firsts = run_calls(work, threads, 2 * seconds / 3 / threads, w.B)
    per = 1 if w.mode == "sample" else w.K
    unit = "sampled tokens/s" if w.mode == "sample" else "verified draft positions/s"
    what = "rows" if w.mode == "sample" else "sequences"
    return {"value": n * per / dt, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": "%d %s (%.2f passes over the %d of the same batch) on %d threads in "
                      "%.2f s, one %s per oracle call, fp64 C" % (n, what, n / w.B, w.B, threads,
                                                                  dt, what[:-1]),
            "single_core_value": n1 * per / dt1,
            "single_core_sample": "%d %s in %.1f s on one thread" % (n1, what, dt1),
            "cpu_model": cpu_model()}, firsts


def oracle_check(w, gpu: dict, firsts: dict, early: bool = False) -> dict:
    """The GPU's outputs for the whole batch against the oracle's (firsts[b] = the oracle on
    sequence b alone), under the tests' parity rule: greedy ids, lengths and next proposals
    exact; sampling, contrastive and the sampler exact wherever the oracle's decision margins
    are >= 1e-6 (low-margin draws may take the id across the interval edge, low-margin accept
    tests need only a well-formed result); probabilities within 1e-5 relative."""
    import numpy as np
    import oracle
    low = oracle.LOW_MARGIN

    def close(g, o):
        g, o = np.asarray(g, np.float64), np.asarray(o, np.float64)
        return bool(np.all(np.abs(g - o) <= 1e-5 * np.maximum(np.abs(g), np.abs(o)) + 1e-30))

    exact = lowm = bad = 0
    for b in range(w.B):
        o = firsts[b]
        if w.mode == "sample":
            tg, to = int(gpu["out"][b, 0]), int(o.tokens[0])
            if o.margin[0] >= low:
                ok = tg == to
                exact += ok
            else:
                lowm += 1
                ok = tg in (to, int(o.alt_token[0]))
            ok = ok and close(gpu["draw_p"][b], o.probs[0])
        elif w.mode in ("greedy", "greedy_heads"):
            ok = (int(gpu["acc"][b]) == int(o.accepted_len[0])
                  and np.array_equal(gpu["out"][b], o.out_tokens[0]))
            if w.mode == "greedy_heads":
                ok = ok and np.array_equal(gpu["next"][b], o.next_proposals[0])
            exact += ok
        else:
            Lg, Lo = int(gpu["acc"][b]), int(o.accepted_len[0])
            tg, to = gpu["out"][b], o.out_tokens[0]
            ma, ms = float(o.margin_accept[0]), float(o.margin_sample[0])
            if Lo < 0:
                ok = Lg == -1 and bool(np.all(tg == -1))
            elif ma >= low and ms >= low:
                ok = Lg == Lo and np.array_equal(tg, to)
                exact += ok
            elif ma >= low:
                lowm += 1
                ok = (Lg == Lo and np.array_equal(tg[:Lo], to[:Lo])
                      and int(tg[Lo]) in (int(to[Lo]), int(o.alt_token[0]))
                      and bool(np.all(tg[Lo + 1:] == -1)))
            else:
                lowm += 1
                ok = (0 <= Lg <= w.K and np.array_equal(tg[:Lg], w.tokens[b, :Lg])
                      and 0 <= int(tg[Lg]) < w.V and bool(np.all(tg[Lg + 1:] == -1)))
            if ok and Lo >= 0 and w.K > 0:
                nj = min(Lg + 1, w.K) if early else w.K   # early exit: probabilities up to L
                ok = close(gpu["probs"][b, :nj], o.out_probs[0, :nj])
        bad += not ok
    return {"items": w.B, "bit_exact": int(exact), "low_margin": int(lowm),
            "mismatched": int(bad),
            "rule": "ids and lengths exact where the oracle's margins are >= 1e-6, "
                    "probabilities within 1e-5 relative"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed calls first: the GPU takes ~60 calls of this size (~12 ms) to reach "
                         "its steady clocks")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="c3")
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
    desc, kind, kname, traffic_file = WORKLOADS[args.workload]
    if args.workload == "cut":
        return bench_cut(args, desc, kind, kname)
    early = args.workload in ("early", "early_c5", "early_c4")
    base = {"early": "c3", "early_c5": "c5", "early_c4": "c4"}.get(args.workload, args.workload)
    w = (synth.CONFIGS.get(base) or synth.NEXT_CONFIGS[base])()
    B, K, V = w.B, w.K, w.V
    log("generated %s (seed %d); uploading %.3f GB of logits x2"
        % (desc, w.seed, w.logit_bytes / 1e9))

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")

    copies = []
    for _ in range(2):
        copies.append((up(w.target), up(w.draft) if w.draft is not None else None))
    toks = up(w.tokens)
    unif = up(w.uniforms) if w.uniforms is not None else None
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    probs = torch.empty((B, K, 2), dtype=torch.float32, device="cuda")
    H = w.meta.get("H", 1)
    nxt = torch.empty((B, max(H - 1, 1)), dtype=torch.int32, device="cuda")
    draw_p = torch.empty(B, dtype=torch.float32, device="cuda")
    ctx = sv.specverify_create(0, B, K, V)
    # The loops pass device addresses and the stream handle as plain integers, which the
    # binding forwards as they are: checking and converting tensors on every call costs the
    # Python side several microseconds, more than the GPU needs for the smallest workloads.
    sh = torch.cuda.current_stream().cuda_stream
    pcopies = [(a.data_ptr(), None if d is None else d.data_ptr()) for a, d in copies]
    p_toks, p_acc, p_out = toks.data_ptr(), acc.data_ptr(), out.data_ptr()
    p_unif = None if unif is None else unif.data_ptr()
    p_probs, p_nxt, p_draw = probs.data_ptr(), nxt.data_ptr(), draw_p.data_ptr()

    def step(i):
        tg, dr = pcopies[i & 1]
        if w.mode == synth.SAMPLE:
            sv.specverify_sample(ctx, sh, w.dtype, B, V, w.temperature, tg, p_unif, p_out, p_draw)
        elif w.mode == synth.GREEDY_HEADS:
            sv.specverify_run_greedy_heads(ctx, sh, w.dtype, B, K, H, V, tg, p_toks, p_acc, p_out,
                                           p_nxt)
        elif w.mode == synth.GREEDY:
            fn = sv.specverify_run_greedy_early_exit if early else sv.specverify_run_greedy
            fn(ctx, sh, w.dtype, B, K, V, tg, p_toks, p_acc, p_out)
        elif early:
            fn = (sv.specverify_run_sampling_early_exit if w.mode == synth.SAMPLING
                  else sv.specverify_run_contrastive_early_exit)
            fn(ctx, sh, w.dtype, B, K, V, w.temperature, tg, dr, p_toks, p_unif, p_acc, p_out,
               p_probs)
        elif w.mode == synth.CONTRASTIVE:
            sv.specverify_run_contrastive(ctx, sh, w.dtype, B, K, V, w.temperature, tg, dr,
                                          p_toks, p_unif, p_acc, p_out, p_probs)
        else:
            sv.specverify_run_sampling(ctx, sh, w.dtype, B, K, V, w.temperature, tg, dr,
                                       p_toks, p_unif, p_acc, p_out, p_probs)

    log("preheat: %d calls" % preheat(step, torch.cuda.synchronize, calls=PREHEAT_FIRST_CALLS))
    log("warmup %d" % args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    # the headline: wall clock over back-to-back calls with no events anywhere
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mean_L = float(acc.float().mean().item())
    kdur, kms, kn, stride, call_ms, bms, bn = timed_passes(args, step, ctx, kind, sv, torch)
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d bytes once for counter calibration" % src.nbytes)
    sv.specverify_destroy(ctx)
    gout = {"acc": acc.cpu().numpy(), "out": out.cpu().numpy(), "probs": probs.cpu().numpy(),
            "next": nxt.cpu().numpy(), "draw_p": draw_p.cpu().numpy()}

    ms_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = kms[kind] / max(kn[kind], 1)
    logit_bytes = w.logit_bytes                      # one read of every logit row
    if w.mode == synth.SAMPLE:
        positions = B / (ms_step * 1e-3)             # tokens drawn per second
        unit = "sampled tokens/s"
        kern_bytes = logit_bytes                     # the statistics read every row once
    elif w.mode == synth.GREEDY_HEADS:
        positions = B * K / (ms_step * 1e-3)
        unit = "verified draft positions/s"
        kern_bytes = logit_bytes // H                # head 0's rows
    elif early:
        positions = B * K / (ms_step * 1e-3)
        unit = "verified draft positions/s"
        # the prefix: positions 0-1 of the target and draft rows (sampling) or of the expert
        # and amateur rows (contrastive), positions 0-2 of the target rows (greedy)
        kern_bytes = (3 if w.mode == synth.GREEDY else 4) * B * V * w.target.itemsize
    else:
        positions = B * K / (ms_step * 1e-3)
        unit = "verified draft positions/s"
        kern_bytes = logit_bytes
    call_bytes = logit_bytes + w.tokens.nbytes + acc.nbytes + out.nbytes
    if w.uniforms is not None:
        call_bytes += w.uniforms.nbytes
    achieved = kern_bytes / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC if args.workload == "c3"
        else "%s + HBM GB/s vs peak, %s" % (unit, desc),
        "value": positions,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type of the dominant kernel (bfloat16 logits are widened to fp32);
        # the accept tests and the draw compute in fp64; config.logits is the input type
        "dtype": "f32",
        "data": "synthetic",
        "per_call_ms": {**percentiles(call_ms), "calls": len(call_ms),
                        "how": "HIP events (no system-scope fence) around each call in a pass of its own"},
        "config": {"workload": desc, "mode": w.mode, "B": B, "K": K, "V": V,
                   "logits": synth.DTYPE_NAMES[w.dtype], "temperature": w.temperature,
                   "seed": w.seed},
        "hbm_gbps_per_call": call_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac_of_peak_per_call": call_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(traffic_file),
                     "kernel": kname, "algorithmic_bytes": kern_bytes, "avg_ms": kern_ms,
                     **percentiles(kdur), "timed_launches": kn[kind],
                     "timing_stride": stride},
        "kernels_ms_per_step": {k: bms[k] / bn[k] for k in bms if bn[k]},
        "mean_accepted_len": mean_L if w.mode != synth.SAMPLE else None,
    }
    if args.cpu_seconds > 0:
        log("CPU oracle baseline (~%.0f s of CPU work)" % args.cpu_seconds)
        res["cpu_baseline"], firsts = cpu_baseline(w, args.cpu_seconds)
        res["oracle_check"] = oracle_check(w, gout, firsts, early)
        if res["oracle_check"]["mismatched"]:
            log("the GPU's outputs disagree with the oracle's: %s" % res["oracle_check"])
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def bench_cut(args, desc, kind, kname):
    """The alpha-quantile cut: P prompts x N scores per call; value = prompts cut per second."""
    import numpy as np
    import torch

    from rejection_sampling_verification_row_amd import binding as sv
    from rejection_sampling_verification_row_amd import synth

    w = synth.NEXT_CONFIGS["cut"]()
    P, N = w.P, w.N
    s = [torch.from_numpy(w.scores).to("cuda") for _ in range(2)]
    cut = torch.empty(P, dtype=torch.float32, device="cuda")
    keep = torch.empty((P, N), dtype=torch.uint8, device="cuda")
    n = torch.empty(P, dtype=torch.int32, device="cuda")
    ctx = sv.specverify_create(0, 1, 0, 1)
    # plain integer addresses and stream handle, as in the verify loops
    sh = torch.cuda.current_stream().cuda_stream
    ps = [x.data_ptr() for x in s]
    p_cut, p_keep, p_n = cut.data_ptr(), keep.data_ptr(), n.data_ptr()

    def step(i):
        sv.specverify_quantile_cut(ctx, sh, P, N, w.alpha, ps[i & 1], p_cut, p_keep, p_n)

    log("preheat: %d calls" % preheat(step, torch.cuda.synchronize, calls=PREHEAT_FIRST_CALLS))
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kdur, kms, kn, stride, call_ms, _, _ = timed_passes(args, step, ctx, kind, sv, torch)
    sv.specverify_destroy(ctx)
    gcut, gkeep, gn = cut.cpu().numpy(), keep.cpu().numpy(), n.cpu().numpy()
    ms_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = kms[kind] / max(kn[kind], 1)
    nbytes = P * N * 4 + P * N + P * 8               # scores in; keep bytes, cut and count out
    res = {
        "metric": "prompts cut/s, " + desc, "value": P / (ms_step * 1e-3),
        "unit": "prompts/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "per_call_ms": {**percentiles(call_ms), "calls": len(call_ms),
                        "how": "HIP events (no system-scope fence) around each call in a pass of its own"},
        "config": {"workload": desc, "P": P, "N": N, "alpha": w.alpha, "seed": w.seed},
        "roofline": {"bound": "hbm", "achieved": nbytes / (kern_ms * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": kname, "algorithmic_bytes": nbytes, "avg_ms": kern_ms,
                     **percentiles(kdur), "timed_launches": kn[kind],
                     "timing_stride": stride,
                     "note": "latency-bound: one workgroup per prompt, four selection passes"},
        "mean_kept": float(n.float().mean().item()),
    }
    if args.cpu_seconds > 0:
        import numpy as np
        import oracle
        oracle.build(force=False)
        threads = host_threads()

        def work(i):
            return oracle.quantile_cut(P, N, w.alpha, w.scores)

        n1, dt1, _ = run_calls(work, 1, args.cpu_seconds / 3, 0)
        done, dt, firsts = run_calls(work, threads, 2 * args.cpu_seconds / 3 / threads, 1)
        res["cpu_baseline"] = {"value": done * P / dt, "unit": "prompts/s", "cores": threads,
                               "kind": "oracle",
                               "sample": "the whole batch %d times on %d threads in %.2f s, "
                                         "C" % (done, threads, dt),
                               "single_core_value": n1 * P / dt1,
                               "single_core_sample": "the whole batch %d times in %.1f s on "
                                                     "one thread" % (n1, dt1),
                               "cpu_model": cpu_model()}
        o = firsts[0]
        # the cut compares as a float: the oracle's sort may return either zero of a tie
        # between -0 and +0, the radix selection on order keys takes -0 first
        same = ((o.r_cut == gcut) & (o.keep == gkeep.astype(bool)).all(axis=1)
                & (o.n_keep == gn))
        res["oracle_check"] = {"items": P, "bit_exact": int(same.sum()), "low_margin": 0,
                               "mismatched": int(P - same.sum()),
                               "rule": "cut value (as a float, -0 == +0), keep mask and count "
                                       "exact"}
        if res["oracle_check"]["mismatched"]:
            log("the GPU's outputs disagree with the oracle's: %s" % res["oracle_check"])
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
