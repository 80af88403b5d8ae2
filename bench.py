#!/usr/bin/env python3
"""Benchmark: scored tokens/s of the fused LM-head scoring op on one MI355X.

Headline workload (one "step" = one vs_score_full call over the batch):
    fused_full: T=4096 tokens, H=4096, V=151,936, bf16 hidden and W_vocab,
    fp32 accumulation, vocabulary merge chunk 8192; outputs LSE, selected
    logprob and full-vocabulary entropy without materialising logits.
Inputs are seeded synthetic (workloads.make(4)) and resident in HBM before
timing starts.

Prints ONE JSON line.  Besides the contract fields it carries
    roofline      the fused sweep kernel vs bf16 dense MFMA peak (2.5 PFLOP/s)
    cpu_baseline  the fp64 CPU oracle on a bounded sample of the same rows
    paths         the other scoring paths, each on its own workload, with an
                  Infinity-Cache flush between timed calls, vs HBM peak (8 TB/s)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
METRIC = "scored tokens/sec at V=151,936 (fused LM head); % MFMA / HBM peak"


def _bf16(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _event_times(vsa, fn, steps, warmup, flush=None):
    """Per-call durations (ms): the whole call (HIP events on torch's current
    stream, which the call launches on) and its main sweep kernel(s) alone
    (the library's own event bracket, recorded on the same stream)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    calls, sweeps = [], []
    vsa.sweep_timer(True)
    try:
        for _ in range(steps):
            if flush is not None:
                flush()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            e.synchronize()
            calls.append(s.elapsed_time(e))
            sweeps.append(vsa.sweep_timer_ms())
    finally:
        vsa.sweep_timer(False)
    return calls, sweeps


# Kernel sources whose HBM counters are recorded in profiles/: a summary's
# figures stand only while these files are unchanged.
_SWEEP_SOURCES = ("logprob_entropy_sampling_amd/csrc/k_fused.hip", "logprob_entropy_sampling_amd/csrc/common.h",
                  "logprob_entropy_sampling_amd/csrc/launch.h")
TRAFFIC_SUMMARY = "profiles/fused_full_hbm_traffic.md"


def sweep_source_sha256() -> str:
    h = hashlib.sha256()
    for rel in _SWEEP_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _recorded_traffic():
    """(bytes per launch, note) from the committed counter summary; None when the
    summary is missing or was taken on kernel sources that have changed since."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None, "no counter summary"
    text = open(path).read()
    m_b = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    m_h = re.search(r"^kernel_source_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not (m_b and m_h):
        return None, "counter summary unreadable"
    if m_h.group(1) != sweep_source_sha256():
        return None, "kernel changed since the counters were taken"
    return int(m_b.group(1)), TRAFFIC_SUMMARY


def _flusher(dev):
    """Writes 512 MiB so the 256 MiB Infinity Cache holds none of the next call's inputs."""
    import torch
    buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def flush():
        buf.fill_(1)
    return flush


def _median_iqr(ts):
    q = np.percentile(ts, [25, 50, 75])
    return float(q[1]), float(q[2] - q[0])


def bench_fused(vsa, dev, steps, warmup):
    import torch
    import workloads
    c = workloads.make(4)
    T, H, V = c["T"], c["H"], c["V"]
    hid, w, y = _bf16(c["hidden"], dev), _bf16(c["weight"], dev), _dev(c["targets"], dev)

    def step():
        return vsa.score_full(y, hidden=hid, weight=w, vocab_chunk=8192)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the contract's timed region: exactly `steps` calls, synchronised on both sides
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-call event timing of the same op (its kernels run on this stream)
    ev, sw = _event_times(vsa, step, steps, 0)
    med, iqr = _median_iqr(ev)
    flops = 2.0 * T * H * V
    sweep_ms = statistics.mean(sw)
    achieved = flops / (sweep_ms * 1e-3) / 1e12
    traffic, traffic_src = _recorded_traffic()
    return c, {
        "value": T * steps / wall,
        "ms_per_step": wall * 1e3 / steps,
        "event_ms_median": med,
        "event_ms_iqr": iqr,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "traffic_source": traffic_src,
            "kernel": "fused_partials_wide_kernel<true, 0> (projection + per-tile softmax statistics)",
            "kernel_ms_mean": round(sweep_ms, 4),
            "flop_per_launch": flops,
            "algorithmic_bytes_per_launch": (T * H + V * H) * 2 + T * ((V + 255) // 256) * 16 + T * 4,
        },
    }


def cpu_baseline(c, budget_s=15.0):
    """fp64 oracle on the first rows of the same workload, batches of 32 rows until the budget is spent."""
    import threadpoolctl
    import oracle
    threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) \
        if threadpoolctl.threadpool_info() else 1
    rows_done = 0
    t0 = time.perf_counter()
    while True:
        rows = np.arange(rows_done, rows_done + 32)
        x = oracle.logits_from_hidden(c["hidden"], "bf16", c["weight"], rows=rows)
        oracle.score_full(x, 1.0, c["targets"][rows])
        rows_done += 32
        if time.perf_counter() - t0 > budget_s or rows_done >= c["T"]:
            break
    el = time.perf_counter() - t0
    return {"value": round(rows_done / el, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {rows_done} of {c['T']} rows of fused_full (projection + LSE/logprob/entropy, "
                      f"numpy float64), {el:.1f} s"}


def _path_entry(T, ev, sw, call_bytes, sweep_bytes, **extra):
    """One secondary path: whole-call and sweep-kernel times, algorithmic bytes, fraction of HBM peak."""
    med, iqr = _median_iqr(ev)
    kms = statistics.mean(sw)
    e = {"T": T, **extra, "ms_median": round(med, 5), "ms_iqr": round(iqr, 5), "tokens_per_s": round(T / (med * 1e-3), 1),
         "bytes": int(call_bytes), "hbm_GBs": round(call_bytes / (med * 1e-3) / 1e9, 1),
         "hbm_frac": round(call_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
         "kernel_ms_mean": round(kms, 5), "kernel_bytes": int(sweep_bytes),
         "kernel_hbm_GBs": round(sweep_bytes / (kms * 1e-3) / 1e9, 1),
         "kernel_hbm_frac": round(sweep_bytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return e


def bench_paths(vsa, dev, steps, warmup):
    """The other scoring paths, each on its own workload.  A 512 MiB write
    before every timed call leaves none of its inputs in the Infinity Cache.
    Bytes are algorithmic: every input element read once, every output written once."""
    import torch
    import workloads
    flush = _flusher(dev)
    res = {}

    # logits-input full-vocabulary scoring: T=512, V=151,936 bf16, per-row temperature
    c = workloads.make(2)
    T, V = c["T"], c["V"]
    lg, y, tau = _bf16(c["logits"], dev), _dev(c["targets"], dev), _dev(c["temperature"], dev)
    ev, sw = _event_times(vsa, lambda: vsa.score_full(y, logits=lg, temperature=tau), steps, warmup, flush)
    byts = T * V * 2 + T * (4 + 8) + T * (3 * 4 + 1)  # logits, tau, targets in; lse, logprob, entropy, status out
    res["logits_full"] = _path_entry(T, ev, sw, byts, byts, V=V)
    del lg

    # recorded support through selected projections: T=2048, H=7168, V=129,280, width 64
    c = workloads.make(3)
    T, H, V = c["T"], c["H"], c["V"]
    hid, w = _bf16(c["hidden"], dev), _bf16(c["weight"], dev)
    y, ids = _dev(c["targets"], dev), _dev(c["support_ids"], dev)
    ev, sw = _event_times(vsa, lambda: vsa.score_support_ids(y, ids, hidden=hid, weight=w), steps, warmup, flush)
    sup = c["support_ids"][c["support_ids"] >= 0]
    uniq = int(np.unique(sup).size)
    # unique basis: each distinct W row and each hidden row read once
    byts = uniq * H * 2 + T * H * 2 + c["support_ids"].nbytes + T * (8 + 2 * 4 + 1)
    res["support_replay"] = _path_entry(T, ev, sw, byts, byts, H=H, V=V, width=int(c["support_ids"].shape[1]),
                                        pairs=int(sup.size), unique_rows=uniq,
                                        bytes_pairs_basis=int(sup.size * H * 2 + T * H * 2 + c["support_ids"].nbytes))
    del hid, w

    # sampling transforms and draft/target L1: T=2048, V=151,936 bf16
    c = workloads.make(5)
    T, V = c["T"], c["V"]
    lg, dr = _bf16(c["logits"], dev), _bf16(c["draft"], dev)
    y = _dev(c["targets"], dev)
    tk, tp, mp, tau = (_dev(c["top_k"], dev), _dev(c["top_p"], dev), _dev(c["min_p"], dev),
                       _dev(c["temperature"], dev))
    ev, sw = _event_times(vsa, lambda: vsa.score_transforms(y, lg, tk, tp, mp, temperature=tau, cap=64), steps,
                          warmup, flush)
    byts = T * V * 2 + T * (4 * 4 + 8) + T * (4 * 4 + 4 + 1 + 64 * 8 + 4)
    res["transforms"] = _path_entry(T, ev, sw, byts, byts, V=V, support_ids_cap=64)
    ev, sw = _event_times(vsa, lambda: vsa.l1_distance(lg, dr), steps, warmup, flush)
    byts = 2 * T * V * 2 + T * 8
    res["l1_distance"] = _path_entry(T, ev, sw, byts, byts, V=V)
    torch.cuda.synchronize()
    return res


def copy_probe(dev, mib, steps):
    """A plain elementwise copy (out = in * 1, fp32) of `mib` MiB, run `steps`
    times: a kernel of known traffic (mib MiB read, mib MiB written) against
    which the HBM byte counters are scaled.  Also reports the copy's own
    read+write bandwidth, the achievable-bandwidth context for the HBM paths."""
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ts = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.mul(src, 1.0, out=dst)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    del src, dst
    best = min(ts)
    return {"mib": mib, "ms_best": round(best, 4), "read_plus_write_GBs": round(2 * (mib << 20) / (best * 1e-3) / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--paths", choices=["all", "none"], default="all")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first run a plain fp32 copy of MIB MiB --steps times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the op is row-local; see the sharding notes); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import logprob_entropy_sampling_amd as vsa
    vsa.lib()
    dev = torch.device("cuda:0")
    probe = None
    if args.copy_probe:
        print(f"bench: copy probe {args.copy_probe} MiB x {args.steps}", file=sys.stderr, flush=True)
        probe = copy_probe(dev, args.copy_probe, args.steps)
    print("bench: fused_full T=4096 H=4096 V=151936", file=sys.stderr, flush=True)
    c, fused = bench_fused(vsa, dev, args.steps, args.warmup)
    out = {
        "metric": METRIC,
        "value": round(fused["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(fused["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init bf16 hidden and W_vocab)",
        "config": {"workload": "fused_full", "T": 4096, "H": 4096, "V": 151936, "vocab_chunk": 8192,
                   "parallelism": "single-gpu"},
        "event_ms_median": round(fused["event_ms_median"], 4),
        "event_ms_iqr": round(fused["event_ms_iqr"], 4),
        "roofline": fused["roofline"],
    }
    if args.paths == "all":
        print("bench: secondary paths", file=sys.stderr, flush=True)
        out["paths"] = bench_paths(vsa, dev, max(5, min(args.steps, 20)), 2)
    if probe is not None:
        out["copy_probe"] = probe
    if args.cpu_baseline == "on":
        print("bench: cpu oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(c)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
