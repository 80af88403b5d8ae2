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
    paths         the other scoring paths (and the seeded sampler, the L1 loss,
                  the support VJP), each on its own workload: 20 warmup calls,
                  then the median and IQR of 100 timed calls, each after an
                  Infinity-Cache flush, vs HBM peak (8 TB/s) or the MFMA peak
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
SAMPLE_SEED = 20260101  # seed of the transforms workload's sampled targets


def _bf16(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _event_times(vsa, fn, steps, warmup, flush=None):
    """Per-call durations (ms): the whole call (HIP events on torch's current
    stream, which the call launches on), then, in a second loop of as many
    calls, its main sweep kernel(s) alone (the library's own event bracket,
    recorded on the same stream).  The loops are separate because the
    library's two events add about 9 us to the whole-call bracket."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    calls, sweeps = [], []
    for timed in (False, True):
        if timed:
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
                if timed:
                    sweeps.append(vsa.sweep_timer_ms())
                else:
                    calls.append(s.elapsed_time(e))
        finally:
            if timed:
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


def _clocks():
    """The shader and memory clock levels the driver reports right now (sysfs
    pp_dpm_sclk / pp_dpm_mclk, the line marked '*'), or None where unreadable."""
    import glob
    out = {}
    for name in ("sclk", "mclk"):
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{name}")):
            try:
                cur = [ln for ln in open(path).read().splitlines() if ln.strip().endswith("*")]
            except OSError:
                continue
            if cur:
                out[name] = cur[0].split(":", 1)[-1].replace("*", "").strip()
                break
    return out or None


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
    clocks = _clocks()  # read while the part is still at its working clocks
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
        "clocks_after_timed_region": clocks,
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


def bench_backward(vsa, dev, c, steps, warmup):
    """The VJP of the fused workload (same inputs as the headline): recomputed
    logits, their gradient, d_hidden and d_weight; three 2 T H V products."""
    import torch
    T, H, V = c["T"], c["H"], c["V"]
    hid, w, y = _bf16(c["hidden"], dev), _bf16(c["weight"], dev), _dev(c["targets"], dev)
    fw = vsa.score_full(y, hidden=hid, weight=w)
    rng = np.random.default_rng(44)
    a = _dev(rng.normal(0, 1, T).astype(np.float32), dev)
    b = _dev(rng.normal(0, 1, T).astype(np.float32), dev)
    # the whole vocabulary as one chunk: one d_hidden product with K = V (no
    # accumulate passes); its workspace is 3 x T x V bf16 (3.7 GB here)
    chunk = V
    o = vsa.score_full_backward(y, fw["lse"], fw["entropy"], hidden=hid, weight=w, grad_logprob=a, grad_entropy=b,
                                vocab_chunk=chunk)
    wsp = torch.empty(vsa.workspace_bytes("score_full_backward", hidden=hid, weight=w, width=chunk),
                      dtype=torch.uint8, device=dev)
    ev, sw = _event_times(vsa, lambda: vsa.score_full_backward(y, fw["lse"], fw["entropy"], hidden=hid, weight=w,
                                                               grad_logprob=a, grad_entropy=b, vocab_chunk=chunk,
                                                               out=o, workspace=wsp), steps, warmup)
    med, iqr = _median_iqr(ev)
    flops = 3 * 2.0 * T * H * V
    return {"T": T, "H": H, "V": V, "vocab_chunk": chunk, "workspace_bytes": int(wsp.numel()),
            "ms_median": round(med, 4), "ms_iqr": round(iqr, 4),
            "tokens_per_s": round(T / (med * 1e-3), 1), "flop_per_call": flops,
            "tflops": round(flops / (med * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (med * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def _oracle_threads():
    """(threads the oracle runs on, CPUs in this process's affinity set): every
    CPU the process may use, at most 16 (one GPU's share of the host)."""
    n_aff = len(os.sched_getaffinity(0))
    return max(1, min(16, n_aff)), n_aff


def _timed_oracle(fn, n_rows, budget_s, block=16):
    """Run ``fn(rows)`` over consecutive row blocks on a pool of threads (numpy
    releases the GIL in the oracle's array work) until every row is done or the
    time budget is spent; BLAS threads are set to the same count.  Returns
    (rows done, seconds, threads, affinity CPUs)."""
    from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait
    import threadpoolctl
    threads, n_aff = _oracle_threads()
    blocks = [np.arange(r0, min(n_rows, r0 + block)) for r0 in range(0, n_rows, block)]
    done = 0
    with threadpoolctl.threadpool_limits(threads):
        t0 = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            pending = set()
            nxt = 0
            while nxt < len(blocks) or pending:
                while nxt < len(blocks) and len(pending) < threads and time.perf_counter() - t0 < budget_s:
                    pending.add(ex.submit(lambda b=blocks[nxt]: (fn(b), len(b))[1]))
                    nxt += 1
                if not pending:
                    break
                fin, pending = wait(pending, return_when=FIRST_COMPLETED)
                done += sum(f.result() for f in fin)
        el = time.perf_counter() - t0
    return done, el, threads, n_aff


def _cpu_entry(done, el, threads, n_aff, what):
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": int(threads), "affinity_cpus": int(n_aff),
            "kind": "oracle", "sample": f"{what}: {done} rows in {el:.1f} s (numpy float64, {threads} threads)"}


def cpu_baseline(c, budget_s=15.0):
    """fp64 oracle on the first rows of the fused workload: blocks of 32 rows in
    order (the projection's matmul uses every BLAS thread) until the budget is spent."""
    import threadpoolctl
    import oracle
    threads, n_aff = _oracle_threads()
    rows_done = 0
    with threadpoolctl.threadpool_limits(threads):
        t0 = time.perf_counter()
        while True:
            rows = np.arange(rows_done, rows_done + 32)
            x = oracle.logits_from_hidden(c["hidden"], "bf16", c["weight"], rows=rows)
            oracle.score_full(x, 1.0, c["targets"][rows])
            rows_done += 32
            if time.perf_counter() - t0 > budget_s or rows_done >= c["T"]:
                break
        el = time.perf_counter() - t0
    return _cpu_entry(rows_done, el, threads, n_aff,
                      f"first rows of fused_full of {c['T']} (projection + LSE/logprob/entropy)")


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


def bench_paths(vsa, dev, steps, warmup, cpu=True, cpu_budget_s=8.0):
    """The other scoring paths, each on its own workload.  A 512 MiB write
    before every timed call leaves none of its inputs in the Infinity Cache.
    Outputs and workspace are allocated once, so the timed calls allocate
    nothing.  Bytes are algorithmic: every input element read once, every
    output written once.  With ``cpu``, each path also times the fp64 oracle
    on the same inputs (all rows, or as many as the budget allows)."""
    import torch
    import workloads
    flush = _flusher(dev)
    res = {}
    if cpu:
        import oracle

    # logits-input full-vocabulary scoring: T=512, V=151,936 bf16, per-row temperature
    c = workloads.make(2)
    T, V = c["T"], c["V"]
    lg, y, tau = _bf16(c["logits"], dev), _dev(c["targets"], dev), _dev(c["temperature"], dev)
    o = vsa.score_full(y, logits=lg, temperature=tau)
    ev, sw = _event_times(vsa, lambda: vsa.score_full(y, logits=lg, temperature=tau, out=o), steps, warmup, flush)
    byts = T * V * 2 + T * (4 + 8) + T * (3 * 4 + 1)  # logits, tau, targets in; lse, logprob, entropy, status out
    res["logits_full"] = _path_entry(T, ev, sw, byts, byts, V=V, inputs_sha256=workloads.digest(c))
    if cpu:
        res["logits_full"]["cpu_baseline"] = _cpu_entry(*_timed_oracle(
            lambda r: oracle.score_full(oracle.logits_from_logits(c["logits"], "bf16", rows=r), c["temperature"][r],
                                        c["targets"][r]), T, cpu_budget_s), "logits_full rows (LSE/logprob/entropy)")
    del lg, o

    # recorded support through selected projections: T=2048, H=7168, V=129,280, width 64
    c = workloads.make(3)
    T, H, V = c["T"], c["H"], c["V"]
    hid, w = _bf16(c["hidden"], dev), _bf16(c["weight"], dev)
    y, ids = _dev(c["targets"], dev), _dev(c["support_ids"], dev)
    o = vsa.score_support_ids(y, ids, hidden=hid, weight=w)
    wsp = torch.empty(max(1, vsa.workspace_bytes("score_support_ids", hidden=hid, weight=w, width=ids.shape[1])),
                      dtype=torch.uint8, device=dev)
    ev, sw = _event_times(vsa, lambda: vsa.score_support_ids(y, ids, hidden=hid, weight=w, out=o, workspace=wsp),
                          steps, warmup, flush)
    sup = c["support_ids"][c["support_ids"] >= 0]
    uniq = int(np.unique(sup).size)
    # unique basis: each distinct W row and each hidden row read once
    byts = uniq * H * 2 + T * H * 2 + c["support_ids"].nbytes + T * (8 + 2 * 4 + 1)
    res["support_replay"] = _path_entry(T, ev, sw, byts, byts, H=H, V=V, width=int(c["support_ids"].shape[1]),
                                        pairs=int(sup.size), unique_rows=uniq, inputs_sha256=workloads.digest(c),
                                        bytes_pairs_basis=int(sup.size * H * 2 + T * H * 2 + c["support_ids"].nbytes))
    if cpu:
        def support_rows(r):
            def fn(t, cols):
                return oracle.logits_from_hidden(c["hidden"], "bf16", c["weight"], rows=[r[t]], cols=cols)[0]
            return oracle.score_support(fn, V, c["support_ids"][r], 1.0, c["targets"][r])
        res["support_replay"]["cpu_baseline"] = _cpu_entry(*_timed_oracle(support_rows, T, cpu_budget_s),
                                                           "support_replay rows (selected projections + scores)")
    # the VJP of the same scores (both gradients, upstream gradients ~N(0,1)); the dense fp32
    # weight gradient is written whole (zeros for the ids in no support)
    rng = np.random.default_rng(45)
    a_np, b_np = rng.normal(0, 1, T).astype(np.float32), rng.normal(0, 1, T).astype(np.float32)
    ga, gb = _dev(a_np, dev), _dev(b_np, dev)
    o = vsa.score_support_backward(y, ids, hidden=hid, weight=w, grad_logprob=ga, grad_entropy=gb)
    wsp = torch.empty(max(1, vsa.workspace_bytes("score_support_backward", hidden=hid, weight=w,
                                                 width=ids.shape[1])), dtype=torch.uint8, device=dev)
    ev, sw = _event_times(vsa, lambda: vsa.score_support_backward(y, ids, hidden=hid, weight=w, grad_logprob=ga,
                                                                  grad_entropy=gb, out=o, workspace=wsp),
                          steps, warmup, flush)
    # distinct W rows read twice (logits, then d_hidden), hidden read twice (the row, then d_weight's
    # gathers), ids, the two dense fp32 gradients written once
    byts = 2 * uniq * H * 2 + 2 * T * H * 2 + c["support_ids"].nbytes + T * (8 + 2 * 4) + (T + V) * H * 4
    res["support_backward"] = _path_entry(T, ev, sw, byts, byts, H=H, V=V, width=int(c["support_ids"].shape[1]),
                                          unique_rows=uniq)
    if cpu:
        def support_bwd_rows(r):
            ids_r = c["support_ids"][r]
            return oracle.score_support_vjp(c["hidden"][r], "bf16", c["weight"], ids_r, 1.0, c["targets"][r],
                                            a_np[r], b_np[r], weight_rows=np.unique(ids_r[ids_r >= 0]))
        res["support_backward"]["cpu_baseline"] = _cpu_entry(*_timed_oracle(support_bwd_rows, T, cpu_budget_s),
                                                             "support_replay rows (support logits, dX, d_hidden, "
                                                             "d_weight contributions)")
    del hid, w, o, wsp

    # sampling transforms and draft/target L1: T=2048, V=151,936 bf16
    c = workloads.make(5)
    T, V = c["T"], c["V"]
    lg, dr = _bf16(c["logits"], dev), _bf16(c["draft"], dev)
    tk, tp, mp, tau = (_dev(c["top_k"], dev), _dev(c["top_p"], dev), _dev(c["min_p"], dev),
                       _dev(c["temperature"], dev))
    # the seeded Gumbel draw from each row's transformed support: the sampled in-support
    # target of the transforms workload (drawn once, outside the timed calls), and a path of its own
    smp = vsa.sample_transforms(lg, tk, tp, mp, temperature=tau, seed=SAMPLE_SEED)
    y = smp["sampled"].clone()
    wsp = torch.empty(max(1, vsa.workspace_bytes("sample_transforms", logits=lg)), dtype=torch.uint8, device=dev)
    ev, sw = _event_times(vsa, lambda: vsa.sample_transforms(lg, tk, tp, mp, temperature=tau, seed=SAMPLE_SEED,
                                                             out=smp, workspace=wsp), steps, warmup, flush)
    byts = T * V * 2 + T * (4 * 4 + 8 + 4 + 4 + 4 + 1)
    res["sample_transforms"] = _path_entry(T, ev, sw, byts, byts, V=V, seed=SAMPLE_SEED)
    del wsp
    o = vsa.score_transforms(y, lg, tk, tp, mp, temperature=tau, cap=64)
    wsp = torch.empty(max(1, vsa.workspace_bytes("score_transforms", logits=lg)), dtype=torch.uint8, device=dev)
    ev, sw = _event_times(vsa, lambda: vsa.score_transforms(y, lg, tk, tp, mp, temperature=tau, cap=64, out=o,
                                                            workspace=wsp), steps, warmup, flush)
    byts = T * V * 2 + T * (4 * 4 + 8) + T * (4 * 4 + 4 + 1 + 64 * 8 + 4)
    res["transforms"] = _path_entry(T, ev, sw, byts, byts, V=V, support_ids_cap=64,
                                    inputs_sha256=workloads.digest(c))
    if cpu:
        # (the oracle takes its own inputs: the workload's row-argmax targets, which lie in every
        # support; a target changes no step of the program's cost)
        res["transforms"]["cpu_baseline"] = _cpu_entry(*_timed_oracle(
            lambda r: oracle.score_transforms(oracle.logits_from_logits(c["logits"], "bf16", rows=r),
                                              c["temperature"][r], c["top_k"][r], c["top_p"][r], c["min_p"][r],
                                              c["targets"][r], cap=64), T, cpu_budget_s),
            "transforms_l1 rows (sort, top-k/top-p/min-p, support scores)")
        res["sample_transforms"]["cpu_baseline"] = _cpu_entry(*_timed_oracle(
            lambda r: oracle.sampling.sample_transforms(oracle.logits_from_logits(c["logits"], "bf16", rows=r),
                                                        c["temperature"][r], c["top_k"][r], c["top_p"][r],
                                                        c["min_p"][r], seed=SAMPLE_SEED, rows=r), T, cpu_budget_s),
            "transforms_l1 rows (support, Philox numbers, Gumbel-max draw)")
    del o, wsp
    o = vsa.l1_distance(lg, dr)
    ev, sw = _event_times(vsa, lambda: vsa.l1_distance(lg, dr, out=o), steps, warmup, flush)
    byts = 2 * T * V * 2 + T * 8
    res["l1_distance"] = _path_entry(T, ev, sw, byts, byts, V=V)
    if cpu:
        res["l1_distance"]["cpu_baseline"] = _cpu_entry(*_timed_oracle(
            lambda r: oracle.l1_distance(oracle.logits_from_logits(c["logits"], "bf16", rows=r),
                                         oracle.logits_from_logits(c["draft"], "bf16", rows=r)), T, cpu_budget_s),
            "transforms_l1 rows (two softmaxes, L1, accept_rate)")
    del o
    # the weighted L1 distillation loss and its draft-logit gradient (bf16): the page's loss-path
    # shapes (V = 151,936 at 128 and 512 rows) and the full draft workload (2048 rows)
    for T_l in (128, 512, T):
        tl, dl = lg[:T_l], dr[:T_l]
        wl = torch.ones(T_l, dtype=torch.float32, device=dev)
        o = vsa.l1_loss(tl, dl, weights=wl)
        wsp = torch.empty(max(1, vsa.workspace_bytes("l1_loss", logits=tl)), dtype=torch.uint8, device=dev)
        ev, sw = _event_times(vsa, lambda: vsa.l1_loss(tl, dl, weights=wl, out=o, workspace=wsp), steps, warmup, flush)
        # reads: both rows twice (distance pass), both again (gradient pass); writes: the bf16 gradient
        byts = 3 * 2 * T_l * V * 2 + T_l * V * 2 + T_l * (4 + 8) + 12
        res[f"l1_loss_T{T_l}"] = _path_entry(T_l, ev, sw, byts, byts, V=V, grad_dtype="bf16",
                                             context_rtx4090_loss_path_ms={128: 2.531, 512: 11.593}.get(T_l))
        del o, wsp
    del lg, dr

    # the transform program on a hidden/weight source: T=2048, H=4096, V=151,936 (grid inputs
    # whose fp32 sums are exact; the timing does not depend on the values)
    c = workloads.make(6)
    T, H, V = c["T"], c["H"], c["V"]
    hid, w = _bf16(c["hidden"], dev), _bf16(c["weight"], dev)
    tk, tp, mp, tau = (_dev(c["top_k"], dev), _dev(c["top_p"], dev), _dev(c["min_p"], dev),
                       _dev(c["temperature"], dev))
    y = torch.zeros(T, dtype=torch.int64, device=dev)  # (the support and its scores cost the same for any target)
    o = vsa.score_transforms(y, None, tk, tp, mp, hidden=hid, weight=w, temperature=tau, cap=64)
    wsp = torch.empty(max(1, vsa.workspace_bytes("score_transforms", hidden=hid, weight=w)), dtype=torch.uint8,
                      device=dev)
    ev, sw = _event_times(vsa, lambda: vsa.score_transforms(y, None, tk, tp, mp, hidden=hid, weight=w, temperature=tau,
                                                            cap=64, out=o, workspace=wsp), steps, warmup, flush)
    med, iqr = _median_iqr(ev)
    flops = 2.0 * T * H * V
    res["transforms_hidden"] = {
        "T": T, "H": H, "V": V, "support_ids_cap": 64, "ms_median": round(med, 4), "ms_iqr": round(iqr, 4),
        "tokens_per_s": round(T / (med * 1e-3), 1), "flop_per_call": flops,
        "tflops": round(flops / (med * 1e-3) / 1e12, 1),
        "mfma_frac": round(flops / (med * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernel_ms_mean": round(statistics.mean(sw), 4), "workspace_bytes": int(wsp.numel()),
        "inputs_sha256": workloads.digest(c)}
    if cpu:
        res["transforms_hidden"]["cpu_baseline"] = _cpu_entry(*_timed_oracle(
            lambda r: oracle.score_transforms(
                oracle.widen_bf16(oracle.bf16_logits_from_hidden(c["hidden"], "bf16", c["weight"], rows=r)),
                c["temperature"][r], c["top_k"][r], c["top_p"][r], c["min_p"][r], np.zeros(r.size, np.int64),
                cap=64), T, cpu_budget_s),
            "transforms_hidden rows (projection, bf16 rounding, sort, top-k/top-p/min-p, support scores)")
    del hid, w, o, wsp
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
    # the paths' timing protocol: 20 warmup calls, then the median and IQR of 100 timed calls
    ap.add_argument("--path-steps", type=int, default=100)
    ap.add_argument("--path-warmup", type=int, default=20)
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
    import workloads
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
        "clocks_after_timed_region": fused["clocks_after_timed_region"],
        "inputs_sha256": {"fused_full": workloads.digest(c)},
        "roofline": fused["roofline"],
    }
    if args.paths == "all":
        print("bench: fused backward", file=sys.stderr, flush=True)
        out["backward"] = bench_backward(vsa, dev, c, max(3, min(args.steps, 10)), 1)
        print("bench: secondary paths", file=sys.stderr, flush=True)
        out["paths"] = bench_paths(vsa, dev, args.path_steps, args.path_warmup, cpu=args.cpu_baseline == "on")
    if probe is not None:
        out["copy_probe"] = probe
    if args.cpu_baseline == "on":
        print("bench: cpu oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(c)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
