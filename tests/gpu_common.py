"""Helpers shared by the GPU parity tests (no scoring arithmetic here)."""

import sys

import numpy as np
import torch

# logprob / entropy / L1 tolerance for bf16 inputs with fp32 accumulation:
# |gpu - oracle| <= ATOL + RTOL * |oracle|
ATOL = 2e-3
RTOL = 1e-3


def dev():
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_tensor(bits, device=None):
    """uint16 bf16 patterns (numpy) -> torch.bfloat16 on the GPU."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return torch.from_numpy(b.view(np.int16)).to(device or dev()).view(torch.bfloat16)


def to_dev(a, device=None):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device or dev())


def assert_close(name, got, ref, atol=ATOL, rtol=RTOL, rows=None):
    """Elementwise tolerance; NaN, -inf and +inf must sit in the same places."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if rows is not None:
        got = got[rows]
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"{name}: NaN mismatch at {np.nonzero(nan_g != nan_r)[0][:10]}"
    for inf_test, what in ((np.isneginf, "-inf"), (np.isposinf, "+inf")):
        g_i, r_i = inf_test(got), inf_test(ref)
        assert np.array_equal(g_i, r_i), f"{name}: {what} mismatch at {np.nonzero(g_i != r_i)[0][:10]}"
    fin = np.isfinite(ref)
    assert np.isfinite(got[fin]).all(), f"{name}: non-finite where the oracle is finite"
    err = np.abs(got[fin] - ref[fin])
    bound = atol + rtol * np.abs(ref[fin])
    if err.size:
        worst = int(np.argmax(err - bound))
        ok = bool((err <= bound).all())
        say(f"  {name}: max abs err {err.max():.3e}, max rel err "
            f"{(err / np.maximum(np.abs(ref[fin]), 1e-30)).max():.3e} over {err.size} values")
        assert ok, (f"{name}: |err| {err[worst]:.4e} > bound {bound[worst]:.4e} at finite index {worst} "
                    f"(gpu {got[fin][worst]!r}, oracle {ref[fin][worst]!r})")


def host_threads():
    """CPU threads this process may use (the box's share, capped at 16)."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_by_rows(fn, n_rows, block=32):
    """Run ``fn(rows) -> dict of per-row arrays`` over row blocks in a thread
    pool and concatenate the results in row order.  numpy releases the GIL in
    the oracle's sorts, exponentials and sums, so threads share the work."""
    from concurrent.futures import ThreadPoolExecutor
    blocks = [np.arange(r0, min(n_rows, r0 + block)) for r0 in range(0, n_rows, block)]
    with ThreadPoolExecutor(host_threads()) as ex:
        parts = list(ex.map(fn, blocks))
    return {k: (np.concatenate([p[k] for p in parts]) if parts[0][k] is not None else None) for k in parts[0]}


_WORKLOADS = {}


def workload(i):
    """Full-size workload i, generated once per test session (read-only)."""
    import workloads
    if i not in _WORKLOADS:
        _WORKLOADS[i] = workloads.make(i)
    return _WORKLOADS[i]
