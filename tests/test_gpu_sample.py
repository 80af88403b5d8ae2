"""GPU parity: the seeded Gumbel draw from the transformed support vs the fp64 oracle.

Both sides compute the same Philox4x32-10 numbers (integers, exact) and the
score (x - x_max)/tau - ln(-ln u) in fp64; the draw is an argmax, so the
kernel's token must equal the oracle's.  The two fp64 logarithms may differ
in the last bit, so where the oracle's best and second-best scores lie within
1e-9 of each other either token is accepted and the row is counted."""

import numpy as np
import pytest
import torch

import oracle
from oracle import sampling
import workloads
from tests.gpu_common import bf16_tensor, oracle_by_rows, say, to_dev, workload

pytestmark = pytest.mark.gpu

NEAR = 1e-9


@pytest.fixture(scope="module")
def vsa():
    import logprob_entropy_sampling_amd as m
    m.lib()
    return m


def _draw(vsa, bits, tau, k, p, mp, seed, offset=0):
    return vsa.sample_transforms(bf16_tensor(bits), to_dev(np.asarray(k, np.int32)), to_dev(np.asarray(p, np.float32)),
                                 to_dev(np.asarray(mp, np.float32)), temperature=to_dev(np.asarray(tau, np.float32)),
                                 seed=seed, offset=offset)


def _check(got, ref, x_rows, tau, seed, offset, rows, label):
    s = got["sampled"].cpu().numpy()
    assert np.array_equal(got["status"].cpu().numpy(), ref["status"]), label
    assert np.array_equal(s < 0, ref["sampled"] < 0), label
    diff = np.nonzero(s != ref["sampled"])[0]
    near = 0
    for i in diff:  # both must be best-scoring support tokens up to NEAR
        assert ref["margin"][i] <= NEAR, f"{label}: row {rows[i]} drew {s[i]}, oracle {ref['sampled'][i]}"
        x = x_rows[i]
        u = sampling.token_uniforms(int(rows[i]), x.size, seed, offset)
        sc = lambda v: (x[v] - x.max()) / tau[i] - np.log(-np.log(u[v]))  # noqa: E731
        assert abs(sc(s[i]) - sc(ref["sampled"][i])) <= NEAR, label
        near += 1
    say(f"  {label}: {len(s)} rows, {len(s) - diff.size} identical draws, {near} draws within {NEAR} of a tie")


def test_workload_rows(vsa):
    say("sample: 72 rows of the transforms workload (every parameter combination twice), V=151936")
    c = workloads.make(5, T=72)
    x64 = oracle.logits_from_logits(c["logits"], "bf16")
    args = (c["temperature"], c["top_k"], c["top_p"], c["min_p"])
    for seed, off in ((1234, 0), (1234, 1), (2 ** 63 + 5, 2 ** 40 + 3)):
        got = _draw(vsa, c["logits"], *args, seed=seed, offset=off)
        ref = sampling.sample_transforms(x64, *args, seed=seed, offset=off)
        _check(got, ref, x64, c["temperature"], seed, off, np.arange(72), f"seed {seed} offset {off}")
        # the draw lies in the support, and its score follows from vs_score_transforms
        sc = vsa.score_transforms(got["sampled"], bf16_tensor(c["logits"]), *(to_dev(a) for a in args[1:]),
                                  temperature=to_dev(args[0]))
        assert ((sc["status"].cpu().numpy() & 0x06) == 0).all()
        assert torch.equal(sc["support_len"], got["support_len"])
    again = _draw(vsa, c["logits"], *args, seed=1234, offset=1)
    first = _draw(vsa, c["logits"], *args, seed=1234, offset=1)
    assert torch.equal(again["sampled"], first["sampled"])


@pytest.mark.parametrize("V", [5, 3001, 100000, 170001])
def test_ties_at_the_threshold(vsa, V):
    # small integer logits: long runs of equal values, so top-k and top-p cut
    # inside a tie group (the support takes its lowest ids: the second pass)
    say(f"sample: tied logits V={V}, cuts inside tie groups, -inf tokens, singleton supports")
    rng = np.random.default_rng(V)
    T = 40
    vals = rng.integers(-3, 4, size=(T, V)).astype(np.float32) * np.float32(0.5)
    vals[::4, ::3] = -np.inf
    bits = workloads.to_bf16_bits(vals)
    k = rng.choice([0, 1, 3, V // 2, V], T).astype(np.int32)
    p = rng.choice([1.0, 0.9, 0.5, 0.2], T).astype(np.float32)
    mp = rng.choice([0.0, 0.0, 0.3], T).astype(np.float32)
    tau = rng.choice([0.5, 1.0, 2.0], T).astype(np.float32)
    x64 = oracle.logits_from_logits(bits, "bf16")
    for seed in (7, 8):
        got = _draw(vsa, bits, tau, k, p, mp, seed=seed)
        ref = sampling.sample_transforms(x64, tau, k, p, mp, seed=seed)
        _check(got, ref, x64, tau, seed, 0, np.arange(T), f"V={V} seed {seed}")
    s = got["sampled"].cpu().numpy()
    assert np.isfinite(x64[np.arange(T), s]).all()  # a -inf token is never drawn


def test_frequencies_follow_the_support_softmax(vsa):
    # one row repeated 6000 times: the row index is in the counter, so each
    # copy is an independent draw; frequencies match softmax over the top 3
    say("sample: 6000 copies of one row, top-k 3: frequencies vs the support softmax")
    T, V = 6000, 64
    x = np.full((T, V), -4.0, np.float32)
    x[:, [10, 20, 30]] = np.log(np.array([1.0, 2.0, 3.0], np.float32))
    bits = workloads.to_bf16_bits(x)
    got = _draw(vsa, bits, np.ones(T), np.full(T, 3), np.ones(T), np.zeros(T), seed=99)
    s = got["sampled"].cpu().numpy()
    assert set(np.unique(s)) <= {10, 20, 30}
    w = np.exp(oracle.logits_from_logits(bits[0], "bf16")[[10, 20, 30]])
    expect = T * w / w.sum()
    counts = np.array([(s == v).sum() for v in (10, 20, 30)])
    assert float(np.sum((counts - expect) ** 2 / expect)) < 13.8, (counts, expect)


def test_full_size_all_rows(vsa):
    say("sample: full transforms workload T=2048 V=151936, every row vs the oracle; determinism")
    c = workload(5)
    T = c["T"]
    args = (c["temperature"], c["top_k"], c["top_p"], c["min_p"])
    seed, off = 20260101, 17
    got = _draw(vsa, c["logits"], *args, seed=seed, offset=off)
    again = _draw(vsa, c["logits"], *args, seed=seed, offset=off)
    assert torch.equal(got["sampled"], again["sampled"])

    def ref_rows(r):
        x = oracle.logits_from_logits(c["logits"], "bf16", rows=r)
        out = sampling.sample_transforms(x, *(a[r] for a in args), seed=seed, offset=off, rows=r)
        return {"sampled": out["sampled"], "status": out["status"], "margin": out["margin"]}
    ref = oracle_by_rows(ref_rows, T)
    s = got["sampled"].cpu().numpy()
    assert np.array_equal(got["status"].cpu().numpy(), ref["status"])
    diff = np.nonzero(s != ref["sampled"])[0]
    assert all(ref["margin"][i] <= NEAR for i in diff), diff[:10]
    say(f"  full size: {T - diff.size} of {T} draws identical, {diff.size} within {NEAR} of a tie")


def test_row_order_mixed_supports_and_bad_rows(vsa):
    """1100 rows (the row-order kernels loop past one workgroup's 1024
    threads) of V = 90,000 (the split transforms path, with its finish-order
    kernel) whose supports range from one token to the whole row in shuffled
    order, with BAD rows (a NaN temperature) among them: every draw is the
    oracle's, whatever order the rows were drawn in."""
    T, V = 1100, 90000
    say(f"sample: T={T} V={V}, supports from 1 token to the whole row in shuffled order, 7 BAD rows")
    rng = np.random.default_rng(77)
    bits = workloads.to_bf16_bits((rng.standard_normal((T, V)) * 2.0).astype(np.float32))
    kind = rng.integers(0, 5, T)
    k = np.where(kind == 0, 1, np.where(kind == 1, 50, 0)).astype(np.int32)
    p = np.where(kind == 2, 0.9, 1.0).astype(np.float32)
    mp = np.where(kind == 3, 0.05, 0.0).astype(np.float32)  # kind 4: the whole row
    tau = rng.uniform(0.6, 1.2, T).astype(np.float32)
    tau[rng.choice(T, 7, replace=False)] = np.nan
    seed, off = 99, 5
    got = _draw(vsa, bits, tau, k, p, mp, seed=seed, offset=off)

    def ref_rows(r):
        x = oracle.logits_from_logits(bits, "bf16", rows=r)
        out = sampling.sample_transforms(x, tau[r], k[r], p[r], mp[r], seed=seed, offset=off, rows=r)
        return {"sampled": out["sampled"], "status": out["status"], "margin": out["margin"]}
    ref = oracle_by_rows(ref_rows, T)
    s = got["sampled"].cpu().numpy()
    assert np.array_equal(got["status"].cpu().numpy(), ref["status"])
    assert (s[np.isnan(tau)] == -1).all() and (ref["status"][np.isnan(tau)] & 0x04).all()
    diff = np.nonzero(s != ref["sampled"])[0]
    assert all(ref["margin"][i] <= NEAR for i in diff), diff[:10]
    sl = got["support_len"].cpu().numpy()
    assert sl[kind == 4][~np.isnan(tau[kind == 4])].min() == V and sl[kind == 0][~np.isnan(tau[kind == 0])].max() == 1
    say(f"  {T - diff.size} of {T} draws identical, {diff.size} within {NEAR} of a tie")


@pytest.mark.parametrize("V", [5000, 90000])
def test_supports_around_the_listed_id_capacity(vsa, V):
    # supports of 1..66 tokens, cut by top-k or min-p inside tie groups of
    # small-integer logits: those of up to 64 tokens are drawn from their
    # listed dense ids, larger ones from the row pass; every draw is the
    # oracle's (the same support, ties taken by ascending id)
    say(f"sample: V={V}, supports of 1 to 66 tokens around the 64 listed ids, cuts inside tie groups")
    rng = np.random.default_rng(V + 64)
    T = 48
    vals = rng.integers(-6, 2, size=(T, V)).astype(np.float32) * np.float32(0.75)
    vals[::5, ::7] = -np.inf
    vals[:, rng.choice(V, 40, replace=False)] = 4.0  # a tie group of 40 at the top of every row
    bits = workloads.to_bf16_bits(vals)
    k = np.array([1, 2, 39, 40, 41, 63, 64, 65, 66, 0, 0, 0] * 4, np.int32)
    p = np.ones(T, np.float32)
    mp = np.where(k == 0, 0.5, 0.0).astype(np.float32)  # min-p alone: the 40 tied maxima
    tau = rng.choice([0.5, 1.0], T).astype(np.float32)
    x64 = oracle.logits_from_logits(bits, "bf16")
    for seed in (3, 4):
        got = _draw(vsa, bits, tau, k, p, mp, seed=seed)
        ref = sampling.sample_transforms(x64, tau, k, p, mp, seed=seed)
        _check(got, ref, x64, tau, seed, 0, np.arange(T), f"V={V} seed {seed}")
    sl = got["support_len"].cpu().numpy()
    assert np.array_equal(sl[k > 0], k[k > 0]) and (sl[k == 0] == 40).all()
