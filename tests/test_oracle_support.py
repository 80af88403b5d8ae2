"""Pins of the oracle's recorded-support scoring (CPU only)."""

import math

import numpy as np
import scipy.special
import scipy.stats

import oracle


def _fn(x):
    return lambda t, cols: x[t, np.asarray(cols, dtype=np.int64)]


def test_singleton_is_exactly_zero():
    rng = np.random.default_rng(10)
    x = rng.normal(0, 3, (20, 50))
    ids = np.full((20, 4), -1)
    ids[:, 2] = rng.integers(0, 50, 20)
    tau = rng.uniform(0.5, 1.5, 20)
    r = oracle.score_support(_fn(x), 50, ids, tau, ids[:, 2])
    assert (r["logprob"] == 0.0).all() and (r["entropy"] == 0.0).all()
    assert (r["status"] == 0).all()


def test_full_support_equals_full_vocabulary():
    rng = np.random.default_rng(11)
    V = 64
    x = rng.normal(0, 2, (6, V))
    ids = np.stack([np.concatenate([rng.permutation(V), [-1, -1]]) for _ in range(6)])
    y = rng.integers(0, V, 6)
    tau = rng.uniform(0.5, 1.5, 6)
    s = oracle.score_support(_fn(x), V, ids, tau, y)
    f = oracle.score_full(x, tau, y)
    np.testing.assert_allclose(s["logprob"], f["logprob"], atol=1e-12)
    np.testing.assert_allclose(s["entropy"], f["entropy"], atol=1e-12)


def test_against_library_on_subsets():
    rng = np.random.default_rng(12)
    V = 100
    for _ in range(30):
        x = rng.normal(0, 2, (1, V))
        w = int(rng.integers(2, 12))
        sup = rng.choice(V, w, replace=False)
        y = int(sup[rng.integers(0, w)])
        tau = float(rng.uniform(0.5, 1.5))
        ids = np.full((1, 16), -1)
        pos = rng.choice(16, w, replace=False)  # padding anywhere in the row
        ids[0, pos] = sup
        r = oracle.score_support(_fn(x), V, ids, tau, [y])
        z = x[0, sup] / tau
        ls = scipy.special.log_softmax(z)
        assert abs(r["logprob"][0] - ls[list(sup).index(y)]) < 1e-12
        assert abs(r["entropy"][0] - scipy.stats.entropy(np.exp(ls))) < 1e-12
        # order and padding position do not matter
        ids2 = np.full((1, 16), -1)
        ids2[0, :w] = sup[::-1]
        r2 = oracle.score_support(_fn(x), V, ids2, tau, [y])
        assert abs(r2["logprob"][0] - r["logprob"][0]) < 1e-13
        assert abs(r2["entropy"][0] - r["entropy"][0]) < 1e-13


def test_support_bounds():
    rng = np.random.default_rng(13)
    V = 200
    x = rng.normal(0, 2, (40, V))
    ids = np.full((40, 10), -1)
    y = np.empty(40, dtype=np.int64)
    for t in range(40):
        w = int(rng.integers(1, 11))
        ids[t, :w] = rng.choice(V, w, replace=False)
        y[t] = ids[t, 0]
    s = oracle.score_support(_fn(x), V, ids, 1.0, y)
    f = oracle.score_full(x, 1.0, y)
    widths = (ids >= 0).sum(1)
    assert (s["logprob"] >= f["logprob"] - 1e-12).all()
    assert (s["entropy"] >= -1e-15).all()
    assert (s["entropy"] <= np.log(widths) + 1e-12).all()


def test_empty_rows_and_synthetic_eos_fallback():
    rng = np.random.default_rng(14)
    V = 30
    x = rng.normal(0, 2, (3, V))
    ids = np.full((3, 5), -1)
    ids[2, :2] = [4, 9]
    y = np.array([7, 8, 4])
    fb = np.array([1, 0, 1], np.uint8)
    r = oracle.score_support(_fn(x), V, ids, 1.0, y, fallback=fb)
    f = oracle.score_full(x, 1.0, y)
    assert r["status"][0] == oracle.ST_EMPTY_SUPPORT | oracle.ST_FULL_VOCAB_FALLBACK
    assert abs(r["logprob"][0] - f["logprob"][0]) < 1e-13 and r["entropy"][0] == 0.0
    assert r["status"][1] == oracle.ST_EMPTY_SUPPORT
    assert r["logprob"][1] == 0.0 and r["entropy"][1] == 0.0
    # the flag does nothing on a non-empty row
    assert r["status"][2] == 0
    assert abs(r["logprob"][2] - (x[2, 4] - math.log(math.exp(x[2, 4]) + math.exp(x[2, 9])))) < 1e-12


def test_target_outside_and_bad_rows():
    V = 10
    x = np.zeros((5, V))
    x[3, 2] = np.nan
    ids = np.array([[1, 2, -1], [1, 1, -1], [1, 10, -1], [2, 3, -1], [4, 5, 6]])
    y = np.array([3, 1, 1, 2, 11])
    r = oracle.score_support(_fn(x), V, ids, 1.0, y)
    assert r["status"][0] == oracle.ST_TARGET_OUTSIDE_SUPPORT and r["logprob"][0] == -np.inf
    assert abs(r["entropy"][0] - math.log(2)) < 1e-15
    assert (r["status"][1:] == oracle.ST_BAD_INPUT).all()
    assert np.isnan(r["logprob"][1:]).all()
    bad_tau = oracle.score_support(_fn(x), V, ids[:1], -1.0, y[:1])
    assert bad_tau["status"][0] == oracle.ST_BAD_INPUT


def test_brute_force_python_floats():
    rng = np.random.default_rng(15)
    V = 12
    for _ in range(40):
        xs = rng.normal(0, 2, V)
        w = int(rng.integers(1, 6))
        sup = [int(v) for v in rng.choice(V, w, replace=False)]
        y = sup[int(rng.integers(0, w))]
        wts = {v: math.exp(float(xs[v])) for v in sup}
        tot = sum(wts.values())
        ids = np.array([sup + [-1] * (6 - w)])
        r = oracle.score_support(_fn(xs[None, :]), V, ids, 1.0, [y])
        assert abs(r["logprob"][0] - math.log(wts[y] / tot)) < 1e-12
        assert abs(r["entropy"][0] + sum(q / tot * math.log(q / tot) for q in wts.values())) < 1e-12
