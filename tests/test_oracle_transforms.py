"""Pins of the oracle's top-k / top-p / min-p transform program (CPU only)."""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "transforms_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_golden_cases(case):
    e = case["expect"]
    r = oracle.score_transforms(np.array([case["x"]]), case["tau"], case["top_k"], case["top_p"],
                                case["min_p"], [case["target"]], cap=8)
    assert r["support_len"][0] == e["support_len"]
    ids = list(r["support_ids"][0][: e["support_len"]])
    assert ids == e["support_ids"]
    assert (r["support_ids"][0][e["support_len"]:] == -1).all()
    assert r["threshold_ties"][0] == e["threshold_ties"]
    if "threshold_logit" in e:
        assert r["threshold_logit"][0] == e["threshold_logit"]
    assert r["status"][0] == e["status"]
    lp = -math.inf if e["logprob"] == "-inf" else e["logprob"]
    if lp == -math.inf:
        assert r["logprob"][0] == -np.inf
    else:
        assert abs(r["logprob"][0] - lp) < 1e-12
    assert abs(r["entropy"][0] - e["entropy"]) < 1e-12


def _rand_rows(rng, R, V, ties=False):
    if ties:
        return rng.integers(-3, 4, size=(R, V)).astype(np.float64) * 0.5
    return rng.normal(0, 2, size=(R, V))


def test_identities_equal_full_scoring():
    rng = np.random.default_rng(20)
    R, V = 12, 300
    x = _rand_rows(rng, R, V)
    tau = rng.uniform(0.5, 1.5, R)
    y = rng.integers(0, V, R)
    f = oracle.score_full(x, tau, y)
    for k in (0, V, V + 5, -1):
        r = oracle.score_transforms(x, tau, k, 1.0, 0.0, y)
        assert (r["support_len"] == V).all()
        np.testing.assert_allclose(r["logprob"], f["logprob"], atol=1e-12)
        np.testing.assert_allclose(r["entropy"], f["entropy"], atol=1e-12)
        np.testing.assert_allclose(r["full_lse"], f["lse"], atol=1e-12)


def test_top_p_one_is_identity_despite_cumulative_overshoot():
    # The running mass before the last rank rounds to 1.0 (float32 and even
    # float64 lose the e^-40 tail), so "keep iff mass before < top_p" would
    # drop it at top_p == 1; the program keeps the full support at top_p == 1
    # (xorl issue #71 section 3, the top_p == 1.0 cumulative-overshoot test).
    x = np.array([[0.0, 0.0, -40.0]])
    m = np.exp(x[0]) / np.exp(x[0]).sum()
    assert np.float32(m[0]) + np.float32(m[1]) >= np.float32(1.0)
    r = oracle.score_transforms(x, 1.0, 0, np.float32(1.0), 0.0, [2], cap=3)
    assert r["support_len"][0] == 3 and r["status"][0] == 0
    r = oracle.score_transforms(x, 1.0, 0, 0.999, 0.0, [2], cap=3)
    assert r["support_len"][0] == 2 and r["status"][0] == oracle.ST_TARGET_OUTSIDE_SUPPORT
    # equal masses 1/V: ranks j with j/V < p are kept
    V = 4000
    r = oracle.score_transforms(np.zeros((1, V)), 1.0, 0, 0.5001, 0.0, [0])
    assert r["support_len"][0] == 2001 and not r["borderline_top_p"][0]
    r = oracle.score_transforms(np.zeros((1, V)), 1.0, 0, 0.5, 0.0, [0])
    assert r["borderline_top_p"][0]  # the mass before rank 2000 is exactly 0.5


def test_top_k_one_is_lowest_id_argmax():
    rng = np.random.default_rng(21)
    x = _rand_rows(rng, 30, 40, ties=True)
    y = np.argmax(x, axis=1)  # numpy returns the first (lowest-id) maximum
    r = oracle.score_transforms(x, 1.0, 1, 1.0, 0.0, y, cap=4)
    assert (r["support_len"] == 1).all()
    np.testing.assert_array_equal(r["support_ids"][:, 0], y)
    assert (r["entropy"] == 0.0).all() and (r["logprob"] == 0.0).all()


def _brute(xrow, tau, k, p, mp):
    """Second formulation: O(V^2) comparison ranks, then prefix searches."""
    V = len(xrow)
    z = [v / tau for v in xrow]
    rank = [sum(1 for j in range(V) if z[j] > z[i] or (z[j] == z[i] and j < i)) for i in range(V)]
    by_rank = [None] * V
    for i, rk in enumerate(rank):
        by_rank[rk] = i
    Lk = V if (k <= 0 or k >= V) else k
    w = [math.exp(z[by_rank[j]] - z[by_rank[0]]) for j in range(Lk)]
    tot = math.fsum(w)
    if p >= 1.0:
        Lp = Lk
    else:
        Lp = 0
        for j in range(Lk):
            if math.fsum(w[:j]) / tot < p:
                Lp = j + 1
    if mp <= 0:
        Lm = V
    else:
        Lm = sum(1 for j in range(V) if math.exp(z[by_rank[j]] - z[by_rank[0]]) >= mp)
    L = min(Lk, Lp, Lm)
    return by_rank[:L]


def test_brute_force_small_vocabularies():
    rng = np.random.default_rng(22)
    for trial in range(400):
        V = int(rng.integers(1, 13))
        x = _rand_rows(rng, 1, V, ties=bool(trial % 2))[0]
        tau = float(rng.choice([0.5, 0.7, 1.0, 1.3]))
        k = int(rng.integers(-1, V + 2))
        p = float(rng.choice([1.0, 0.95, 0.8, 0.5, 0.3, 0.1]))
        mp = float(rng.choice([0.0, 0.05, 0.2, 0.6, 1.0]))
        r = oracle.score_transforms(x[None, :], tau, k, p, mp, [0], cap=V)
        if r["borderline_top_p"][0] or r["borderline_min_p"][0]:
            continue
        sup = _brute(list(x), tau, k, p, mp)
        L = int(r["support_len"][0])
        assert list(r["support_ids"][0][:L]) == sup, (x, tau, k, p, mp)


def test_monotone_in_parameters():
    rng = np.random.default_rng(23)
    x = _rand_rows(rng, 10, 200)
    y = np.zeros(10, dtype=np.int64)
    prev = None
    for k in (1, 5, 20, 100, 0):
        L = oracle.score_transforms(x, 1.0, k, 0.9, 0.01, y)["support_len"]
        if prev is not None:
            assert (L >= prev).all()
        prev = L
    prev = None
    for p in (0.1, 0.5, 0.9, 0.99, 1.0):
        L = oracle.score_transforms(x, 1.0, 0, p, 0.0, y)["support_len"]
        if prev is not None:
            assert (L >= prev).all()
        prev = L
    prev = None
    for mp in (0.9, 0.3, 0.05, 0.001, 0.0):
        L = oracle.score_transforms(x, 1.0, 0, 1.0, mp, y)["support_len"]
        if prev is not None:
            assert (L >= prev).all()
        prev = L


def test_scores_match_recorded_support_scoring():
    rng = np.random.default_rng(24)
    R, V = 20, 500
    x = _rand_rows(rng, R, V)
    tau = rng.choice([0.7, 1.0], R)
    k = rng.choice([0, 20, 50], R)
    p = rng.choice([1.0, 0.95, 0.8], R)
    mp = rng.choice([0.0, 0.05], R)
    r0 = oracle.score_transforms(x, tau, k, p, mp, np.zeros(R, np.int64), cap=V)
    y = r0["support_ids"][:, 0].copy()
    y[::3] = r0["support_ids"][::3, 1].clip(min=0)  # second-ranked token where present
    r = oracle.score_transforms(x, tau, k, p, mp, y, cap=V)
    s = oracle.score_support(lambda t, c: x[t, c], V, r["support_ids"], tau, y)
    np.testing.assert_allclose(r["logprob"], s["logprob"], atol=1e-12)
    np.testing.assert_allclose(r["entropy"], s["entropy"], atol=1e-12)
    assert ((r["status"] & oracle.ST_TARGET_OUTSIDE_SUPPORT) == (s["status"] & oracle.ST_TARGET_OUTSIDE_SUPPORT)).all()


def test_descriptor_and_truncation():
    x = np.array([[2.0, 1.0, 2.0, 2.0, 0.0, 2.0]])
    r = oracle.score_transforms(x, 1.0, 3, 1.0, 0.0, [0], cap=2)
    assert r["support_len"][0] == 3
    assert list(r["support_ids"][0]) == [0, 2]
    assert r["status"][0] == oracle.ST_SUPPORT_TRUNCATED
    assert r["threshold_logit"][0] == 2.0 and r["threshold_ties"][0] == 3
    r = oracle.score_transforms(x, 1.0, 5, 1.0, 0.0, [4], cap=0)
    assert r["support_len"][0] == 5 and r["threshold_logit"][0] == 1.0 and r["threshold_ties"][0] == 1
    assert r["status"][0] == oracle.ST_TARGET_OUTSIDE_SUPPORT and r["logprob"][0] == -np.inf


def test_bad_parameters():
    x = np.zeros((6, 5))
    x[5, 1] = np.nan
    bad = [dict(tau=0.0), dict(top_p=0.0), dict(top_p=float("nan")), dict(min_p=1.5), dict(target=5), dict()]
    for t, b in enumerate(bad):
        r = oracle.score_transforms(x[t:t + 1], b.get("tau", 1.0), 0, b.get("top_p", 1.0), b.get("min_p", 0.0),
                                    [b.get("target", 0)], cap=3)
        assert r["status"][0] == oracle.ST_BAD_INPUT, b
        assert r["support_len"][0] == 0 and (r["support_ids"][0] == -1).all()
        assert np.isnan(r["logprob"][0])


def test_min_p_one_keeps_all_maxima():
    x = np.array([[1.0, 3.0, 3.0, 0.0, 3.0]])
    r = oracle.score_transforms(x, 1.0, 0, 1.0, 1.0, [2], cap=5)
    assert r["support_len"][0] == 3 and list(r["support_ids"][0][:3]) == [1, 2, 4]
    assert abs(r["entropy"][0] - math.log(3)) < 1e-12


def test_neg_inf_tokens_are_dropped_by_top_p():
    x = np.array([[0.0, -np.inf, 0.0, -np.inf]])
    r = oracle.score_transforms(x, 1.0, 0, 0.99, 0.0, [2], cap=4)
    assert r["support_len"][0] == 2 and list(r["support_ids"][0][:2]) == [0, 2]
    r = oracle.score_transforms(x, 1.0, 0, 1.0, 0.0, [1], cap=4)
    assert r["support_len"][0] == 4 and r["logprob"][0] == -np.inf and r["status"][0] == 0


def test_every_combination_small():
    rng = np.random.default_rng(25)
    V = 9
    for k, p, mp, tau in itertools.product([0, 2, 4, 9], [1.0, 0.9, 0.6], [0.0, 0.1], [0.7, 1.0]):
        x = _rand_rows(rng, 1, V, ties=True)[0]
        r = oracle.score_transforms(x[None, :], tau, k, p, mp, [0], cap=V)
        if r["borderline_top_p"][0] or r["borderline_min_p"][0]:
            continue
        L = int(r["support_len"][0])
        assert list(r["support_ids"][0][:L]) == _brute(list(x), tau, k, p, mp)


@pytest.mark.parametrize("mag", [2.0 ** 45, 2.0 ** 60, -(2.0 ** 60), 3.0e38])
def test_tied_maxima_at_large_magnitude(mag):
    # four equal maxima far above the rest: each carries 1/4 of the mass, so
    # top-p 0.6 keeps three of them (exclusive prefixes 0, 1/4, 1/2 < 0.6),
    # the three lowest ids; the support entropy is ln 3 and a kept target
    # scores -ln 3, at any magnitude
    V = 40
    x = np.full((1, V), mag - abs(mag))
    x[0, [31, 4, 17, 8]] = mag
    r = oracle.score_transforms(x, 1.0, 0, 0.6, 0.0, [8], cap=5)
    assert r["support_len"][0] == 3 and list(r["support_ids"][0]) == [4, 8, 17, -1, -1]
    assert r["threshold_logit"][0] == mag and r["threshold_ties"][0] == 3
    assert abs(r["entropy"][0] - math.log(3)) < 1e-12
    assert abs(r["logprob"][0] + math.log(3)) < 1e-12
    assert not r["borderline_top_p"][0]
    # the full-vocabulary LSE: four equal maxima
    assert abs(r["full_lse"][0] - (mag + math.log(4))) <= 1e-12 * max(1.0, abs(mag))


def test_cut_band_and_forced_length():
    # a row whose top-p cut lies exactly on a prefix mass: masses 1/2, 1/4,
    # 1/8, 1/8 (logits ln 4, ln 2, 0, 0); with top_p = 0.75 the exclusive
    # prefix before rank 2 is 0.75 up to rounding, so whether rank 2 is kept
    # (L = 3) or dropped (L = 2) turns on the last bit; the band is [2, 3]
    x = np.array([[0.0, math.log(4.0), 0.0, math.log(2.0)]])
    r = oracle.score_transforms(x, 1.0, 0, 0.75, 0.0, [1], cap=4)
    assert r["borderline_top_p"][0]
    assert r["support_len"][0] in (2, 3) and r["support_len_lo"][0] == 2 and r["support_len_hi"][0] == 3
    # forcing each cut of the band reproduces the program's outputs for that cut
    for L, ids in ((2, [1, 3, -1, -1]), (3, [1, 3, 0, -1]), (4, [1, 3, 0, 2])):
        f = oracle.score_prefix_support(x, 1.0, [L], [1], cap=4)
        assert f["support_len"][0] == L and list(f["support_ids"][0]) == ids
        w = np.array([4.0, 2.0, 1.0, 1.0])[:L]
        assert abs(f["logprob"][0] - math.log(4.0 / w.sum())) < 1e-12
        q = w / w.sum()
        assert abs(f["entropy"][0] + np.sum(q * np.log(q))) < 1e-12
    assert oracle.score_prefix_support(x, 1.0, [3], [1], cap=4)["threshold_ties"][0] == 1
    g = oracle.score_prefix_support(x, 1.0, r["support_len"], [1], cap=4)
    for k in ("support_len", "threshold_logit", "threshold_ties", "support_ids", "logprob", "entropy", "status"):
        np.testing.assert_array_equal(g[k], r[k])
    # a row that is not borderline has a one-value band
    r = oracle.score_transforms(x, 1.0, 0, 0.6, 0.0, [1], cap=4)
    assert not r["borderline_top_p"][0] and r["support_len_lo"][0] == r["support_len_hi"][0] == r["support_len"][0]
    # min-p band: weights 1, 1/2, 1/4, 1/4 relative to the max; min_p = 0.25 sits on the last two
    r = oracle.score_transforms(x, 1.0, 0, 1.0, 0.25, [1], cap=4)
    assert r["borderline_min_p"][0] and r["support_len"][0] == 4
    assert r["support_len_lo"][0] == 2 and r["support_len_hi"][0] == 4
