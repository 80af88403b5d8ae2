"""Pins of the oracle's seeded Gumbel draw (CPU only).

The generator is pinned by Philox4x32-10's published known-answer vectors;
the draw by what Gumbel-max sampling must give: the softmax frequencies of
the support (a chi-square test over many offsets), the support restriction,
singleton and top-k 1 supports, and shift invariance."""

import json
import math
import os

import numpy as np
import pytest

from oracle import sampling
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")


def test_philox_known_answer_vectors():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ctr = np.array([int(w, 16) for w in c["counter"]], dtype=np.uint64)
        key = np.array([int(w, 16) for w in c["key"]], dtype=np.uint64)
        out = sampling.philox4x32_10(ctr, key)
        assert [f"{int(w):08x}" for w in out] == c["out"]
    # batched counters give the same words as one at a time
    ctr = np.array([[int(w, 16) for w in c["counter"]] for c in cases], dtype=np.uint64)
    key = np.array([[int(w, 16) for w in c["key"]] for c in cases], dtype=np.uint64)
    got = sampling.philox4x32_10(ctr, key)
    assert [[f"{int(w):08x}" for w in row] for row in got] == [c["out"] for c in cases]


def test_token_uniforms_layout():
    # token v takes word v mod 4 of the block v div 4; rows and offsets are counter words
    u = sampling.token_uniforms(row=7, V=10, seed=0x123456789ABCDEF0, offset=(5 << 32) | 3)
    blk = sampling.philox4x32_10(np.array([[0, 7, 3, 5], [1, 7, 3, 5], [2, 7, 3, 5]], dtype=np.uint64),
                                 np.array([[0x9ABCDEF0, 0x12345678]] * 3, dtype=np.uint64)).reshape(-1)
    np.testing.assert_array_equal(u, (blk[:10].astype(np.float64) + 0.5) * 2.0 ** -32)
    assert (u > 0).all() and (u < 1).all()
    assert not np.array_equal(u, sampling.token_uniforms(row=8, V=10, seed=0x123456789ABCDEF0, offset=(5 << 32) | 3))


@pytest.mark.parametrize("tau", [1.0, 0.5])
def test_draw_frequencies_are_the_support_softmax(tau):
    # support {0, 1, 2} of a 6-token row (top_k 3); 6000 draws over offsets
    x = np.array([[0.0, math.log(2.0), math.log(3.0), -5.0, -6.0, -7.0]])
    n = 6000
    counts = np.zeros(6)
    for o in range(n):
        r = sampling.sample_transforms(x, tau, 3, 1.0, 0.0, seed=42, offset=o)
        counts[r["sampled"][0]] += 1
    assert counts[3:].sum() == 0  # never outside the support
    w = np.exp(x[0, :3] / tau)
    p = w / w.sum()
    chi2 = float(np.sum((counts[:3] - n * p) ** 2 / (n * p)))
    assert chi2 < 13.8, (counts, n * p)  # 2 degrees of freedom, p < 0.001


def test_full_vocabulary_frequencies():
    # no filter: the draw follows softmax(x / tau) over all 4 tokens
    x = np.array([[1.0, 0.0, -1.0, 0.5]])
    n = 8000
    counts = np.bincount([sampling.sample_transforms(x, 0.8, 0, 1.0, 0.0, seed=7, offset=o)["sampled"][0]
                          for o in range(n)], minlength=4)
    p = np.exp(x[0] / 0.8) / np.exp(x[0] / 0.8).sum()
    chi2 = float(np.sum((counts - n * p) ** 2 / (n * p)))
    assert chi2 < 16.3, (counts, n * p)  # 3 degrees of freedom, p < 0.001


def test_singleton_and_top1_supports():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 2, size=(20, 50))
    x[5, [3, 9]] = x[5].max() + 1.0  # tied maxima: top-k 1 keeps the lower id
    r = sampling.sample_transforms(x, 1.0, 1, 1.0, 0.0, seed=99)
    argmax_low_id = np.array([int(np.nonzero(x[t] == x[t].max())[0][0]) for t in range(20)])
    np.testing.assert_array_equal(r["sampled"], argmax_low_id)
    assert r["sampled"][5] == 3
    assert np.isinf(r["margin"]).all()


def test_draw_stays_in_support_and_is_shift_invariant():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 2, size=(30, 300))
    k = rng.choice([0, 5, 40], 30)
    p = rng.choice([1.0, 0.9, 0.5], 30)
    mp = rng.choice([0.0, 0.05], 30)
    tau = rng.choice([0.7, 1.0, 1.3], 30)
    r = sampling.sample_transforms(x, tau, k, p, mp, seed=2026, offset=11)
    d = oracle.score_transforms(x, tau, k, p, mp, r["sampled"], cap=300)
    assert ((d["status"] & oracle.ST_TARGET_OUTSIDE_SUPPORT) == 0).all()
    for t in range(30):
        assert r["sampled"][t] in d["support_ids"][t][: d["support_len"][t]]
    # shifting a row's logits by a constant leaves every decision unchanged (the score
    # subtracts the row maximum); scaling the logits with tau leaves it unchanged too
    s = sampling.sample_transforms(x + 1000.0, tau, k, p, mp, seed=2026, offset=11)
    np.testing.assert_array_equal(s["sampled"], r["sampled"])
    q = sampling.sample_transforms(2.0 * x, 2.0 * tau, k, p, mp, seed=2026, offset=11)
    np.testing.assert_array_equal(q["sampled"], r["sampled"])
    # another seed draws differently somewhere
    o = sampling.sample_transforms(x, tau, k, p, mp, seed=2027, offset=11)
    assert (o["sampled"] != r["sampled"]).any()


def test_bad_rows_draw_nothing():
    x = np.zeros((3, 8))
    x[1, 2] = np.nan
    r = sampling.sample_transforms(x, np.array([1.0, 1.0, 0.0]), 0, 1.0, 0.0, seed=1)
    assert r["sampled"][0] >= 0 and list(r["sampled"][1:]) == [-1, -1]
    assert list(r["status"]) == [0, oracle.ST_BAD_INPUT, oracle.ST_BAD_INPUT]
