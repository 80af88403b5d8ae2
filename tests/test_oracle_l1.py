"""Pins of the oracle's draft/target softmax-L1 distance (CPU only)."""

import json
import math
import os

import numpy as np
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_cases():
    with open(os.path.join(GOLDEN, "l1_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        r = oracle.l1_distance(np.array([c["target"]]), np.array([c["draft"]]))
        assert abs(r["l1"][0] - c["l1"]) < 1e-14, c["name"]
        assert abs(r["accept_rate"][0] - c["accept_rate"]) < 1e-14, c["name"]


def test_identical_is_zero_and_accept_one():
    rng = np.random.default_rng(30)
    x = rng.normal(0, 2, (5, 1000))
    r = oracle.l1_distance(x, x)
    assert (r["l1"] == 0.0).all() and (r["accept_rate"] == 1.0).all()


def test_bounded_symmetric_and_library():
    rng = np.random.default_rng(31)
    a = rng.normal(0, 3, (20, 400))
    b = a + rng.normal(0, 2, (20, 400))
    r = oracle.l1_distance(a, b)
    s = oracle.l1_distance(b, a)
    np.testing.assert_allclose(r["l1"], s["l1"], atol=1e-14)
    assert (r["l1"] <= 2.0).all() and (r["l1"] >= 0.0).all()
    ref = np.abs(scipy.special.softmax(a, axis=1) - scipy.special.softmax(b, axis=1)).sum(1)
    np.testing.assert_allclose(r["l1"], ref, atol=1e-13)
    np.testing.assert_allclose(r["accept_rate"], np.clip(1 - 0.5 * ref, 0, 1), atol=1e-13)


def test_two_token_closed_form():
    rng = np.random.default_rng(32)
    for _ in range(50):
        a0, a1, b0, b1 = rng.normal(0, 3, 4)
        sa = 1 / (1 + math.exp(-(a0 - a1)))
        sb = 1 / (1 + math.exp(-(b0 - b1)))
        r = oracle.l1_distance(np.array([[a0, a1]]), np.array([[b0, b1]]))
        assert abs(r["l1"][0] - 2 * abs(sa - sb)) < 1e-13


def test_disjoint_near_one_hots():
    a = np.full((1, 50), -40.0)
    b = a.copy()
    a[0, 3] = 40.0
    b[0, 7] = 40.0
    r = oracle.l1_distance(a, b)
    assert abs(r["l1"][0] - 2.0) < 1e-12 and r["accept_rate"][0] < 1e-12


def test_nonfinite_rows():
    a = np.zeros((2, 4))
    b = np.zeros((2, 4))
    a[0, 1] = np.nan
    b[1, :] = -np.inf
    r = oracle.l1_distance(a, b)
    assert np.isnan(r["l1"]).all() and np.isnan(r["accept_rate"]).all()
