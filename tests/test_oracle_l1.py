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


def test_ties_at_large_magnitude():
    # target mass split over 2 tied maxima, draft mass over 4 (a superset):
    # |1/2 - 1/4| twice plus 1/4 twice = 1, at any magnitude of the logits
    for mag in (2.0 ** 45, 2.0 ** 60, -(2.0 ** 60), 3.0e38):
        a = np.full((1, 30), mag - abs(mag))
        b = a.copy()
        a[0, [2, 7]] = mag
        b[0, [2, 7, 11, 12]] = mag
        r = oracle.l1_distance(a, b)
        assert abs(r["l1"][0] - 1.0) < 1e-12, mag
        assert abs(r["accept_rate"][0] - 0.5) < 1e-12


def test_weighted_loss_num_den_and_finite_differences():
    # the loss is sum w L1 / sum w; its draft-logit gradient matches central
    # differences of that loss (where no p_v - q_v changes sign in the step)
    rng = np.random.default_rng(11)
    R, V = 4, 7
    a = rng.normal(0, 1.5, (R, V))
    b = a + rng.normal(0, 0.8, (R, V))
    w = np.array([1.0, 0.5, 0.0, 2.0])
    r = oracle.weighted_l1_loss(a, b, w, grad_scale=3.0)
    l1 = oracle.l1_distance(a, b)["l1"]
    assert abs(r["num"] - float(np.sum(w * l1))) < 1e-14 and r["den"] == 3.5
    assert abs(r["loss"] - r["num"] / 3.5) < 1e-15
    h = 1e-6
    for t in range(R):
        for v in range(V):
            bp, bm = b.copy(), b.copy()
            bp[t, v] += h
            bm[t, v] -= h
            fd = 3.0 * (oracle.weighted_l1_loss(a, bp, w)["loss"] - oracle.weighted_l1_loss(a, bm, w)["loss"]) / (2 * h)
            assert abs(fd - r["grad"][t, v]) < 1e-7, (t, v, fd, r["grad"][t, v])
    assert (r["grad"][2] == 0).all()  # weight 0: no gradient
    np.testing.assert_allclose(r["grad"].sum(axis=1), 0.0, atol=1e-15)  # softmax gradients sum to 0


def test_weighted_loss_closed_forms():
    # two tokens: L1 = 2 |sigma(a0 - a1) - sigma(b0 - b1)|, and dL1/db0 = 2 sign(q0 - p0) q0 (1 - q0)
    a, b = np.array([[0.3, -0.4]]), np.array([[1.1, 0.2]])
    r = oracle.weighted_l1_loss(a, b)
    p0 = 1.0 / (1.0 + math.exp(-(0.3 + 0.4)))
    q0 = 1.0 / (1.0 + math.exp(-(1.1 - 0.2)))
    assert abs(r["loss"] - 2 * abs(q0 - p0)) < 1e-14
    assert abs(r["grad"][0, 0] - 2 * np.sign(q0 - p0) * q0 * (1 - q0)) < 1e-14
    assert abs(r["grad"][0, 1] + r["grad"][0, 0]) < 1e-15
    # identical rows: zero distance and exactly zero gradient (every sign is 0)
    x = np.random.default_rng(2).normal(0, 2, (3, 50))
    z = oracle.weighted_l1_loss(x, x.copy())
    assert z["loss"] == 0.0 and (z["grad"] == 0.0).all()
    # a masked NaN row adds nothing
    y = x.copy()
    y[1, 4] = np.nan
    m = oracle.weighted_l1_loss(x, y, [1.0, 0.0, 1.0])
    assert np.isnan(m["l1"][1]) and np.isfinite(m["loss"]) and (m["grad"][1] == 0).all()
