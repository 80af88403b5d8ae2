"""Pins of the oracle's full-vocabulary scoring and projection (CPU only).

Each test checks the oracle against something other than itself: a closed
form, a library routine (scipy / torch CPU), brute force with plain Python
floats, or a metamorphic relation that the definition fixes.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)["cases"]


def test_golden_full_cases():
    for c in _golden("full_cases.json"):
        if "V" in c:
            V = c["V"]
            x = np.full((1, V), 0.375)
            r = oracle.score_full(x, 1.0, [V // 3])
            assert abs(r["entropy"][0] - c["entropy"]) < 1e-12, c["name"]
            assert abs(r["logprob"][0] - c["logprob"]) < 1e-12, c["name"]
        else:
            r = oracle.score_full(np.array([c["x"]]), c["tau"], [c["target"]])
            for k in ("lse", "logprob", "entropy"):
                assert abs(r[k][0] - c[k]) < 1e-13, (c["name"], k)
            assert r["status"][0] == 0


def test_two_token_closed_form():
    rng = np.random.default_rng(0)
    for _ in range(50):
        a, b = rng.normal(0, 4, size=2)
        p = 1.0 / (1.0 + math.exp(-(a - b)))
        r = oracle.score_full(np.array([[a, b]]), 1.0, [0])
        h = -(p * math.log(p) + (1 - p) * math.log(1 - p))
        assert abs(r["entropy"][0] - h) < 1e-12
        assert abs(r["logprob"][0] - math.log(p)) < 1e-12


def test_against_library_routines():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 3, size=(8, 1000))
    tau = rng.uniform(0.5, 1.5, size=8)
    y = rng.integers(0, 1000, size=8)
    r = oracle.score_full(x, tau, y)
    z = x / tau[:, None]
    lse = scipy.special.logsumexp(z, axis=1)
    np.testing.assert_allclose(r["lse"], lse, rtol=0, atol=1e-11)
    ls = torch.log_softmax(torch.from_numpy(z), dim=1).numpy()
    np.testing.assert_allclose(r["logprob"], ls[np.arange(8), y], rtol=0, atol=1e-11)
    ent = torch.distributions.Categorical(logits=torch.from_numpy(z)).entropy().numpy()
    np.testing.assert_allclose(r["entropy"], ent, rtol=0, atol=1e-11)
    p = scipy.special.softmax(z, axis=1)
    np.testing.assert_allclose(r["entropy"], scipy.stats.entropy(p, axis=1), rtol=0, atol=1e-11)


def test_brute_force_tiny_python_floats():
    rng = np.random.default_rng(2)
    for V in range(1, 9):
        for _ in range(10):
            xs = [float(v) for v in rng.normal(0, 2, size=V)]
            tau = float(rng.uniform(0.3, 2.0))
            y = int(rng.integers(0, V))
            w = [math.exp(v / tau) for v in xs]
            tot = sum(w)
            probs = [wi / tot for wi in w]
            r = oracle.score_full(np.array([xs]), tau, [y])
            assert abs(r["logprob"][0] - math.log(probs[y])) < 1e-12
            assert abs(r["entropy"][0] - (-sum(p * math.log(p) for p in probs))) < 1e-12
            assert abs(r["lse"][0] - math.log(tot)) < 1e-12


def test_shift_and_temperature_relations():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 2, size=(4, 500))
    y = rng.integers(0, 500, size=4)
    base = oracle.score_full(x, 1.0, y)
    sh = oracle.score_full(x + 7.25, 1.0, y)
    np.testing.assert_allclose(sh["logprob"], base["logprob"], atol=1e-12)
    np.testing.assert_allclose(sh["entropy"], base["entropy"], atol=1e-12)
    np.testing.assert_allclose(sh["lse"], base["lse"] + 7.25, atol=1e-12)
    # temperature divides the logits: score(x, tau) == score(x / tau, 1), exact for tau = 2^j
    for tau in (0.25, 0.5, 2.0, 4.0):
        a = oracle.score_full(x, tau, y)
        b = oracle.score_full(x / tau, 1.0, y)
        for k in ("lse", "logprob", "entropy"):
            np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("shift_exp,unit_exp", [(40, 0), (60, 8), (100, 48), (1000, 948)])
def test_huge_shift_invariance(shift_exp, unit_exp):
    # logits c + 2^u * k_v with tau = 2^u: every value is exact in float64
    # (the spacing at c = 2^e is 2^(e-52) <= 2^u) and z = c / tau + k_v, so
    # logprob and entropy must equal those of the small integers k_v with
    # tau = 1 (a shift changes neither), and LSE moves by exactly c / tau.
    rng = np.random.default_rng(shift_exp)
    k = rng.integers(-12, 13, size=(5, 300)).astype(np.float64)
    y = rng.integers(0, 300, size=5)
    c, unit = 2.0 ** shift_exp, 2.0 ** unit_exp
    base = oracle.score_full(k, 1.0, y)
    for sign in (1.0, -1.0):
        x = sign * c + unit * k
        assert np.array_equal((x - sign * c) / unit, k)  # exactly representable
        r = oracle.score_full(x, unit, y)
        np.testing.assert_allclose(r["logprob"], base["logprob"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["entropy"], base["entropy"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["lse"] - sign * c / unit, base["lse"], rtol=0, atol=1e-12 * c / unit)


@pytest.mark.parametrize("mag", [2.0 ** 43, 2.0 ** 50, 2.0 ** 60, 3.0e38])
@pytest.mark.parametrize("n_tied", [2, 4, 7])
def test_k_way_tie_at_large_magnitude(mag, n_tied):
    # n_tied equal maxima far above every other logit: softmax puts 1/n_tied
    # on each, so entropy = ln n_tied and a tied target has logprob -ln n_tied,
    # whatever the magnitude (and for maxima at -mag above -2 mag as well)
    V = 64
    for top, rest in ((mag, 0.0), (-mag, -2.0 * mag)):
        x = np.full((1, V), rest)
        x[0, 5:5 + n_tied] = top
        r = oracle.score_full(x, 1.0, [5 + n_tied - 1])
        assert abs(r["entropy"][0] - math.log(n_tied)) < 1e-12, (top, r["entropy"][0])
        assert abs(r["logprob"][0] + math.log(n_tied)) < 1e-12, (top, r["logprob"][0])
        assert r["status"][0] == 0
        r = oracle.score_full(x, 1.0, [0])  # a target far below the maxima
        assert r["logprob"][0] < -1e10 and abs(r["entropy"][0] - math.log(n_tied)) < 1e-12


def test_bounds():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 5, size=(16, 300))
    r = oracle.score_full(x, 1.0, rng.integers(0, 300, size=16))
    assert (r["entropy"] >= 0).all() and (r["entropy"] <= math.log(300) + 1e-12).all()
    assert (r["logprob"] <= 0).all()


def test_neg_inf_logits_are_zero_probability():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, size=(1, 20))
    x2 = x.copy()
    x2[0, [3, 7, 11]] = -np.inf
    a = oracle.score_full(x2, 1.0, [0])
    keep = [i for i in range(20) if i not in (3, 7, 11)]
    b = oracle.score_full(x[:, keep], 1.0, [0])
    for k in ("lse", "logprob", "entropy"):
        assert abs(a[k][0] - b[k][0]) < 1e-12
    assert a["status"][0] == 0
    c = oracle.score_full(x2, 1.0, [3])
    assert c["logprob"][0] == -np.inf and c["status"][0] == 0


def test_bad_rows():
    x = np.zeros((6, 4))
    x[1, 2] = np.nan
    x[2, 0] = np.inf
    x[3, :] = -np.inf
    tau = np.array([1.0, 1.0, 1.0, 1.0, 0.0, 1.0])
    y = np.array([0, 0, 0, 0, 0, 4])
    r = oracle.score_full(x, tau, y)
    assert r["status"][0] == 0
    assert (r["status"][1:] == oracle.ST_BAD_INPUT).all()
    assert np.isnan(r["logprob"][1:]).all() and np.isnan(r["entropy"][1:]).all()


def test_round_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(6)
    x = np.concatenate([
        rng.normal(0, 1, 20000).astype(np.float32),
        rng.normal(0, 1e-38, 2000).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32),
    ])
    # exact ties: low 16 bits == 0x8000
    u = rng.integers(0, 2 ** 31, 1000).astype(np.uint32)
    ties = ((u & np.uint32(0x7F7F0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    ours = oracle.round_f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    nan = oracle.round_f32_to_bf16(np.array([np.nan], np.float32))
    assert np.isnan(oracle.widen_bf16(nan))[0]


def test_widen_bf16_matches_torch():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))


def test_projection_brute_force():
    rng = np.random.default_rng(7)
    T, H, V = 3, 17, 11
    hid = rng.normal(0, 1, (T, H)).astype(np.float32)
    w = torch.from_numpy(rng.normal(0, 0.1, (V, H)).astype(np.float32)).to(torch.bfloat16)
    wbits = w.view(torch.int16).numpy().view(np.uint16)
    x = oracle.logits_from_hidden(hid, "f32", wbits)
    hb = torch.from_numpy(hid).to(torch.bfloat16).double()
    wd = w.double()
    for t in range(T):
        for v in range(V):
            s = math.fsum(float(hb[t, h]) * float(wd[v, h]) for h in range(H))
            assert abs(x[t, v] - s) < 1e-14
    # selected rows / columns
    xs = oracle.logits_from_hidden(hid, "f32", wbits, rows=[2, 0], cols=[5, 1, 9])
    np.testing.assert_array_equal(xs, x[[2, 0]][:, [5, 1, 9]])
    # bf16 hidden input takes no extra rounding
    hbits = torch.from_numpy(hid).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.logits_from_hidden(hbits, "bf16", wbits), x)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_logits_from_logits(dtype):
    rng = np.random.default_rng(8)
    v = rng.normal(0, 2, (3, 9)).astype(np.float32)
    if dtype == "bf16":
        bits = torch.from_numpy(v).to(torch.bfloat16)
        ref = bits.double().numpy()
        arr = bits.view(torch.int16).numpy().view(np.uint16)
    else:
        arr, ref = v, v.astype(np.float64)
    np.testing.assert_array_equal(oracle.logits_from_logits(arr, dtype), ref)
    np.testing.assert_array_equal(oracle.logits_from_logits(arr, dtype, rows=[1]), ref[[1]])


def _scores_objective(h, w, tau, y, a, b):
    r = oracle.score_full(h @ w.T, tau, y)
    return float(np.sum(a * r["logprob"] + b * r["entropy"]))


def test_vjp_matches_finite_differences():
    # the gradient of sum a logprob + b H with respect to the logits, the
    # hidden state and the weight, against central differences of the scores
    rng = np.random.default_rng(31)
    T, H, V = 3, 5, 7
    h = rng.normal(0, 1, (T, H))
    w = rng.normal(0, 0.5, (V, H))
    tau = np.array([1.0, 0.7, 1.6])
    y = np.array([2, 0, 6])
    a = np.array([1.0, -0.5, 2.0])
    b = np.array([0.3, 1.0, -0.8])
    x = h @ w.T
    dx = oracle.logit_vjp(x, tau, y, a, b)
    eps = 1e-6
    for t in range(T):
        for v in range(V):
            xp, xm = x.copy(), x.copy()
            xp[t, v] += eps
            xm[t, v] -= eps
            rp, rm = oracle.score_full(xp, tau, y), oracle.score_full(xm, tau, y)
            fd = (np.sum(a * rp["logprob"] + b * rp["entropy"]) - np.sum(a * rm["logprob"] + b * rm["entropy"])) / (2 * eps)
            assert abs(fd - dx[t, v]) < 1e-7, (t, v)
    # through the projection: d_hidden = dX W, d_weight = dX^T h
    for (m, arr) in (("h", h), ("w", w)):
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += eps
            am[idx] -= eps
            hp, wp = (ap, w) if m == "h" else (h, ap)
            hm, wm = (am, w) if m == "h" else (h, am)
            fd = (_scores_objective(hp, wp, tau, y, a, b) - _scores_objective(hm, wm, tau, y, a, b)) / (2 * eps)
            ref = (dx @ w)[idx] if m == "h" else (dx.T @ h)[idx]
            assert abs(fd - ref) < 1e-7, (m, idx)


def test_vjp_invariants():
    rng = np.random.default_rng(32)
    x = rng.normal(0, 2, (6, 40))
    y = rng.integers(0, 40, 6)
    a, b = rng.normal(size=6), rng.normal(size=6)
    dx = oracle.logit_vjp(x, 1.3, y, a, b)
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-14)  # sum_v dp_v = 0 for both terms
    # a one-token vocabulary: logprob and entropy are constant, the gradient exactly 0
    assert (oracle.logit_vjp(x[:, :1], 1.0, np.zeros(6, int), a, b) == 0.0).all()
    # logprob alone: onehot - p; entropy alone at uniform logits: 0 (H is at its maximum)
    g = oracle.logit_vjp(x, 1.0, y, np.ones(6), None)
    p = np.exp(x - x.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(g, np.eye(40)[y] - p, atol=1e-15)
    assert np.abs(oracle.logit_vjp(np.zeros((2, 9)), 1.0, [0, 3], None, [1.0, 2.0])).max() < 1e-15
    # bad rows get zero rows
    bad = oracle.logit_vjp(np.array([[0.0, np.nan], [1.0, 2.0]]), 1.0, [0, 5], [1, 1], [1, 1])
    assert (bad == 0).all()
