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


def test_ties_at_large_magnitude():
    # a support of n equal logits far from zero: renormalised uniform, so
    # entropy ln n and logprob -ln n at any magnitude; one id far below the
    # others adds nothing
    for mag in (2.0 ** 45, 2.0 ** 60, -(2.0 ** 60), 3.0e38):
        x = np.zeros((1, 50))
        x[0, [3, 9, 20]] = mag
        x[0, 30] = mag - abs(mag) * 0.5
        ids = np.array([[20, 3, 30, 9, -1]])
        r = oracle.score_support(lambda t, cols: x[t, cols], 50, ids, 1.0, [9])
        assert abs(r["entropy"][0] - math.log(3)) < 1e-12, mag
        assert abs(r["logprob"][0] + math.log(3)) < 1e-12, mag
        r = oracle.score_support(lambda t, cols: x[t, cols], 50, ids[:, 1:2], 1.0, [3])
        assert r["entropy"][0] == 0.0 and r["logprob"][0] == 0.0


def _support_objective(h64, w64, ids, tau, y, a, b):
    """sum_t a_t logprob_t + b_t H_t of score_support over x = h w^T (float64), where finite."""
    r = oracle.score_support(lambda t, cols: h64[t] @ w64[np.asarray(cols)].T, w64.shape[0], ids, tau, y)
    lp = np.where(np.isfinite(r["logprob"]), r["logprob"], 0.0)  # a -inf logprob is a constant
    ent = np.where(np.isfinite(r["entropy"]), r["entropy"], 0.0)
    return float(np.sum(a * lp + b * ent))


def test_support_vjp_matches_finite_differences():
    # the gradient of sum a logprob_S + b H_S with respect to the hidden state
    # and every weight row, against central differences of score_support itself
    rng = np.random.default_rng(41)
    T, H, V, W = 5, 6, 11, 6
    hb = oracle.round_f32_to_bf16(rng.normal(0, 1, (T, H)).astype(np.float32))
    wb = oracle.round_f32_to_bf16(rng.normal(0, 0.5, (V, H)).astype(np.float32))
    h64, w64 = oracle.widen_bf16(hb), oracle.widen_bf16(wb)
    ids = np.full((T, W), -1, np.int64)
    ids[0, :4] = [3, 7, 1, 9]          # target inside
    ids[1, [0, 2, 5]] = [2, 10, 4]     # padding in the middle, target outside the support
    ids[2, :1] = [5]                   # singleton
    ids[3, :6] = [0, 1, 2, 3, 4, 5]
    ids[4, 1:3] = [8, 6]
    y = np.array([7, 0, 5, 4, 6])
    tau = np.array([1.0, 0.7, 1.3, 0.9, 2.0])
    a = np.array([1.0, -0.5, 2.0, 0.7, -1.2])
    b = np.array([0.3, 1.0, -0.8, 0.5, 0.9])
    g = oracle.score_support_vjp(hb, "bf16", wb, ids, tau, y, a, b)
    eps = 1e-6
    for (name, arr, ref) in (("hidden", h64, g["d_hidden"]), ("weight", w64, g["d_weight"])):
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += eps
            am[idx] -= eps
            hp, wp = (ap, w64) if name == "hidden" else (h64, ap)
            hm, wm = (am, w64) if name == "hidden" else (h64, am)
            fd = (_support_objective(hp, wp, ids, tau, y, a, b) - _support_objective(hm, wm, ids, tau, y, a, b)) / (2 * eps)
            assert abs(fd - ref[idx]) < 1e-7, (name, idx, fd, ref[idx])


def test_support_vjp_singleton_and_empty_rows_are_exactly_zero():
    rng = np.random.default_rng(42)
    T, H, V = 4, 8, 20
    hb = oracle.round_f32_to_bf16(rng.normal(0, 1, (T, H)).astype(np.float32))
    wb = oracle.round_f32_to_bf16(rng.normal(0, 0.5, (V, H)).astype(np.float32))
    ids = np.array([[7, -1, -1], [-1, -1, -1], [3, 3, -1], [25, 1, -1]])  # singleton, empty, repeated, id >= V
    y = np.array([7, 0, 3, 1])
    g = oracle.score_support_vjp(hb, "bf16", wb, ids, 1.0, y, np.ones(T), np.ones(T))
    assert (g["d_hidden"] == 0).all() and (g["d_weight"] == 0).all() and (g["d_support"] == 0).all()


def test_full_support_vjp_equals_full_vocabulary_vjp():
    # a support holding every id (in any order) is the full vocabulary
    rng = np.random.default_rng(43)
    T, H, V = 4, 16, 30
    hb = oracle.round_f32_to_bf16(rng.normal(0, 1, (T, H)).astype(np.float32))
    wb = oracle.round_f32_to_bf16(rng.normal(0, 0.5, (V, H)).astype(np.float32))
    ids = np.stack([rng.permutation(V) for _ in range(T)])
    y = rng.integers(0, V, T)
    tau = np.array([1.0, 0.6, 1.7, 1.1])
    a, b = rng.normal(0, 1, T), rng.normal(0, 1, T)
    s = oracle.score_support_vjp(hb, "bf16", wb, ids, tau, y, a, b)
    f = oracle.score_full_vjp(hb, "bf16", wb, tau, y, a, b)
    assert np.allclose(s["d_hidden"], f["d_hidden"], rtol=1e-12, atol=1e-14)
    assert np.allclose(s["d_weight"], f["d_weight"], rtol=1e-12, atol=1e-14)
    for t in range(T):
        assert np.allclose(s["d_support"][t], f["d_logits"][t, ids[t]], rtol=1e-12, atol=1e-15)


def test_support_vjp_weight_rows_and_outside_target():
    rng = np.random.default_rng(44)
    T, H, V, W = 6, 8, 40, 5
    hb = oracle.round_f32_to_bf16(rng.normal(0, 1, (T, H)).astype(np.float32))
    wb = oracle.round_f32_to_bf16(rng.normal(0, 0.5, (V, H)).astype(np.float32))
    ids = np.stack([rng.choice(V, W, replace=False) for _ in range(T)])
    y = ids[:, 0].copy()
    y[2] = int(np.setdiff1d(np.arange(V), ids[2])[0])  # outside its support
    a, b = rng.normal(0, 1, T), rng.normal(0, 1, T)
    full = oracle.score_support_vjp(hb, "bf16", wb, ids, 1.0, y, a, b)
    some = oracle.score_support_vjp(hb, "bf16", wb, ids, 1.0, y, a, b, weight_rows=[ids[1, 2], 0, ids[4, 4]])
    assert np.array_equal(some["d_weight"], full["d_weight"][[ids[1, 2], 0, ids[4, 4]]])
    # outside the support only the entropy term remains
    only_b = oracle.score_support_vjp(hb[2:3], "bf16", wb, ids[2:3], 1.0, y[2:3], np.zeros(1), b[2:3])
    assert np.allclose(full["d_hidden"][2], only_b["d_hidden"][0], rtol=0, atol=1e-15)
