"""Pins of the oracle's float64 -> bf16 rounding (the logits the transform
program ranks on a hidden/weight source, xorl issue #71 "Proposed direction"
item 3), against a brute-force nearest search over every bf16 number and
IEEE special cases worked by hand."""

import numpy as np

import oracle

pytestmark = []


def _table():
    """Every non-NaN bf16 value (float64) with its bit pattern, ascending; the
    infinities included, and +/-0 both kept."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.widen_bf16(bits)
    keep = ~np.isnan(vals)
    order = np.lexsort((bits[keep], vals[keep]))
    return vals[keep][order], bits[keep][order]


def _nearest(x, vals, bits):
    """Brute force: the closest bf16 value; on a tie the one with an even last
    significand bit; beyond the largest finite value, the infinity is the next
    candidate at 2^128 (the rule of rounding with an unbounded exponent)."""
    out = np.empty(x.shape, np.uint16)
    big = 2.0 ** 128
    for i, xv in enumerate(x):
        if xv == 0:
            out[i] = 0x8000 if np.signbit(xv) else 0
            continue
        cand_v = vals.copy()
        cand_v[cand_v == np.inf] = big
        cand_v[cand_v == -np.inf] = -big
        d = np.abs(cand_v - xv)
        best = d.min()
        idx = np.nonzero(d == best)[0]
        ids = bits[idx]
        if len(set(ids.tolist()) - {0, 0x8000}) == 0:  # rounds to zero: keep the sign
            out[i] = 0x8000 if xv < 0 else 0
            continue
        ids = np.array([b for b in ids if b not in (0, 0x8000)] or ids)
        even = ids[(ids & 1) == 0]
        out[i] = even[0] if even.size else ids[0]
    return out


def test_matches_brute_force_nearest():
    vals, bits = _table()
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.normal(0, 2, 300),
        rng.normal(0, 1, 100) * 2.0 ** rng.integers(-140, 127, 100),
        # exact midpoints between neighbours: the ties
        (oracle.widen_bf16(rng.integers(0, 0x7F7F, 100).astype(np.uint16)) +
         oracle.widen_bf16((rng.integers(0, 0x7F7F, 100) + 1).astype(np.uint16))) / 2,
    ])
    x = np.concatenate([x, -x])
    assert np.array_equal(oracle.round_f64_to_bf16(x), _nearest(x, vals, bits))


def test_agrees_with_the_float32_rounding_on_float32_values():
    # a float32 input needs one rounding either way
    rng = np.random.default_rng(1)
    f = (rng.normal(0, 1, 20000) * 2.0 ** rng.integers(-130, 120, 20000)).astype(np.float32)
    assert np.array_equal(oracle.round_f64_to_bf16(f.astype(np.float64)), oracle.round_f32_to_bf16(f))


def test_special_cases():
    r = lambda v: int(oracle.round_f64_to_bf16(np.array([v]))[0])  # noqa: E731
    assert r(1.0) == 0x3F80
    assert r(1.0 + 2.0 ** -8) == 0x3F80            # tie: down to the even 1.0
    assert r(1.0 + 3 * 2.0 ** -8) == 0x3F82        # tie: up to the even 1 + 2^-6
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # just past the midpoint: a double-rounding trap for fp32
    assert r(-1.5) == 0xBFC0
    big = 2.0 ** 128 - 2.0 ** 120                  # the largest finite bf16
    assert r(big) == 0x7F7F
    assert r(big + 2.0 ** 119 - 2.0 ** 100) == 0x7F7F
    assert r(big + 2.0 ** 119) == 0x7F80           # the midpoint to 2^128 rounds to even: +inf
    assert r(-(2.0 ** 200)) == 0xFF80
    assert r(2.0 ** -133) == 0x0001                # the smallest subnormal
    assert r(2.0 ** -134) == 0x0000                # tie with 0: even
    assert r(3 * 2.0 ** -134) == 0x0002            # tie: up to the even pattern
    assert r(-(2.0 ** -140)) == 0x8000             # underflow keeps the sign
    assert r(-0.0) == 0x8000
    assert r(float("inf")) == 0x7F80 and r(float("-inf")) == 0xFF80
    assert r(float("nan")) == 0x7FC0


def test_projected_logits_are_the_rounded_projection():
    # on a grid where every sum is exact, bf16(fp64 sum) is also bf16 of the
    # exact value computed by hand
    rng = np.random.default_rng(2)
    h = oracle.round_f32_to_bf16(rng.integers(-8, 9, (3, 16)).astype(np.float32) / 4)
    w = oracle.round_f32_to_bf16(rng.integers(-8, 9, (5, 16)).astype(np.float32) / 128)
    exact = np.array([[sum(oracle.widen_bf16(h)[t, k] * oracle.widen_bf16(w)[v, k] for k in range(16))
                       for v in range(5)] for t in range(3)])
    got = oracle.bf16_logits_from_hidden(h, "bf16", w)
    assert np.array_equal(got, oracle.round_f32_to_bf16(exact.astype(np.float32)))
