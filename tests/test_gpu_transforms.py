"""GPU parity: top-k / top-p / min-p support, descriptor, dense ids and scores vs the fp64 oracle.

Support membership, support_len, threshold_logit, threshold_ties, dense ids
and status are compared bit-exactly on every row the oracle does not flag as
borderline (a cumulative mass within 1e-6 of top_p, or a weight within 1e-6
of min_p); borderline rows are counted and reported separately.
logprob / entropy / full_lse use the float tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_common import assert_close, bf16_tensor, oracle_by_rows, say, to_dev, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsa():
    import logprob_entropy_sampling_amd as m
    m.lib()
    return m


def _run(vsa, bits, tau, k, p, mp, y, cap, ld_pad=0):
    T, V = bits.shape
    if ld_pad:
        full = np.zeros((T, V + ld_pad), np.uint16)
        full[:, :V] = bits
        lg = bf16_tensor(full)[:, :V]
    else:
        lg = bf16_tensor(bits)
    return vsa.score_transforms(to_dev(np.asarray(y, np.int64)), lg, to_dev(np.asarray(k, np.int32)),
                                to_dev(np.asarray(p, np.float32)), to_dev(np.asarray(mp, np.float32)),
                                temperature=to_dev(np.asarray(tau, np.float32)), cap=cap)


def _compare(got, ref, cap, label, x64=None, tau=None, y=None):
    """Bit-exact descriptor, ids and status on every row that is not
    borderline; float scores within the tolerance.  On a borderline row the
    kernel's cut must lie in the oracle's band (top_p / min_p moved by up to
    1e-6); given x64 / tau / y, that row's descriptor, ids, status and scores
    are then checked against the oracle's outputs for the kernel's own cut."""
    T = len(ref["status"])
    border = ref["borderline_top_p"] | ref["borderline_min_p"]
    exact = ~border
    g = {k: (v.cpu().numpy() if v is not None else None) for k, v in got.items()}
    for name in ("support_len", "threshold_ties", "status"):
        bad = np.nonzero(exact & (g[name] != ref[name]))[0]
        assert bad.size == 0, f"{label}: {name} differs at rows {bad[:10]}: gpu {g[name][bad[:5]]} oracle {ref[name][bad[:5]]}"
    tl_g = g["threshold_logit"].astype(np.float64)
    same = (tl_g == ref["threshold_logit"]) | (np.isnan(tl_g) & np.isnan(ref["threshold_logit"]))
    bad = np.nonzero(exact & ~same)[0]
    assert bad.size == 0, f"{label}: threshold_logit differs at rows {bad[:10]}"
    if cap:
        bad = np.nonzero(exact & ~(g["support_ids"] == ref["support_ids"]).all(1))[0]
        assert bad.size == 0, f"{label}: support ids differ at rows {bad[:10]}"
    rows = np.nonzero(exact)[0]
    # the outputs are fp32: the expected value is the oracle's rounded to fp32
    # (a logprob beyond the fp32 range is -inf there too)
    f32 = lambda a: np.asarray(a, np.float64).astype(np.float32).astype(np.float64)  # noqa: E731
    with np.errstate(over="ignore"):
        assert_close(f"{label} logprob", g["logprob"], f32(ref["logprob"][rows]), rows=rows)
        assert_close(f"{label} entropy", g["entropy"], f32(ref["entropy"][rows]), rows=rows)
        assert_close(f"{label} full_lse", g["full_lse"], f32(ref["full_lse"]))
    brow = np.nonzero(border)[0]
    n_b = int(brow.size)
    if n_b:
        L = g["support_len"][brow]
        lo, hi = ref["support_len_lo"][brow], ref["support_len_hi"][brow]
        out = np.nonzero((L < lo) | (L > hi))[0]
        assert out.size == 0, f"{label}: borderline rows {brow[out][:10]} cut {L[out][:5]} outside [{lo[out][:5]}, {hi[out][:5]}]"
        if x64 is not None:
            tau_b = np.broadcast_to(np.asarray(tau, np.float64), (T,))[brow]
            forced = oracle.score_prefix_support(x64[brow], tau_b, L, np.asarray(y)[brow], cap=cap)
            for name in ("threshold_ties", "status"):
                assert np.array_equal(g[name][brow], forced[name]), f"{label}: borderline {name}"
            assert np.array_equal(g["threshold_logit"][brow].astype(np.float64), forced["threshold_logit"])
            if cap:
                assert np.array_equal(g["support_ids"][brow], forced["support_ids"]), f"{label}: borderline ids"
            with np.errstate(over="ignore"):
                assert_close(f"{label} borderline logprob", g["logprob"][brow], f32(forced["logprob"]))
                assert_close(f"{label} borderline entropy", g["entropy"][brow], f32(forced["entropy"]))
    mism = int(((g["support_len"] != ref["support_len"]) & border).sum())
    say(f"  {label}: {T} rows, {n_b} borderline ({mism} of them cut on the other side of the band, "
        f"{'all checked against that cut' if x64 is not None else 'cut inside the band'})")
    return n_b


def _support_sample(x64, tau, k, p, mp, u):
    """An in-support target per row: inverse CDF of the renormalised support distribution."""
    r = oracle.score_transforms(x64, tau, k, p, mp, np.zeros(len(x64), np.int64), cap=0)
    y = np.empty(len(x64), np.int64)
    for t in range(len(x64)):
        z = x64[t] / float(tau[t])
        order = np.lexsort((np.arange(z.size), -z))
        S = order[: int(r["support_len"][t])]
        w = np.exp(z[S] - z[S[0]])
        c = np.cumsum(w)
        y[t] = S[min(int(np.searchsorted(c, u[t] * c[-1], side="right")), S.size - 1)]
    return y


def test_workload_rows_full_vocab(vsa):
    say("transforms: 72 rows (two cycles of the 36 parameter combinations), V=151936, cap 64")
    c = workloads.make(5, T=72)
    x64 = oracle.logits_from_logits(c["logits"], "bf16")
    y = _support_sample(x64, c["temperature"], c["top_k"], c["top_p"], c["min_p"], c["u"])
    got = _run(vsa, c["logits"], c["temperature"], c["top_k"], c["top_p"], c["min_p"], y, 64)
    ref = oracle.score_transforms(x64, c["temperature"], c["top_k"], c["top_p"], c["min_p"], y, cap=64)
    assert (ref["status"] & oracle.ST_TARGET_OUTSIDE_SUPPORT == 0).all()
    n_b = _compare(got, ref, 64, "workload", x64, c["temperature"], y)
    assert n_b <= 8
    again = _run(vsa, c["logits"], c["temperature"], c["top_k"], c["top_p"], c["min_p"], y, 64)
    for k in ("logprob", "entropy", "support_len", "support_ids", "full_lse"):
        assert torch.equal(got[k], again[k]), k


@pytest.mark.parametrize("V", [1, 5, 37, 1000, 5003, 40000, 90000])
def test_small_and_medium_rows_with_ties(vsa, V):
    say(f"transforms: tied rows V={V}, every parameter combination")
    rng = np.random.default_rng(V)
    ks = [0, 1, 2, 5, V, V + 3]
    ps = [1.0, 0.9, 0.5, 0.1]
    mps = [0.0, 0.1, 0.5, 1.0]
    taus = [0.5, 1.0]
    combos = [(k, p, mp, tau) for k in ks for p in ps for mp in mps for tau in taus]
    T = len(combos)
    vals = rng.integers(-6, 7, size=(T, V)).astype(np.float32) * np.float32(0.375)
    bits = workloads.to_bf16_bits(vals)
    k = np.array([c[0] for c in combos], np.int32)
    p = np.array([c[1] for c in combos], np.float32)
    mp = np.array([c[2] for c in combos], np.float32)
    tau = np.array([c[3] for c in combos], np.float32)
    y = rng.integers(0, V, T)
    x64 = oracle.logits_from_logits(bits, "bf16")
    for cap in (0, 3, 64):
        got = _run(vsa, bits, tau, k, p, mp, y, cap)
        ref = oracle.score_transforms(x64, tau, k, p, mp, y, cap=cap)
        _compare(got, ref, cap, f"V={V} cap={cap}", x64, tau, y)


def test_unaligned_rows_and_neg_inf(vsa):
    say("transforms: unaligned rows (ld odd), -inf logits")
    rng = np.random.default_rng(4)
    T, V = 40, 3001
    vals = (rng.standard_normal((T, V)) * 2).astype(np.float32)
    vals[:, ::5] = -np.inf
    bits = workloads.to_bf16_bits(vals)
    k = rng.choice([0, 3, 20], T).astype(np.int32)
    p = rng.choice([1.0, 0.95, 0.5], T).astype(np.float32)
    mp = rng.choice([0.0, 0.05], T).astype(np.float32)
    tau = rng.choice([0.7, 1.0], T).astype(np.float32)
    y = rng.integers(0, V, T)
    x64 = oracle.logits_from_logits(bits, "bf16")
    got = _run(vsa, bits, tau, k, p, mp, y, 16, ld_pad=1)
    ref = oracle.score_transforms(x64, tau, k, p, mp, y, cap=16)
    _compare(got, ref, 16, "unaligned", x64, tau, y)


def test_bad_rows(vsa):
    say("transforms: BAD rows (NaN, +inf, all -inf, tau, top_p, min_p, target)")
    V = 100
    vals = np.zeros((9, V), np.float32)
    vals[0, 3] = np.nan
    vals[1, 4] = np.inf
    vals[2, :] = -np.inf
    bits = workloads.to_bf16_bits(vals)
    tau = np.array([1, 1, 1, 0, 1, 1, 1, 1, 1], np.float32)
    p = np.array([1, 1, 1, 1, 0, np.nan, 1, 1, 1], np.float32)
    mp = np.array([0, 0, 0, 0, 0, 0, 1.5, 0, 0], np.float32)
    y = np.array([0, 0, 0, 0, 0, 0, 0, V, 5], np.int64)
    k = np.zeros(9, np.int32)
    got = _run(vsa, bits, tau, k, p, mp, y, 4)
    ref = oracle.score_transforms(oracle.logits_from_logits(bits, "bf16"), tau, k, p, mp, y, cap=4)
    assert list(ref["status"]) == [4] * 8 + [oracle.ST_SUPPORT_TRUNCATED]  # last row: 100 ids, cap 4
    _compare(got, ref, 4, "bad")
    assert (got["support_ids"][:8] == -1).all()


def test_streaming_rows_special_values(vsa):
    """Rows longer than the register budget (the streaming kernel): NaN, +inf, a negative NaN, -inf,
    -0 next to +0 (one key), a row whose maximum is -0, a zero key whose -0 and +0 counts only
    together pass 16 bits.  V is odd, so rows alternate between
    16-byte-vector loads (even rows) and the per-element path (odd rows)."""
    say("transforms: streaming rows V=90001 with NaN / +inf / -NaN / -inf / signed zeros")
    rng = np.random.default_rng(17)
    T, V = 10, 90001
    vals = (rng.standard_normal((T, V)) * 2).astype(np.float32)
    bits = workloads.to_bf16_bits(vals)
    bits[0, 7] = 0x7FC0                     # NaN
    bits[1, V - 1] = 0x7F80                 # +inf in the last column
    bits[2, 12345] = 0xFFC0                 # negative NaN
    bits[3, ::3] = 0xFF80                   # -inf: legal
    bits[4, :] = np.where(rng.random(V) < 0.5, 0x8000, 0x0000)  # only signed zeros: one tie group
    bits[4, :50] = workloads.to_bf16_bits(np.abs(vals[4, :50]) + np.float32(0.5))
    bits[5, :] = workloads.to_bf16_bits(-np.abs(vals[5]) - np.float32(0.25))
    bits[5, rng.choice(V, 40, replace=False)] = 0x8000   # the row maximum is -0 (40 tokens)
    bits[5, rng.choice(V, 40, replace=False)] = 0x0000   # ... tied with +0
    bits[6, rng.choice(V, 300, replace=False)] = 0x8000
    bits[6, rng.choice(V, 300, replace=False)] = 0x0000
    zs = rng.permutation(V)[:89000]  # 45000 x -0 and 44000 x +0: each fits 16 bits, together they do not
    bits[8, zs[:45000]] = 0x8000
    bits[8, zs[45000:]] = 0x0000
    k = np.array([0, 0, 0, 20, 60, 30, 0, 5, 600, 1000], np.int32)  # row 8: the cut falls inside the zero key
    p = np.array([1, 1, 1, 0.9, 1, 1, 0.95, 0.8, 1, 1], np.float32)
    mp = np.array([0, 0, 0, 0.05, 0, 0, 0, 0, 0, 0], np.float32)
    tau = np.array([1, 1, 1, 0.7, 1, 1, 1, 0.7, 1, 1], np.float32)
    x64 = oracle.logits_from_logits(bits, "bf16")
    y = _support_sample(np.where(np.isnan(x64) | (x64 == np.inf), 0.0, x64), tau, k, p, mp, rng.random(T))
    got = _run(vsa, bits, tau, k, p, mp, y, 64)
    ref = oracle.score_transforms(x64, tau, k, p, mp, y, cap=64)
    assert list(ref["status"][:3] & oracle.ST_BAD_INPUT) == [oracle.ST_BAD_INPUT] * 3
    _compare(got, ref, 64, "streaming special values", x64, tau, y)


def test_streamed_rows_cap_paths(vsa):
    """Long rows at cap 2048 (count kernel + finish kernel, candidates from the
    stored per-thread units) and cap 2049 / 4096 (one-kernel streaming form),
    with targets on the threshold key so the id tie-break sweeps the row."""
    say("transforms: streamed rows V=100000, caps 2048 / 2049 / 4096, targets tied at the threshold")
    T, V = 6, 100000
    rng = np.random.default_rng(11)
    bits = workloads.to_bf16_bits((rng.standard_normal((T, V)) * 2.0).astype(np.float32))
    k = np.array([0, 3000, 50, 0, 2500, 0], np.int32)
    p = np.array([1.0, 1.0, 0.95, 0.9, 1.0, 1.0], np.float32)
    mp = np.array([0.0, 0.0, 0.0, 0.0, 0.001, 0.0], np.float32)
    tau = np.array([1.0, 0.7, 1.0, 1.3, 1.0, 1.0], np.float32)
    x64 = oracle.logits_from_logits(bits, "bf16")
    thr = oracle.score_transforms(x64, tau, k, p, mp, np.zeros(T, np.int64), cap=0)["threshold_logit"]
    y = rng.integers(0, V, T)
    for t in range(0, T, 2):  # every other row: a target whose logit is the threshold logit
        tied = np.nonzero(x64[t] == thr[t])[0]
        y[t] = tied[len(tied) // 2]
    for cap in (2048, 2049, 4096):
        got = _run(vsa, bits, tau, k, p, mp, y, cap)
        ref = oracle.score_transforms(x64, tau, k, p, mp, y, cap=cap)
        _compare(got, ref, cap, f"V={V} cap={cap}", x64, tau, y)


def test_streamed_rows_spread_over_many_segments(vsa):
    """Long rows whose keys spread over most of the 1024 key segments (random
    finite bf16 patterns over the whole finite range, subnormals to 2^127):
    more non-empty segments than the split path's record holds, so these rows
    go to the 32-bit stream kernel; segments whose weights cannot follow one
    geometric recurrence; and ties at the largest magnitudes.  The masses are
    fp64, so no tempered logit overflows."""
    say("transforms: V=100000 rows of random finite bf16 patterns (|x| < 2^128), caps 0 / 64 / 2048")
    T, V = 8, 100000
    rng = np.random.default_rng(12)
    sign = rng.integers(0, 2, size=(T, V)) << 15
    expo = rng.integers(0, 255, size=(T, V)) << 7  # biased exponents 0 .. 254: every finite bf16
    mant = rng.integers(0, 128, size=(T, V))
    bits = (sign | expo | mant).astype(np.uint16)
    bits[1] = np.where(np.arange(V) % 3 == 0, bits[1], bits[1] & 0x80FF)  # a third spread, the rest tiny
    bits[6, rng.choice(V, 5, replace=False)] = 0x7F7F  # more tied maxima at the largest finite bf16
    bits[7, rng.choice(V, 3, replace=False)] = 0x5D80  # tied maxima at 2^60 ...
    bits[7] = np.where(bits[7] == 0x5D80, bits[7], bits[7] & 0x5CFF)  # ... the rest below 2^58
    k = np.array([0, 0, 40, 1000, 0, 5, 0, 0], np.int32)
    p = np.array([1.0, 0.9, 1.0, 0.5, 1.0, 1.0, 0.6, 0.9], np.float32)
    mp = np.array([0.0, 0.0, 0.0, 0.0, 1e-30, 0.0, 0.0, 0.0], np.float32)
    tau = np.array([1.0, 1.0, 0.5, 2.0, 1.0, 1e-3, 1.0, 1.0], np.float32)
    x64 = oracle.logits_from_logits(bits, "bf16")
    y = rng.integers(0, V, T)
    y[6] = int(np.nonzero(bits[6] == 0x7F7F)[0][1])
    y[7] = int(np.nonzero(bits[7] == 0x5D80)[0][2])
    for cap in (0, 64, 2048):
        got = _run(vsa, bits, tau, k, p, mp, y, cap)
        ref = oracle.score_transforms(x64, tau, k, p, mp, y, cap=cap)
        for t in (6, 7):  # top-p keeps some of the tied maxima: a uniform support
            assert ref["support_len"][t] >= 2 and not ref["borderline_top_p"][t]
            assert abs(ref["entropy"][t] - np.log(ref["support_len"][t])) < 1e-12
        _compare(got, ref, cap, f"spread V={V} cap={cap}", x64, tau, y)


def _segment_rows(rng, T, V, n_exp):
    """Rows of bf16 logits whose keys fill about 4 * n_exp[t] of the 1024 key
    segments: both signs, biased exponents 100 .. 100 + n_exp[t] - 1, every
    mantissa (a segment is a sign, an exponent and the top mantissa bit)."""
    bits = np.empty((T, V), np.uint16)
    for t in range(T):
        sign = rng.integers(0, 2, size=V) << 15
        expo = (100 + rng.integers(0, n_exp[t], size=V)) << 7
        bits[t] = (sign | expo | rng.integers(0, 128, size=V)).astype(np.uint16)
    return bits


def test_split_path_segment_counts_around_the_record(vsa):
    """Long rows (the split path) with 64 to 520 non-empty key segments: up to
    128 the finish kernel keeps every segment's counts in LDS, up to 256 it also
    reads them from the row's record, beyond 256 the record cannot hold them
    and the row is redone by the 32-bit stream kernel.  Descriptor, ids and
    status bit-exact, scores within the tolerance, at caps 0 and 64."""
    say("transforms: V=100000 rows with 64 .. 520 non-empty key segments (record limit 256), caps 0 / 64")
    T, V = 8, 100000
    rng = np.random.default_rng(31)
    n_exp = [16, 32, 40, 60, 64, 65, 80, 130]  # about 4 segments per exponent: 64 .. 520 segments
    bits = _segment_rows(rng, T, V, n_exp)
    keys = np.where(bits >> 15, 0xFFFF - bits.astype(np.int64), bits.astype(np.int64) | 0x8000)
    nseg = [len(np.unique(keys[t] >> 6)) for t in range(T)]
    assert min(nseg) <= 128 and any(128 < n <= 256 for n in nseg) and max(nseg) > 256, nseg
    k = np.array([0, 20, 0, 50, 0, 0, 1000, 0], np.int32)
    p = np.array([0.9, 1.0, 0.5, 0.95, 1.0, 0.8, 1.0, 0.9], np.float32)
    mp = np.array([0.0, 0.0, 0.05, 0.0, 0.0, 0.0, 0.0, 1e-3], np.float32)
    tau = np.array([1.0, 0.7, 1.0, 2.0, 1.0, 1.0, 0.5, 1.0], np.float32)
    x64 = oracle.logits_from_logits(bits, "bf16")
    y = rng.integers(0, V, T)
    for cap in (0, 64):
        got = _run(vsa, bits, tau, k, p, mp, y, cap)
        ref = oracle.score_transforms(x64, tau, k, p, mp, y, cap=cap)
        _compare(got, ref, cap, f"segments {nseg} cap={cap}", x64, tau, y)


def test_identity_and_singleton(vsa):
    say("transforms: identity program == full-vocabulary scoring; top-k 1 == exact zeros")
    c = workloads.make(5, T=8, V=30000)
    T, V = 8, 30000
    y = torch.from_numpy(c["targets"]).cuda()
    lg = bf16_tensor(c["logits"])
    tau = to_dev(c["temperature"])
    ident = vsa.score_transforms(y, lg, to_dev(np.zeros(T, np.int32)), to_dev(np.ones(T, np.float32)),
                                 to_dev(np.zeros(T, np.float32)), temperature=tau)
    full = vsa.score_full(y, logits=lg, temperature=tau)
    assert (ident["support_len"] == V).all()
    assert_close("identity logprob", ident["logprob"].cpu().numpy(), full["logprob"].cpu().numpy().astype(np.float64))
    assert_close("identity entropy", ident["entropy"].cpu().numpy(), full["entropy"].cpu().numpy().astype(np.float64))
    one = vsa.score_transforms(y, lg, to_dev(np.ones(T, np.int32)), to_dev(np.ones(T, np.float32)),
                               to_dev(np.zeros(T, np.float32)), temperature=tau, cap=2)
    assert (one["support_len"] == 1).all()
    assert (one["entropy"] == 0).all() and (one["logprob"] == 0).all()  # targets are the row argmax
    assert (one["support_ids"][:, 0].cpu() == y.cpu()).all() and (one["support_ids"][:, 1] == -1).all()


def test_all_equal_long_row_uses_32bit_counts(vsa):
    say("transforms: 151936 equal logits (a key count beyond 16 bits), large tie groups")
    V = 151936
    bits = workloads.to_bf16_bits(np.full((4, V), 0.75, np.float32))
    k = np.array([5, 0, 0, 0], np.int32)
    p = np.array([1.0, 0.50001, 1.0, 0.25], np.float32)
    mp = np.zeros(4, np.float32)
    tau = np.ones(4, np.float32)
    y = np.array([3, 75969, 151935, 40000], np.int64)
    got = _run(vsa, bits, tau, k, p, mp, y, 64)
    x64 = oracle.logits_from_logits(bits, "bf16")
    ref = oracle.score_transforms(x64, tau, k, p, mp, y, cap=64)
    assert list(ref["support_len"][:3]) == [5, 75970, V]  # row 3 sits exactly on a cut (borderline)
    _compare(got, ref, 64, "all-equal", x64, tau, y)
    assert list(got["support_ids"][0, :6].cpu().numpy()) == [0, 1, 2, 3, 4, -1]
    assert list(got["support_ids"][1, :64].cpu().numpy()) == list(range(64))


class _WidenedRows:
    """x64[rows] of a bf16 logits array, widened only for the rows asked for."""

    def __init__(self, bits):
        self.bits = bits

    def __getitem__(self, rows):
        return oracle.logits_from_logits(self.bits, "bf16", rows=np.atleast_1d(rows))


def test_full_size_all_rows(vsa):
    say("transforms: full workload T=2048 V=151936 cap 64, every row vs the oracle, in-support sampled targets")
    c = workload(5)
    T = c["T"]
    k, p, mp, tau = c["top_k"], c["top_p"], c["min_p"], c["temperature"]
    xr = _WidenedRows(c["logits"])
    y = oracle_by_rows(lambda r: {"y": _support_sample(xr[r], tau[r], k[r], p[r], mp[r], c["u"][r])}, T)["y"]
    got = _run(vsa, c["logits"], tau, k, p, mp, y, 64)
    again = _run(vsa, c["logits"], tau, k, p, mp, y, 64)
    for key in got:
        assert torch.equal(got[key], again[key]), key
    ref = oracle_by_rows(lambda r: oracle.score_transforms(xr[r], tau[r], k[r], p[r], mp[r], y[r], cap=64), T)
    assert (ref["status"] & (oracle.ST_TARGET_OUTSIDE_SUPPORT | oracle.ST_BAD_INPUT) == 0).all()
    # about a tenth of the rows have a prefix mass within 1e-6 of top_p (a few
    # hundred thousand tokens carry masses of 1e-5 or less); each of them is
    # checked against the cut the kernel chose
    n_b = _compare(got, ref, 64, "full size", xr, tau, y)
    assert n_b < T // 4
