"""GPU parity: draft/target softmax L1 distance and accept_rate vs the fp64 oracle."""

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


def test_workload_rows(vsa):
    say("l1: 24 rows of the transforms/draft recipe, V=151936 bf16")
    c = workloads.make(5, T=24)
    got = vsa.l1_distance(bf16_tensor(c["logits"]), bf16_tensor(c["draft"]))
    ref = oracle.l1_distance(oracle.logits_from_logits(c["logits"], "bf16"),
                             oracle.logits_from_logits(c["draft"], "bf16"))
    assert_close("l1", got["l1"].cpu().numpy(), ref["l1"])
    assert_close("accept_rate", got["accept_rate"].cpu().numpy(), ref["accept_rate"])


def test_identical_is_exactly_zero(vsa):
    say("l1: identical rows -> exactly 0 and accept 1")
    c = workloads.make(5, T=8, V=40000)
    t = bf16_tensor(c["logits"])
    got = vsa.l1_distance(t, t.clone())
    assert (got["l1"] == 0).all() and (got["accept_rate"] == 1).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_and_bounds(vsa, dtype):
    say(f"l1: ragged V, far-apart rows, NaN rows, dtype={dtype}")
    rng = np.random.default_rng(3)
    T, V = 20, 30001
    a = (rng.standard_normal((T, V)) * 2).astype(np.float32)
    b = a + (rng.standard_normal((T, V)) * rng.uniform(0, 6, (T, 1))).astype(np.float32)
    b[3] = -30.0
    b[3, 5] = 30.0
    a[3] = -30.0
    a[3, 9] = 30.0
    a[7, 100] = np.nan
    b[8] = -np.inf
    if dtype == "bf16":
        ab, bb = workloads.to_bf16_bits(a), workloads.to_bf16_bits(b)
        ta, tb = bf16_tensor(ab), bf16_tensor(bb)
        a64, b64 = oracle.logits_from_logits(ab, "bf16"), oracle.logits_from_logits(bb, "bf16")
    else:
        ta, tb = to_dev(a), to_dev(b)
        a64, b64 = a.astype(np.float64), b.astype(np.float64)
    got = vsa.l1_distance(ta, tb)
    ref = oracle.l1_distance(a64, b64)
    assert_close("l1", got["l1"].cpu().numpy(), ref["l1"])
    assert_close("accept_rate", got["accept_rate"].cpu().numpy(), ref["accept_rate"])
    l1 = got["l1"].cpu().numpy()
    fin = np.isfinite(l1)
    assert (l1[fin] <= 2.0).all() and (l1[fin] >= 0).all()
    sym = vsa.l1_distance(tb, ta)
    assert torch.allclose(sym["l1"][fin], got["l1"][fin], atol=2e-6)


def test_full_size_all_rows(vsa):
    say("l1: full workload T=2048 V=151936 bf16, every row vs the oracle; determinism")
    c = workload(5)
    got = vsa.l1_distance(bf16_tensor(c["logits"]), bf16_tensor(c["draft"]))
    again = vsa.l1_distance(bf16_tensor(c["logits"]), bf16_tensor(c["draft"]))
    assert torch.equal(got["l1"], again["l1"]) and torch.equal(got["accept_rate"], again["accept_rate"])
    ref = oracle_by_rows(lambda r: oracle.l1_distance(oracle.logits_from_logits(c["logits"], "bf16", rows=r),
                                                      oracle.logits_from_logits(c["draft"], "bf16", rows=r)), c["T"])
    assert_close("l1", got["l1"].cpu().numpy(), ref["l1"])
    assert_close("accept_rate", got["accept_rate"].cpu().numpy(), ref["accept_rate"])


def _l1_case(vsa, a, b, ld_pad=0):
    ab, bb = workloads.to_bf16_bits(a), workloads.to_bf16_bits(b)
    if ld_pad:
        T, V = ab.shape
        ab = np.concatenate([ab, np.zeros((T, ld_pad), ab.dtype)], axis=1)
        bb = np.concatenate([bb, np.zeros((T, ld_pad), bb.dtype)], axis=1)
        ta, tb = bf16_tensor(ab)[:, :V], bf16_tensor(bb)[:, :V]
        ab, bb = ab[:, :V], bb[:, :V]
    else:
        ta, tb = bf16_tensor(ab), bf16_tensor(bb)
    got = vsa.l1_distance(ta, tb)
    ref = oracle.l1_distance(oracle.logits_from_logits(ab, "bf16"), oracle.logits_from_logits(bb, "bf16"))
    assert_close("l1", got["l1"].cpu().numpy(), ref["l1"])
    assert_close("accept_rate", got["accept_rate"].cpu().numpy(), ref["accept_rate"])
    return got


def test_resident_rows_more_than_cus(vsa):
    # one workgroup per CU walks several rows: a NaN row and an all -inf draft
    # row must not disturb the rows the same workgroup takes after them
    T, V = 300, 100003
    say(f"l1 resident form: T={T} V={V} bf16 (tail of 3), bad rows 5 and 6, identical row 7")
    rng = np.random.default_rng(11)
    a = (rng.standard_normal((T, V)) * 2).astype(np.float32)
    b = (a + rng.standard_normal((T, V)) * rng.uniform(0, 4, (T, 1))).astype(np.float32)
    a[5, 77] = np.nan
    b[6] = -np.inf
    b[7] = a[7]
    b[8] = -20.0
    b[8, V - 1] = 20.0  # all the draft mass on the last (tail) element
    got = _l1_case(vsa, a, b)
    l1 = got["l1"].cpu().numpy()
    assert np.isnan(l1[5]) and np.isnan(l1[6]) and l1[7] == 0.0
    assert np.isfinite(l1[np.r_[0:5, 8:T]]).all()


@pytest.mark.parametrize("V", [65537, 131072, 155648, 155655, 155656])
def test_resident_bounds(vsa, V):
    # the smallest and largest rows of the resident form, and the first row
    # length past it (two-pass form)
    say(f"l1 resident bounds: T=5 V={V} bf16")
    rng = np.random.default_rng(V)
    a = (rng.standard_normal((5, V)) * 3).astype(np.float32)
    b = (a + rng.standard_normal((5, V))).astype(np.float32)
    b[1] = a[1]
    a[2, :] = -np.inf
    a[2, V // 2] = 1.0  # a one-hot target
    a[3] = np.float32(0.25)  # a uniform target
    got = _l1_case(vsa, a, b)
    assert float(got["l1"][1]) == 0.0


@pytest.mark.parametrize("pad", [8, 5])
def test_resident_leading_dimension(vsa, pad):
    # ld = V + 8 keeps rows 16-byte aligned (resident form); ld = V + 5 does not
    # (two-pass form)
    T, V = 40, 151936
    say(f"l1 leading dimension: T={T} V={V} ld=V+{pad}")
    rng = np.random.default_rng(pad)
    a = (rng.standard_normal((T, V)) * 2).astype(np.float32)
    b = (a + rng.standard_normal((T, V)) * 0.5).astype(np.float32)
    _l1_case(vsa, a, b, ld_pad=pad)


@pytest.mark.parametrize("V", [1000, 100003, 151936])
def test_ties_at_large_magnitude(vsa, V):
    # tied maxima far from zero: the target's mass split over 2 ids, the
    # draft's over 4 (a superset) gives L1 = 1 at any magnitude.  Maxima past
    # 2^13 in base-2 units take the accurate exponent form (the resident form
    # hands such rows to the redo kernel); row 0 stays small for contrast.
    say(f"l1: tied maxima at 2^12 .. 2^120 (bf16), V={V}")
    mags = [4.0, 2.0 ** 12, 2.0 ** 20, 2.0 ** 60, 2.0 ** 100, 2.0 ** 120, -(2.0 ** 100)]
    T = len(mags)
    rng = np.random.default_rng(V)
    a = np.zeros((T, V), np.float32)
    b = np.zeros((T, V), np.float32)
    for t, mag in enumerate(mags):
        base = mag - abs(mag) * 0.5 if mag > 0 else 2.0 * mag
        a[t] = base
        b[t] = base
        ids = rng.choice(V, 4, replace=False)
        a[t, ids[:2]] = mag
        b[t, ids] = mag
    got = _l1_case(vsa, a, b)
    l1 = got["l1"].cpu().numpy()
    assert np.all(np.abs(l1[1:] - 1.0) < 2e-3), l1
