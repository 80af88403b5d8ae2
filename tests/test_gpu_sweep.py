"""GPU parity sweep: seeded random shapes, dtypes, strides, value mixes and
parameters for every entry point, against the fp64 oracle.

Each case prints its seed and shape before running.  Magnitudes: see
``_values`` (every finite bf16 value for the transforms, bf16 up to 2^123 for
the fp32 kernels, |x| < 2^7 for fp32 logits).
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import assert_close, bf16_tensor, say, to_dev
from tests.test_gpu_support import _cmp as _cmp_support
from tests.test_gpu_transforms import _compare as _cmp_transforms
from tests.test_gpu_transforms import _run as _run_transforms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsa():
    import logprob_entropy_sampling_amd as m
    m.lib()
    return m


def _values(rng, kind, shape, wide=False, dtype="bf16"):
    """fp32 logits of one of several mixes.

    Magnitudes: the sampling transforms (fp64 masses, ``wide``) take every
    finite value; the fp32 kernels take bf16 logits up to 2^123, where every
    difference |x_u - x_v| * log2(e) / tau of two logits of a row stays inside
    the fp32 range for every tau >= 0.3 used here; fp32 logits stay within |x| < 2^7, the range where the fp32
    rounding of x * log2(e) / tau (about |x / tau| * 2^-24 per term) meets the
    float tolerance.
    """
    if kind == "huge" and dtype != "bf16":
        kind = "ties"
    if kind == "normal":
        x = rng.standard_normal(shape) * rng.choice([0.05, 1.0, 4.0])
    elif kind == "ties":
        x = rng.integers(-4, 5, size=shape) * 0.5
    elif kind == "peaked":
        x = rng.standard_normal(shape) * 0.5
        spikes = rng.random(shape) < 0.001
        x[spikes] += 20.0
    elif kind == "neg_inf":
        x = rng.standard_normal(shape) * 2.0
        x[rng.random(shape) < 0.3] = -np.inf
    elif kind == "zeros":
        x = rng.choice([-0.0, 0.0, 1.0, -1.0], size=shape, p=[0.3, 0.3, 0.2, 0.2])
    elif kind == "spread":  # random exponents: subnormal to large magnitudes in one row
        lo, hi = (-133, 127) if wide else ((-133, 123) if dtype == "bf16" else (-40, 7))
        e = rng.integers(lo, hi, size=shape).astype(np.float64)
        x = np.sign(rng.standard_normal(shape)) * rng.uniform(1.0, 1.99, shape) * np.exp2(e)
    elif kind == "huge":  # small integers times 2^E, E up to 121: tied maxima far from zero
        E = float(rng.integers(20, 122 if not wide else 125))
        x = rng.integers(-3, 4, size=shape) * np.exp2(E)
    else:
        raise ValueError(kind)
    return np.asarray(x, dtype=np.float32)


KINDS = ["normal", "ties", "peaked", "neg_inf", "zeros", "spread", "huge"]


@pytest.mark.parametrize("seed", range(32))
def test_sweep_logits_full(vsa, seed):
    rng = np.random.default_rng(5000 + seed)
    T = int(rng.integers(1, 8))
    V = int(rng.choice([1, 2, 7, 100, 4097, 65536, 150001]))
    dtype = str(rng.choice(["bf16", "f32"]))
    pad = int(rng.choice([0, 1, 8]))
    kind = str(rng.choice(KINDS))
    say(f"sweep logits_full seed={seed}: T={T} V={V} {dtype} ld_pad={pad} values={kind}")
    x = _values(rng, kind, (T, V + pad), dtype=dtype)
    tau = rng.uniform(0.3, 2.0, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    y[0] = V - 1
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x)
        lg = bf16_tensor(bits)[:, :V]
        x64 = oracle.logits_from_logits(bits, "bf16")[:, :V]
    else:
        lg = to_dev(x)[:, :V]
        x64 = oracle.logits_from_logits(x, "f32")[:, :V]
    got = vsa.score_full(to_dev(y), logits=lg, temperature=to_dev(tau))
    ref = oracle.score_full(x64, tau, y)
    st = got["status"].cpu().numpy()
    assert np.array_equal(st, ref["status"]), f"status {st} vs {ref['status']}"
    for k in ("lse", "logprob", "entropy"):
        assert_close(k, got[k].cpu().numpy(), ref[k])


@pytest.mark.parametrize("seed", range(12))
def test_sweep_fused(vsa, seed):
    rng = np.random.default_rng(6000 + seed)
    T = int(rng.integers(1, 300))
    H = int(rng.choice([8, 24, 64, 128, 200, 264]))
    V = int(rng.choice([1, 17, 300, 5000]))
    hdt = str(rng.choice(["bf16", "f32"]))
    say(f"sweep fused seed={seed}: T={T} H={H} V={V} hidden {hdt}")
    h = rng.standard_normal((T, H)).astype(np.float32)
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * 0.2).astype(np.float32))
    tau = rng.uniform(0.5, 1.5, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    if hdt == "bf16":
        hb = workloads.to_bf16_bits(h)
        hid = bf16_tensor(hb)
        x = oracle.logits_from_hidden(hb, "bf16", wb)
    else:
        hid = to_dev(h)
        x = oracle.logits_from_hidden(h, "f32", wb)
    got = vsa.score_full(to_dev(y), hidden=hid, weight=bf16_tensor(wb), temperature=to_dev(tau))
    ref = oracle.score_full(x, tau, y)
    assert np.array_equal(got["status"].cpu().numpy(), ref["status"])
    for k in ("lse", "logprob", "entropy"):
        assert_close(k, got[k].cpu().numpy(), ref[k])


@pytest.mark.parametrize("seed", range(48))
def test_sweep_transforms(vsa, seed):
    rng = np.random.default_rng(7000 + seed)
    T = int(rng.integers(2, 8))
    V = int(rng.choice([1, 3, 64, 1000, 30001, 81920, 81921, 100003, 140000]))
    kind = str(rng.choice(KINDS))
    cap = int(rng.choice([0, 1, 7, 64, 300, 2048, 3000]))
    say(f"sweep transforms seed={seed}: T={T} V={V} values={kind} cap={cap}")
    bits = workloads.to_bf16_bits(_values(rng, kind, (T, V), wide=True))
    k = rng.choice([0, 1, 5, 50, V, V + 3], size=T).astype(np.int32)
    p = np.where(rng.random(T) < 0.5, 1.0, rng.uniform(0.05, 0.99, T)).astype(np.float32)
    mp = np.where(rng.random(T) < 0.5, 0.0, 10.0 ** rng.uniform(-6, -0.1, T)).astype(np.float32)
    tau = rng.uniform(0.1, 3.0, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    got = _run_transforms(vsa, bits, tau, k, p, mp, y, cap)
    ref = oracle.score_transforms(oracle.logits_from_logits(bits, "bf16"), tau, k, p, mp, y, cap=cap)
    _cmp_transforms(got, ref, cap, f"sweep seed={seed}")


@pytest.mark.parametrize("seed", range(24))
def test_sweep_l1(vsa, seed):
    rng = np.random.default_rng(8000 + seed)
    T = int(rng.integers(1, 8))
    V = int(rng.choice([1, 2, 9, 1000, 65537, 151936]))
    dtype = str(rng.choice(["bf16", "f32"]))
    kind = str(rng.choice(["normal", "ties", "peaked", "zeros", "spread", "huge"]))
    noise = float(rng.choice([0.0, 0.01, 1.0, 10.0]))
    say(f"sweep l1 seed={seed}: T={T} V={V} {dtype} values={kind} noise={noise}")
    a = _values(rng, kind, (T, V), dtype=dtype)
    b = (a + rng.standard_normal((T, V)) * noise).astype(np.float32)
    b[0] = a[0]  # one identical row: exactly 0
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
    assert float(got["l1"][0]) == 0.0


@pytest.mark.parametrize("seed", range(24))
def test_sweep_support_logits(vsa, seed):
    rng = np.random.default_rng(9000 + seed)
    T = int(rng.integers(1, 40))
    V = int(rng.choice([1, 5, 300, 20000]))
    W = int(rng.choice([1, 3, 16, 64]))
    dtype = str(rng.choice(["bf16", "f32"]))
    kind = str(rng.choice(KINDS))
    say(f"sweep support seed={seed}: T={T} V={V} width={W} {dtype} values={kind}")
    x = _values(rng, kind, (T, V), dtype=dtype)
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x)
        lg = bf16_tensor(bits)
        x64 = oracle.logits_from_logits(bits, "bf16")
    else:
        lg = to_dev(x)
        x64 = x.astype(np.float64)
    ids = np.full((T, W), -1, np.int64)
    y = rng.integers(0, V, T).astype(np.int64)
    for t in range(T):
        w = int(rng.integers(0, min(W, V) + 1))
        row = rng.choice(V, w, replace=False)
        ids[t, rng.choice(W, w, replace=False)] = row
        if w and rng.random() < 0.7:
            y[t] = row[int(rng.integers(0, w))]
        if w >= 2 and rng.random() < 0.1:  # a repeated id: BAD_INPUT
            ids[t, np.nonzero(ids[t] >= 0)[0][1]] = row[0]
    tau = rng.uniform(0.3, 2.0, T).astype(np.float32)
    fb = (rng.random(T) < 0.5).astype(np.uint8)
    got = vsa.score_support_ids(to_dev(y), to_dev(ids), logits=lg, temperature=to_dev(tau), fallback=to_dev(fb))
    ref = oracle.score_support(lambda t, cols: x64[t, cols], V, ids, tau, y, fb)
    _cmp_support(got, ref)
