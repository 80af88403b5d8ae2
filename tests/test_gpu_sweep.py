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


# ---- the entry points added with the backward, the loss, the draw and the hidden/weight transforms ----

@pytest.mark.parametrize("seed", range(12))
def test_sweep_backward(vsa, seed):
    from tests.test_gpu_backward import REL, _close, term_sizes
    rng = np.random.default_rng(10000 + seed)
    T = int(rng.integers(1, 260))
    H = int(rng.choice([8, 40, 64, 96, 128, 192, 264]))
    V = int(rng.choice([1, 7, 300, 5000, 20001]))
    chunk = int(rng.choice([1, 256, 1000, 100000]))
    hdt = str(rng.choice(["bf16", "f32"]))
    terms = str(rng.choice(["both", "logprob", "entropy"]))
    say(f"sweep backward seed={seed}: T={T} H={H} V={V} chunk={chunk} hidden {hdt} terms={terms}")
    h = rng.standard_normal((T, H)).astype(np.float32)
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * (1.0 / np.sqrt(H))).astype(np.float32))
    tau = rng.uniform(0.5, 1.5, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    a = rng.normal(0, 1, T).astype(np.float32) if terms != "entropy" else None
    b = rng.normal(0, 1, T).astype(np.float32) if terms != "logprob" else None
    if hdt == "bf16":
        hb = workloads.to_bf16_bits(h)
        hid, h_arg = bf16_tensor(hb), hb
    else:
        hid, h_arg = to_dev(h), h
    w = bf16_tensor(wb)
    fw = vsa.score_full(to_dev(y), hidden=hid, weight=w, temperature=to_dev(tau))
    got = vsa.score_full_backward(to_dev(y), fw["lse"], fw["entropy"], hidden=hid, weight=w,
                                  grad_logprob=None if a is None else to_dev(a),
                                  grad_entropy=None if b is None else to_dev(b), temperature=to_dev(tau),
                                  vocab_chunk=chunk)
    ref = oracle.score_full_vjp(h_arg, hdt, wb, tau, y, a, b)
    adx = np.abs(ref["d_logits"])
    h64 = oracle.widen_bf16(oracle.round_f32_to_bf16(h) if hdt == "f32" else h_arg)
    w64 = oracle.widen_bf16(wb)
    M, eps = term_sizes(h64 @ w64.T, tau, y, a, b)
    eM = eps[:, None] * M
    _close("grad_hidden", got["grad_hidden"].cpu().numpy(), ref["d_hidden"],
           REL * (adx @ np.abs(w64)) + eM @ np.abs(w64) + 1e-30)
    _close("grad_weight", got["grad_weight"].cpu().numpy(), ref["d_weight"],
           REL * (adx.T @ np.abs(h64)) + eM.T @ np.abs(h64) + 1e-30)


@pytest.mark.parametrize("seed", range(12))
def test_sweep_support_backward(vsa, seed):
    from tests.test_gpu_support_backward import _check, _magnitudes
    rng = np.random.default_rng(11000 + seed)
    T = int(rng.integers(1, 80))
    H = int(rng.choice([8, 16, 40, 128, 520]))
    V = int(rng.choice([1, 6, 50, 3000]))
    W = int(rng.choice([1, 2, 7, 64, 300]))
    hdt = str(rng.choice(["bf16", "f32"]))
    say(f"sweep support backward seed={seed}: T={T} H={H} V={V} width={W} hidden {hdt}")
    hb = workloads.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * (1.5 / np.sqrt(H))).astype(np.float32))
    ids = np.full((T, W), -1, np.int64)
    y = rng.integers(0, V, T).astype(np.int64)
    for t in range(T):
        w = int(rng.integers(0, min(W, V) + 1))
        row = rng.choice(V, w, replace=False)
        ids[t, rng.choice(W, w, replace=False)] = row
        if w and rng.random() < 0.8:
            y[t] = row[int(rng.integers(0, w))]
        if w >= 2 and rng.random() < 0.1:
            ids[t, np.nonzero(ids[t] >= 0)[0][1]] = row[0]  # a repeated id: no gradient
    tau = rng.uniform(0.4, 2.0, T).astype(np.float32)
    a, b = rng.normal(0, 1, T).astype(np.float32), rng.normal(0, 1, T).astype(np.float32)
    h_arg = hb if hdt == "bf16" else workloads.bf16_bits_to_f32(hb).copy()
    got = vsa.score_support_backward(to_dev(y), to_dev(ids), hidden=bf16_tensor(hb) if hdt == "bf16" else to_dev(h_arg),
                                     weight=bf16_tensor(wb), grad_logprob=to_dev(a), grad_entropy=to_dev(b),
                                     temperature=to_dev(tau))
    ref = oracle.score_support_vjp(h_arg, hdt, wb, ids, tau, y, a, b)
    h64, w64 = oracle.widen_bf16(hb), oracle.widen_bf16(wb)
    M = _magnitudes(h64, w64, ids, tau.astype(np.float64), y, a.astype(np.float64), b.astype(np.float64))
    _check(got, ref, M, h64, w64, ids, f"sweep seed={seed}")


@pytest.mark.parametrize("seed", range(16))
def test_sweep_sample(vsa, seed):
    from oracle import sampling
    rng = np.random.default_rng(12000 + seed)
    T = int(rng.integers(1, 24))
    V = int(rng.choice([1, 3, 64, 1000, 30001, 100003]))
    kind = str(rng.choice(["normal", "ties", "peaked", "neg_inf", "zeros"]))
    say(f"sweep sample seed={seed}: T={T} V={V} values={kind}")
    bits = workloads.to_bf16_bits(_values(rng, kind, (T, V)))
    k = rng.choice([0, 1, 5, 50, V], size=T).astype(np.int32)
    p = np.where(rng.random(T) < 0.5, 1.0, rng.uniform(0.05, 0.99, T)).astype(np.float32)
    mp = np.where(rng.random(T) < 0.5, 0.0, 10.0 ** rng.uniform(-4, -0.1, T)).astype(np.float32)
    tau = rng.uniform(0.2, 2.5, T).astype(np.float32)
    s, off = int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 40))
    got = vsa.sample_transforms(bf16_tensor(bits), to_dev(k), to_dev(p), to_dev(mp), temperature=to_dev(tau), seed=s,
                                offset=off)
    x64 = oracle.logits_from_logits(bits, "bf16")
    ref = sampling.sample_transforms(x64, tau, k, p, mp, seed=s, offset=off)
    assert np.array_equal(got["status"].cpu().numpy(), ref["status"])
    drawn = got["sampled"].cpu().numpy()
    diff = np.nonzero(drawn != ref["sampled"])[0]
    assert all(ref["margin"][i] <= 1e-9 for i in diff), (diff[:5], drawn[diff[:5]], ref["sampled"][diff[:5]])


@pytest.mark.parametrize("seed", range(12))
def test_sweep_l1_loss(vsa, seed):
    import torch
    from tests.test_gpu_l1_loss import _grad_close, sign_flip_bound
    rng = np.random.default_rng(13000 + seed)
    T = int(rng.integers(1, 12))
    V = int(rng.choice([1, 2, 9, 1000, 65537]))
    kind = str(rng.choice(["normal", "ties", "peaked", "zeros"]))
    noise = float(rng.choice([0.0, 0.1, 2.0]))
    gdt = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    wt = str(rng.choice(["none", "mixed"]))
    say(f"sweep l1 loss seed={seed}: T={T} V={V} values={kind} noise={noise} grad {gdt} weights={wt}")
    a = _values(rng, kind, (T, V))
    b = (a + rng.standard_normal((T, V)) * noise).astype(np.float32)
    w = None if wt == "none" else np.where(rng.random(T) < 0.3, 0.0, rng.uniform(0.1, 3.0, T)).astype(np.float32)
    ab, bb = workloads.to_bf16_bits(a), workloads.to_bf16_bits(b)
    a64, b64 = oracle.logits_from_logits(ab, "bf16"), oracle.logits_from_logits(bb, "bf16")
    scale = float(rng.choice([1.0, -0.5, 4.0]))
    got = vsa.l1_loss(bf16_tensor(ab), bf16_tensor(bb), weights=None if w is None else to_dev(w), grad_scale=scale,
                      grad_dtype=gdt)
    ref = oracle.weighted_l1_loss(a64, b64, w, grad_scale=scale)
    assert_close("l1", got["l1"].cpu().numpy(), ref["l1"])
    if np.isfinite(ref["den"]) and ref["den"] > 0:
        assert_close("loss", got["loss"].cpu().numpy(), np.array([ref["num"], ref["den"], ref["loss"]]))
        wv = np.ones(T) if w is None else w.astype(np.float64)
        extra = sign_flip_bound(a64, b64, np.abs(scale * wv / ref["den"]))
        _grad_close("grad", got["grad"].float().cpu().numpy(), ref["grad"], bf16=gdt == torch.bfloat16, extra=extra)


@pytest.mark.parametrize("seed", range(8))
def test_sweep_transforms_hidden(vsa, seed):
    from tests.test_gpu_transforms_hidden import _grid
    rng = np.random.default_rng(14000 + seed)
    T = int(rng.choice([1, 5, 70, 2049]))
    H = int(rng.choice([8, 64, 96, 200]))
    V = int(rng.choice([1, 17, 3000, 90001]))
    if T > 2048:
        V = min(V, 3000)  # two logits blocks; the oracle's sorts stay short
    cap = int(rng.choice([0, 4, 64]))
    say(f"sweep transforms on hidden x W seed={seed}: T={T} H={H} V={V} cap={cap} (exact-sum grid inputs)")
    hb, wb = _grid(rng, (T, H), 0.25), _grid(rng, (V, H), 1.0 / 128)
    k = rng.choice([0, 1, 5, V], size=T).astype(np.int32)
    p = np.where(rng.random(T) < 0.5, 1.0, rng.uniform(0.05, 0.99, T)).astype(np.float32)
    mp = np.where(rng.random(T) < 0.5, 0.0, 10.0 ** rng.uniform(-4, -0.1, T)).astype(np.float32)
    tau = rng.uniform(0.3, 2.0, T).astype(np.float32)
    x64 = oracle.widen_bf16(oracle.bf16_logits_from_hidden(hb, "bf16", wb))
    y = np.argmax(x64, axis=1)
    got = vsa.score_transforms(to_dev(y), None, to_dev(k), to_dev(p), to_dev(mp), hidden=bf16_tensor(hb),
                               weight=bf16_tensor(wb), temperature=to_dev(tau), cap=cap)
    ref = oracle.score_transforms(x64, tau, k, p, mp, y, cap=cap)
    _cmp_transforms(got, ref, cap, f"sweep hidden seed={seed}", x64, tau, y)
