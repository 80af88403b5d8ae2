"""GPU parity: the transform program (and its seeded draw) on a hidden/weight source vs the fp64 oracle.

The logits the program ranks are the projection rounded to bf16 (xorl issue
#71, "Proposed direction" item 3; the oracle's ``bf16_logits_from_hidden``).
The device rounds its fp32 MFMA sums; on inputs whose every partial sum is
exact in fp32 (hidden = k/4 and W = j/128 with |k|, |j| <= 16: products are
multiples of 2^-9 of magnitude <= 1/2, so H <= 65536 terms fit 24 bits) the
two roundings see the same number, and the comparison is the one of the
logits source: bit-exact descriptors and ids away from the 1e-6 band,
scores within the float tolerance.  On Gaussian inputs the fp32 sums round
differently from the exact ones in about one logit in a thousand (by one
bf16 unit), so there the test only bounds how often a row's support differs."""

import numpy as np
import pytest
import torch

import oracle
from oracle import sampling
import workloads
from tests.gpu_common import bf16_tensor, oracle_by_rows, say, to_dev, workload
from tests.test_gpu_transforms import _compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsa():
    import logprob_entropy_sampling_amd as m
    m.lib()
    return m


def _grid(rng, shape, unit):
    k = np.clip(np.rint(rng.standard_normal(shape) * 4.0), -16, 16).astype(np.float32)
    return workloads.to_bf16_bits(k * np.float32(unit))


def _params(rng, T, V):
    k = rng.choice([0, 1, 20, 50, V // 3, V], T).astype(np.int32)
    p = rng.choice([1.0, 0.95, 0.8, 0.3], T).astype(np.float32)
    mp = rng.choice([0.0, 0.0, 0.05, 0.5], T).astype(np.float32)
    tau = rng.choice([0.7, 1.0, 1.3], T).astype(np.float32)
    return k, p, mp, tau


def _hidden_arg(h_bits, dtype):
    """The device hidden state: the bf16 bits, or the same values as fp32 (exact)."""
    if dtype == "bf16":
        return bf16_tensor(h_bits)
    return to_dev(workloads.bf16_bits_to_f32(h_bits).copy())


def _score(vsa, hid, w, k, p, mp, tau, y, cap):
    return vsa.score_transforms(to_dev(np.asarray(y, np.int64)), None, to_dev(k), to_dev(p), to_dev(mp), hidden=hid,
                                weight=w, temperature=to_dev(tau), cap=cap)


@pytest.mark.parametrize("T,H,V,hdt", [
    (300, 256, 5003, "bf16"),      # one block, register-resident transforms rows, 64-wide K stages
    (2125, 64, 3001, "bf16"),      # two blocks: 2048 rows and a ragged 77
    (77, 96, 700, "f32"),          # H = 96: the 32-wide pipelined sweep; an fp32 hidden state
    (130, 40, 2000, "bf16"),       # H = 40: the register-staged sweep
    (96, 512, 151936, "bf16"),     # the full vocabulary: the count and finish kernels
])
def test_grid_inputs_match_the_oracle(vsa, T, H, V, hdt):
    say(f"transforms on hidden x W: T={T} H={H} V={V} hidden {hdt}, exact-sum grid inputs, cap 64")
    rng = np.random.default_rng(T * 7 + H + V)
    hb, wb = _grid(rng, (T, H), 0.25), _grid(rng, (V, H), 1.0 / 128)
    k, p, mp, tau = _params(rng, T, V)
    xb = oracle.bf16_logits_from_hidden(hb, "bf16", wb)
    x64 = oracle.widen_bf16(xb)
    y = np.argmax(x64, axis=1)
    y[::5] = rng.integers(0, V, y[::5].size)  # some targets outside the support
    hid, w = _hidden_arg(hb, hdt), bf16_tensor(wb)
    got = _score(vsa, hid, w, k, p, mp, tau, y, 64)
    ref = oracle.score_transforms(x64, tau, k, p, mp, y, cap=64)
    _compare(got, ref, 64, f"hidden T={T} V={V}", x64, tau, y)
    # the same bf16 logits as a logits source give the same outputs, bit for bit
    direct = vsa.score_transforms(to_dev(np.asarray(y, np.int64)), bf16_tensor(xb), to_dev(k), to_dev(p), to_dev(mp),
                                  temperature=to_dev(tau), cap=64)
    for name in got:
        if got[name] is not None:
            assert torch.equal(got[name], direct[name]) or (
                got[name].is_floating_point() and torch.equal(torch.nan_to_num(got[name], 7.0),
                                                              torch.nan_to_num(direct[name], 7.0))), name


def test_sampler_over_two_blocks(vsa):
    say("sample on hidden x W: T=2125 (blocks of 2048 and 77), H=128, V=3001, grid inputs: draws vs the oracle")
    rng = np.random.default_rng(5)
    T, H, V = 2125, 128, 3001
    hb, wb = _grid(rng, (T, H), 0.25), _grid(rng, (V, H), 1.0 / 128)
    k, p, mp, tau = _params(rng, T, V)
    x64 = oracle.widen_bf16(oracle.bf16_logits_from_hidden(hb, "bf16", wb))
    seed, off = 77, 2 ** 33 + 1
    got = vsa.sample_transforms(None, to_dev(k), to_dev(p), to_dev(mp), hidden=bf16_tensor(hb), weight=bf16_tensor(wb),
                                temperature=to_dev(tau), seed=seed, offset=off)
    ref = sampling.sample_transforms(x64, tau, k, p, mp, seed=seed, offset=off)
    s = got["sampled"].cpu().numpy()
    assert np.array_equal(got["status"].cpu().numpy(), ref["status"])
    diff = np.nonzero(s != ref["sampled"])[0]
    assert all(ref["margin"][i] <= 1e-9 for i in diff), diff[:10]
    assert diff.size <= 3, diff
    say(f"  {T - diff.size} of {T} draws identical (rows past 2048 draw with their batch row index)")


def test_gaussian_inputs_rarely_differ(vsa):
    say("transforms on hidden x W: Gaussian hidden and W (fp32 sums not exact), T=200 H=1024 V=20000")
    rng = np.random.default_rng(11)
    T, H, V = 200, 1024, 20000
    hb = workloads.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) / 32).astype(np.float32))
    k, p, mp, tau = _params(rng, T, V)
    x64 = oracle.widen_bf16(oracle.bf16_logits_from_hidden(hb, "bf16", wb))
    y = np.argmax(x64, axis=1)
    got = _score(vsa, bf16_tensor(hb), bf16_tensor(wb), k, p, mp, tau, y, 64)
    ref = oracle.score_transforms(x64, tau, k, p, mp, y, cap=64)
    g = {n: v.cpu().numpy() for n, v in got.items() if v is not None}
    same = (g["support_len"] == ref["support_len"]) & (g["support_ids"] == ref["support_ids"]).all(1)
    say(f"  {int(same.sum())} of {T} rows with the oracle's support and ids")
    assert same.mean() >= 0.5
    # on those rows the scores differ only through the few logits rounded the other way
    rows = np.nonzero(same)[0]
    assert np.allclose(g["logprob"][rows], ref["logprob"][rows], rtol=0, atol=0.05)
    assert np.allclose(g["entropy"][rows], ref["entropy"][rows], rtol=0, atol=0.05)


def test_full_size_sampled_rows(vsa):
    say("transforms on hidden x W: the workload T=2048 H=4096 V=151936 (grid inputs), 256 rows vs the oracle, "
        "determinism, and the seeded draw")
    c = workload(6)
    T, V = c["T"], c["V"]
    rows = np.unique(np.linspace(0, T - 1, 256).astype(np.int64))
    xb = oracle_by_rows(lambda r: {"x": oracle.bf16_logits_from_hidden(c["hidden"], "bf16", c["weight"], rows=rows[r])},
                        rows.size, block=64)["x"]
    x64 = oracle.widen_bf16(xb)
    y_rows = np.argmax(x64, axis=1)
    y = np.zeros(T, np.int64)
    y[rows] = y_rows
    hid, w = bf16_tensor(c["hidden"]), bf16_tensor(c["weight"])
    args = [c[n] for n in ("top_k", "top_p", "min_p", "temperature")]
    got = _score(vsa, hid, w, *args, y, 64)
    again = _score(vsa, hid, w, *args, y, 64)
    for n in got:
        if got[n] is not None:
            assert torch.equal(torch.nan_to_num(got[n], 7.0) if got[n].is_floating_point() else got[n],
                               torch.nan_to_num(again[n], 7.0) if again[n].is_floating_point() else again[n]), n
    sub = {n: (v[torch.from_numpy(rows).to(v.device)] if v is not None else None) for n, v in got.items()}
    ref = oracle.score_transforms(x64, args[3][rows], args[0][rows], args[1][rows], args[2][rows], y_rows, cap=64)
    _compare(sub, ref, 64, "hidden workload rows", x64, args[3][rows], y_rows)
    seed = 20260101
    smp = vsa.sample_transforms(None, *(to_dev(a) for a in args[:3]), hidden=hid, weight=w,
                                temperature=to_dev(args[3]), seed=seed)
    sref = sampling.sample_transforms(x64, args[3][rows], args[0][rows], args[1][rows], args[2][rows], seed=seed,
                                      rows=rows)
    s = smp["sampled"].cpu().numpy()[rows]
    diff = np.nonzero(s != sref["sampled"])[0]
    assert all(sref["margin"][i] <= 1e-9 for i in diff), diff[:10]
    say(f"  draws: {rows.size - diff.size} of {rows.size} identical")
