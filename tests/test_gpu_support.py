"""GPU parity: recorded-support scoring (logits gather and selected projections) vs the fp64 oracle."""

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


def _cmp(got, ref, rows=None):
    st = got["status"].cpu().numpy()
    if rows is not None:
        st = st[rows]
    assert np.array_equal(st, ref["status"]), f"status mismatch at {np.nonzero(st != ref['status'])[0][:10]}"
    assert_close("logprob", got["logprob"].cpu().numpy(), ref["logprob"], rows=rows)
    assert_close("entropy", got["entropy"].cpu().numpy(), ref["entropy"], rows=rows)


def test_tiny_workload_fused_with_fallback(vsa):
    say("support: tiny workload, selected projections, width 8, synthetic-EOS fallback")
    c = workloads.make(1)
    x = oracle.logits_from_hidden(c["hidden"], "f32", c["weight"])
    got = vsa.score_support_ids(to_dev(c["targets"]), to_dev(c["support_ids"]), hidden=to_dev(c["hidden"]),
                                weight=bf16_tensor(c["weight"]), fallback=to_dev(c["fallback"]))
    ref = oracle.score_support(lambda t, cols: x[t, cols], c["V"], c["support_ids"], 1.0, c["targets"],
                               c["fallback"])
    assert (ref["status"] & oracle.ST_FULL_VOCAB_FALLBACK).any() and (ref["status"] & 2).any()
    _cmp(got, ref)
    # singleton rows: exactly zero logprob and entropy
    widths = (c["support_ids"] >= 0).sum(1)
    single = np.nonzero((widths == 1) & (ref["status"] == 0))[0]
    assert single.size
    assert (got["logprob"].cpu().numpy()[single] == 0.0).all()
    assert (got["entropy"].cpu().numpy()[single] == 0.0).all()
    # without the fallback flag, empty rows score 0 / 0
    got2 = vsa.score_support_ids(to_dev(c["targets"]), to_dev(c["support_ids"]), hidden=to_dev(c["hidden"]),
                                 weight=bf16_tensor(c["weight"]))
    ref2 = oracle.score_support(lambda t, cols: x[t, cols], c["V"], c["support_ids"], 1.0, c["targets"])
    _cmp(got2, ref2)


@pytest.mark.parametrize("H", [96, 160, 224])
def test_fused_fallback_rows_gathered_sweep(vsa, H):
    say(f"support: fused source, H={H} (K not a multiple of 128), a third of the rows empty -> full-vocab fallback")
    rng = np.random.default_rng(H)
    T, V, W = 600, 3000, 8
    hb = workloads.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * 0.2).astype(np.float32))
    ids = np.argsort(rng.random((T, V)), axis=1)[:, :W].astype(np.int64)  # distinct ids per row
    ids[rng.random((T, W)) < 0.3] = -1
    empty = rng.random(T) < 0.33
    ids[empty] = -1
    y = rng.integers(0, V, T).astype(np.int64)
    fb = empty.astype(np.uint8)
    got = vsa.score_support_ids(to_dev(y), to_dev(ids), hidden=bf16_tensor(hb), weight=bf16_tensor(wb),
                                fallback=to_dev(fb))
    x = oracle.logits_from_hidden(hb, "bf16", wb)
    ref = oracle.score_support(lambda t, cols: x[t, cols], V, ids, 1.0, y, fb)
    assert ((ref["status"] & oracle.ST_FULL_VOCAB_FALLBACK) != 0).sum() == empty.sum()
    _cmp(got, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_logits_gather_matches_oracle(vsa, dtype):
    say(f"support over materialised logits: dtype={dtype}")
    rng = np.random.default_rng(7)
    T, V, W = 200, 5000, 24
    xf = (rng.standard_normal((T, V)) * 2).astype(np.float32)
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(xf)
        lg = bf16_tensor(bits)
        x64 = oracle.logits_from_logits(bits, "bf16")
    else:
        lg = to_dev(xf)
        x64 = xf.astype(np.float64)
    ids = np.full((T, W), -1, np.int64)
    y = np.empty(T, np.int64)
    for t in range(T):
        w = int(rng.integers(0, W + 1))
        row = rng.choice(V, w, replace=False)
        pos = rng.choice(W, w, replace=False)  # padding anywhere
        ids[t, pos] = row
        y[t] = row[0] if (w and t % 5) else int(rng.integers(0, V))
    tau = rng.uniform(0.5, 1.5, T).astype(np.float32)
    fb = (rng.random(T) < 0.5).astype(np.uint8)
    got = vsa.score_support_ids(to_dev(y), to_dev(ids), logits=lg, temperature=to_dev(tau), fallback=to_dev(fb))
    ref = oracle.score_support(lambda t, cols: x64[t, cols], V, ids, tau, y, fb)
    _cmp(got, ref)


def test_bad_rows_and_singletons(vsa):
    say("support: duplicates, id >= V, bad target, bad tau, NaN/-inf support logits, singletons")
    V = 100
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((8, V))).astype(np.float32)
    x[5, 3] = np.nan
    x[6, 4] = -np.inf
    x[7, [1, 2]] = -np.inf
    ids = np.array([[1, 1, -1], [1, 100, -1], [4, 5, 6], [9, -1, -1], [-1, 7, -1], [3, 8, -1], [4, 9, -1],
                    [1, 2, -1]], np.int64)
    y = np.array([1, 1, 200, 9, 7, 8, 4, 1], np.int64)
    tau = np.array([1, 1, 1, 1, 0.0, 1, 1, 1], np.float32)
    bits = workloads.to_bf16_bits(x)
    got = vsa.score_support_ids(to_dev(y), to_dev(ids), logits=bf16_tensor(bits), temperature=to_dev(tau))
    x64 = oracle.logits_from_logits(bits, "bf16")
    ref = oracle.score_support(lambda t, cols: x64[t, cols], V, ids, tau, y)
    assert list(ref["status"]) == [4, 4, 4, 0, 4, 4, 0, 4]
    _cmp(got, ref)
    assert float(got["logprob"][3]) == 0.0 and float(got["entropy"][3]) == 0.0
    assert float(got["logprob"][6]) == -np.inf


def test_full_support_equals_full_vocabulary(vsa):
    say("support: every id in the support == full-vocabulary scores")
    rng = np.random.default_rng(11)
    T, V = 6, 1000
    bits = workloads.to_bf16_bits((rng.standard_normal((T, V)) * 2).astype(np.float32))
    ids = np.stack([rng.permutation(V) for _ in range(T)]).astype(np.int64)
    y = rng.integers(0, V, T).astype(np.int64)
    s = vsa.score_support_ids(to_dev(y), to_dev(ids), logits=bf16_tensor(bits))
    f = vsa.score_full(to_dev(y), logits=bf16_tensor(bits))
    assert_close("logprob", s["logprob"].cpu().numpy(), f["logprob"].cpu().numpy().astype(np.float64))
    assert_close("entropy", s["entropy"].cpu().numpy(), f["entropy"].cpu().numpy().astype(np.float64))


def test_replay_workload_reduced(vsa):
    say("support replay recipe at T=256 (H=7168, V=129280, width 64)")
    c = workloads.make(3, T=256)
    got = vsa.score_support_ids(to_dev(c["targets"]), to_dev(c["support_ids"]), hidden=bf16_tensor(c["hidden"]),
                                weight=bf16_tensor(c["weight"]))
    ids = c["support_ids"]

    def fn(t, cols):
        return oracle.logits_from_hidden(c["hidden"], "bf16", c["weight"], rows=[t], cols=cols)[0]
    ref = oracle.score_support(fn, c["V"], ids, 1.0, c["targets"])
    _cmp(got, ref)


def test_permuted_ids_and_moved_padding(vsa):
    # the support is a set: permuting a row's ids or moving its padding changes
    # only the order of the fold's fp32 sums
    say("support: ids permuted and padding moved to the front, fused and logits sources")
    c = workloads.make(3, T=96, V=20000, H=512)
    rng = np.random.default_rng(21)
    ids = c["support_ids"]
    moved = np.full_like(ids, -1)
    for t in range(ids.shape[0]):
        sup = rng.permutation(ids[t][ids[t] >= 0])
        moved[t, ids.shape[1] - sup.size:] = sup
    hid, w, y = bf16_tensor(c["hidden"]), bf16_tensor(c["weight"]), to_dev(c["targets"])
    x = oracle.logits_from_hidden(c["hidden"], "bf16", c["weight"])
    lg = to_dev(x.astype(np.float32))
    for src in (dict(hidden=hid, weight=w), dict(logits=lg)):
        a = vsa.score_support_ids(y, to_dev(ids), **src)
        b = vsa.score_support_ids(y, to_dev(moved), **src)
        assert torch.equal(a["status"], b["status"])
        for k in ("logprob", "entropy"):
            d = (a[k] - b[k]).abs().nan_to_num(0.0)
            assert float(d.max()) <= 1e-5 * (1.0 + float(a[k].abs().nan_to_num(0.0).max())), k
    ref = oracle.score_support(lambda t, cols: x[t, np.asarray(cols)], c["V"], moved, 1.0, c["targets"])
    _cmp(b, ref)


def test_replay_workload_full_size_all_rows(vsa):
    say("support replay full size T=2048 H=7168 V=129280 width 64: every row vs the oracle; determinism")
    c = workload(3)
    T = c["T"]
    hid, w = bf16_tensor(c["hidden"]), bf16_tensor(c["weight"])
    y, ids = to_dev(c["targets"]), to_dev(c["support_ids"])
    got = vsa.score_support_ids(y, ids, hidden=hid, weight=w)
    again = vsa.score_support_ids(y, ids, hidden=hid, weight=w)
    assert torch.equal(got["logprob"], again["logprob"]) and torch.equal(got["entropy"], again["entropy"])
    widths = (c["support_ids"] >= 0).sum(1)
    st = got["status"].cpu().numpy()
    assert np.array_equal(st, np.where(widths == 0, 1, 0).astype(np.uint8))

    def ref_rows(rows):
        def fn(t, cols):
            return oracle.logits_from_hidden(c["hidden"], "bf16", c["weight"], rows=[rows[t]], cols=cols)[0]
        return oracle.score_support(fn, c["V"], c["support_ids"][rows], 1.0, c["targets"][rows])
    _cmp(got, oracle_by_rows(ref_rows, T))
    single = np.nonzero(widths == 1)[0]
    assert single.size and (got["logprob"].cpu().numpy()[single] == 0).all()
    assert (got["entropy"].cpu().numpy()[single] == 0).all()


def test_fused_max_width_duplicates_far_apart(vsa):
    # the widest support (1024 ids, sized LDS arrays at their largest) on the
    # fused source: distinct ids with padding anywhere, a repeated id far
    # from its first use (BAD_INPUT), an id >= V, an empty row
    T, H, V, W = 12, 256, 4000, 1024
    say(f"support: fused source, width {W} (maximum), duplicates far apart, id >= V, empty row")
    rng = np.random.default_rng(41)
    hb = workloads.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * 0.1).astype(np.float32))
    ids = np.full((T, W), -1, np.int64)
    y = np.empty(T, np.int64)
    for t in range(T):
        w = int(rng.integers(W // 2, W + 1))
        row = rng.choice(V, w, replace=False)
        ids[t, rng.choice(W, w, replace=False)] = row
        y[t] = row[int(rng.integers(0, w))]
    used = np.nonzero(ids[2] >= 0)[0]
    ids[2, used[-1]] = ids[2, used[0]]  # a repeat, hundreds of positions after the first use
    ids[4, 1000] = V  # out of range
    ids[7] = -1  # empty
    tau = rng.uniform(0.5, 1.5, T).astype(np.float32)
    got = vsa.score_support_ids(to_dev(y), to_dev(ids), hidden=bf16_tensor(hb), weight=bf16_tensor(wb),
                                temperature=to_dev(tau))
    x = oracle.logits_from_hidden(hb, "bf16", wb)
    ref = oracle.score_support(lambda t, cols: x[t, cols], V, ids, tau, y)
    st = ref["status"]
    assert st[2] == oracle.ST_BAD_INPUT and st[4] == oracle.ST_BAD_INPUT, st
    _cmp(got, ref)
