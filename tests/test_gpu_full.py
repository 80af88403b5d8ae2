"""GPU parity: full-vocabulary scoring (logits input and fused LM head) vs the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_common import assert_close, bf16_tensor, dev, oracle_by_rows, say, to_dev, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsa():
    import logprob_entropy_sampling_amd as m
    m.lib()
    return m


def _cmp_full(got, ref, rows=None):
    st = got["status"].cpu().numpy()
    if rows is not None:
        st = st[rows]
    assert np.array_equal(st, ref["status"]), "status mismatch"
    for k in ("lse", "logprob", "entropy"):
        assert_close(k, got[k].cpu().numpy(), ref[k], rows=rows)


def test_logits_bf16_full_vocab_workload_all_rows(vsa):
    say("logits_full: the full workload T=512 V=151936 bf16, per-row tau, every row vs the oracle")
    c = workload(2)
    lg = bf16_tensor(c["logits"])
    tau = to_dev(c["temperature"])
    got = vsa.score_full(to_dev(c["targets"]), logits=lg, temperature=tau)
    again = vsa.score_full(to_dev(c["targets"]), logits=lg, temperature=tau)
    assert all(torch.equal(got[k], again[k]) for k in ("lse", "logprob", "entropy", "status"))
    ref = oracle_by_rows(lambda r: oracle.score_full(oracle.logits_from_logits(c["logits"], "bf16", rows=r),
                                                     c["temperature"][r], c["targets"][r]), c["T"])
    _cmp_full(got, ref)


@pytest.mark.parametrize("ld_pad", [0, 3, 5])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_logits_ragged_and_strided(vsa, dtype, ld_pad):
    say(f"logits ragged: dtype={dtype} ld_pad={ld_pad} T=37 V=20001")
    rng = np.random.default_rng(100)
    T, V = 37, 20001
    x = (rng.standard_normal((T, V + ld_pad)) * 3).astype(np.float32)
    tau = rng.uniform(0.5, 1.5, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x)
        full = bf16_tensor(bits)
        x64 = oracle.logits_from_logits(bits, "bf16")[:, :V]
    else:
        full = to_dev(x)
        x64 = oracle.logits_from_logits(x, "f32")[:, :V]
    lg = full[:, :V]
    got = vsa.score_full(to_dev(y), logits=lg, temperature=to_dev(tau))
    _cmp_full(got, oracle.score_full(x64, tau, y))


@pytest.mark.parametrize("V", [4096 * 8 - 1, 4096 * 8, 4096 * 8 + 5, 512 * 8 * 9 + 3, 512 * 8 * 15 + 7, 512 * 8 * 16,
                               512 * 8 * 17 + 1])
def test_logits_load_ring_lengths(vsa, V):
    # bf16 rows whose threads hold fewer than 8 vectors, exactly 8, between 9
    # and 15, 16, and 17 or more (the load ring's plain, drain-only, drain and
    # tail, one-pass and steady paths), each with a ragged scalar tail
    say(f"logits load ring: T=6 V={V} bf16, NaN and -inf rows")
    rng = np.random.default_rng(V)
    T = 6
    x = (rng.standard_normal((T, V)) * 2).astype(np.float32)
    x[1, V - 1] = 30.0  # the row's mass on its last (tail) logit
    x[2, :] = -np.inf
    x[2, V // 3] = 0.5
    x[3, V - 2] = np.nan
    tau = rng.uniform(0.5, 1.5, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    y[1] = V - 1
    bits = workloads.to_bf16_bits(x)
    got = vsa.score_full(to_dev(y), logits=bf16_tensor(bits), temperature=to_dev(tau))
    _cmp_full(got, oracle.score_full(oracle.logits_from_logits(bits, "bf16"), tau, y))


def test_vocab_chunk_and_determinism(vsa):
    # vocab_chunk groups the fused sweep's 256-wide tile partials before the
    # groups are merged: every grouping gives the same values up to rounding,
    # and each one is bitwise reproducible
    T, H, V = 96, 256, 40000
    say(f"fused vocab_chunk 1 / 256 / 512 / 8192 / 65536 / V + bitwise run-to-run equality, T={T} H={H} V={V}")
    rng = np.random.default_rng(77)
    hb = workloads.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * 0.15).astype(np.float32))
    tau = rng.uniform(0.5, 1.5, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    hid, w, yd, td = bf16_tensor(hb), bf16_tensor(wb), to_dev(y), to_dev(tau)
    ref = oracle.score_full(oracle.logits_from_hidden(hb, "bf16", wb), tau, y)
    outs = {}
    for chunk in (1, 256, 512, 8192, 65536, V):
        outs[chunk] = vsa.score_full(yd, hidden=hid, weight=w, temperature=td, vocab_chunk=chunk)
        _cmp_full(outs[chunk], ref)
        again = vsa.score_full(yd, hidden=hid, weight=w, temperature=td, vocab_chunk=chunk)
        for k in ("lse", "logprob", "entropy"):
            assert torch.equal(again[k], outs[chunk][k]), (chunk, k)
    # the chunk rounds down to whole tiles: 1 and 256 are the same grouping
    assert all(torch.equal(outs[1][k], outs[256][k]) for k in ("lse", "logprob", "entropy"))
    # a logits source ignores vocab_chunk (one workgroup folds the whole row)
    c = workloads.make(2, T=8)
    lg = bf16_tensor(c["logits"])
    a = vsa.score_full(to_dev(c["targets"]), logits=lg, temperature=to_dev(c["temperature"]), vocab_chunk=1)
    b = vsa.score_full(to_dev(c["targets"]), logits=lg, temperature=to_dev(c["temperature"]), vocab_chunk=151936)
    assert all(torch.equal(a[k], b[k]) for k in ("lse", "logprob", "entropy"))


def test_edge_rows(vsa):
    say("edge rows: uniform, -inf, NaN, +inf, all -inf, bad tau, bad targets, T=1")
    V = 9000
    rows = []
    x = np.zeros((11, V), np.float32)
    x[1] = np.linspace(-3, 3, V)
    x[1, ::7] = -np.inf
    x[2] = 1.0
    x[2, 5] = np.nan
    x[3, 17] = np.inf
    x[4] = -np.inf
    x[5] = np.linspace(-2, 2, V)
    x[6] = np.linspace(-2, 2, V)
    x[7] = np.linspace(-2, 2, V)
    x[8] = np.linspace(-2, 2, V)
    x[9] = 0.5
    x[10] = -np.inf
    x[10, 4100] = np.nan  # a NaN that is the only non -inf value a thread sees
    tau = np.array([1, 1, 1, 1, 1, 0, np.nan, 1, 1, 0.25, 1], np.float32)
    y = np.array([3, 7, 0, 0, 0, 0, 0, -1, V, 8999, 0], np.int64)
    bits = workloads.to_bf16_bits(x)
    got = vsa.score_full(to_dev(y), logits=bf16_tensor(bits), temperature=to_dev(tau))
    ref = oracle.score_full(oracle.logits_from_logits(bits, "bf16"), tau, y)
    assert list(ref["status"]) == [0, 0, 4, 4, 4, 4, 4, 4, 4, 0, 4]
    _cmp_full(got, ref)
    assert abs(float(got["entropy"][0]) - math.log(V)) < 2e-3 + 1e-3 * math.log(V)
    one = vsa.score_full(to_dev(y[:1]), logits=bf16_tensor(bits[:1]), temperature=1.0)
    _cmp_full(one, oracle.score_full(oracle.logits_from_logits(bits[:1], "bf16"), 1.0, y[:1]))


def test_fused_tiny_workload(vsa):
    say("fused: tiny workload T=64 H=256 V=4096 fp32 hidden")
    c = workloads.make(1)
    got = vsa.score_full(to_dev(c["targets"]), hidden=to_dev(c["hidden"]), weight=bf16_tensor(c["weight"]))
    x = oracle.logits_from_hidden(c["hidden"], "f32", c["weight"])
    _cmp_full(got, oracle.score_full(x, c["temperature"], c["targets"]))


@pytest.mark.parametrize("T,H,V", [(300, 200, 5003), (257, 64, 256), (1, 8, 1), (513, 1024, 30000),
                                   (2333, 160, 9000), (700, 96, 2100)])
def test_fused_ragged(vsa, T, H, V):
    say(f"fused ragged: T={T} H={H} V={V} bf16 hidden, per-row tau")
    rng = np.random.default_rng(T + H + V)
    hb = workloads.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * 0.1).astype(np.float32))
    tau = rng.uniform(0.5, 1.5, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    got = vsa.score_full(to_dev(y), hidden=bf16_tensor(hb), weight=bf16_tensor(wb), temperature=to_dev(tau),
                         vocab_chunk=512)
    x = oracle.logits_from_hidden(hb, "bf16", wb)
    _cmp_full(got, oracle.score_full(x, tau, y))


def test_fused_many_tiles_ragged(vsa):
    # more tiles than CUs at an even stage count (H = 128, 64-wide stages), so
    # CUs run several tiles back to back; the last vocabulary and token tiles
    # are ragged (136 and 184 rows)
    T, H, V = 3000, 128, 5000
    say(f"fused, many tiles: T={T} H={H} V={V}, ragged last tiles")
    rng = np.random.default_rng(31)
    hb = workloads.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * 0.2).astype(np.float32))
    tau = rng.uniform(0.5, 1.5, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    y[:4] = [0, V - 1, 4863, 4864]  # ids in the first, the ragged last and its neighbouring tile
    got = vsa.score_full(to_dev(y), hidden=bf16_tensor(hb), weight=bf16_tensor(wb), temperature=to_dev(tau))
    x = oracle.logits_from_hidden(hb, "bf16", wb)
    _cmp_full(got, oracle.score_full(x, tau, y))
    again = vsa.score_full(to_dev(y), hidden=bf16_tensor(hb), weight=bf16_tensor(wb), temperature=to_dev(tau))
    assert all(torch.equal(got[k], again[k]) for k in ("lse", "logprob", "entropy"))


def test_fused_strided_weight(vsa):
    say("fused: padded leading dims (ld_hidden=136, ld_weight=264)")
    rng = np.random.default_rng(5)
    T, H, V = 130, 128, 3000
    hb = workloads.to_bf16_bits(rng.standard_normal((T, 136)).astype(np.float32))
    wb = workloads.to_bf16_bits((rng.standard_normal((V, 264)) * 0.1).astype(np.float32))
    y = rng.integers(0, V, T).astype(np.int64)
    got = vsa.score_full(to_dev(y), hidden=bf16_tensor(hb)[:, :H], weight=bf16_tensor(wb)[:, :H])
    x = oracle.logits_from_hidden(hb[:, :H], "bf16", wb[:, :H])
    _cmp_full(got, oracle.score_full(x, 1.0, y))


def test_fused_full_size_rows_in_every_tile(vsa):
    say("fused: full LM-head workload T=4096 H=4096 V=151936; 256 rows (16 in each token tile) vs the oracle")
    c = workload(4)
    hid = bf16_tensor(c["hidden"])
    w = bf16_tensor(c["weight"])
    y = to_dev(c["targets"])
    got = vsa.score_full(y, hidden=hid, weight=w, vocab_chunk=8192)
    again = vsa.score_full(y, hidden=hid, weight=w, vocab_chunk=8192)
    for k in ("lse", "logprob", "entropy"):
        assert torch.equal(got[k], again[k]), k
    st = got["status"].cpu().numpy()
    ent = got["entropy"].cpu().numpy()
    lp = got["logprob"].cpu().numpy()
    assert (st == 0).all()
    assert np.isfinite(ent).all() and (ent >= 0).all() and (ent <= math.log(151936) + 1e-3).all()
    assert (lp <= 1e-6).all()
    # 16 rows of each 256-row token tile, first and last row of every tile included;
    # every row's 594 vocabulary tiles (the last one ragged) are in its sums
    rows = (np.arange(16)[:, None] * 256 + np.arange(0, 256, 17)[None, :]).ravel()
    x = oracle.logits_from_hidden(c["hidden"], "bf16", c["weight"], rows=rows)
    ref = oracle.score_full(x, 1.0, c["targets"][rows])
    _cmp_full(got, ref, rows=rows)
    # another vocab_chunk groups the same tile partials differently: same values up to rounding
    for chunk in (256, 65536, 151936):
        other = vsa.score_full(y, hidden=hid, weight=w, vocab_chunk=chunk)
        _cmp_full(other, ref, rows=rows)


def test_fused_agrees_with_logits_input_path(vsa):
    # the fused sweep against the logits-input kernel fed the oracle's
    # projection rounded to fp32: both match the oracle, and each other
    # up to the fp32 roundings of the projection
    say("fused vs logits-input path on the same projection: T=300 H=512 V=30001, per-row tau")
    rng = np.random.default_rng(123)
    T, H, V = 300, 512, 30001
    hb = workloads.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * 0.1).astype(np.float32))
    tau = rng.uniform(0.6, 1.2, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    x = oracle.logits_from_hidden(hb, "bf16", wb)
    fused = vsa.score_full(to_dev(y), hidden=bf16_tensor(hb), weight=bf16_tensor(wb), temperature=to_dev(tau))
    direct = vsa.score_full(to_dev(y), logits=to_dev(x.astype(np.float32)), temperature=to_dev(tau))
    ref = oracle.score_full(x, tau, y)
    _cmp_full(fused, ref)
    _cmp_full(direct, ref)
    for k in ("lse", "logprob", "entropy"):
        d = float((fused[k] - direct[k]).abs().max())
        assert d <= 1e-4 * (1.0 + float(direct[k].abs().max())), (k, d)


def test_fp32_range_of_the_tempered_logits(vsa):
    # The kernels work in fp32 base-2 units u = x * log2(e) / tau.  A row whose
    # largest logit has |x| * log2(e) / tau beyond the fp32 range is
    # BAD_INPUT (documented limit); below it, huge logits score like any
    # others, and a logit that falls below -FLT_MAX in those units has
    # probability 0 (its true weight underflows anyway).
    say("fp32 range: rows at 3e38 with tau 0.5 / 1 / 2, all at -3e38, one id at -3e38")
    V = 5000
    rng = np.random.default_rng(21)
    x = rng.standard_normal((6, V)).astype(np.float32)
    x[0, [10, 20]] = 3.0e38   # tau 0.5: u overflows -> BAD
    x[1, [10, 20]] = 3.0e38   # tau 1: 4.3e38 overflows -> BAD
    x[2, [10, 20]] = 3.0e38   # tau 2: 2.2e38 fits: two tied maxima
    x[3, :] = -3.0e38         # tau 0.5: every u is -inf -> BAD
    x[4, 30] = -3.0e38        # tau 0.5: that id has probability 0
    x[5, 40] = 1.0e38         # tau 1: one maximum far above the rest
    tau = np.array([0.5, 1.0, 2.0, 0.5, 0.5, 1.0], np.float32)
    y = np.array([10, 10, 20, 0, 30, 40], np.int64)
    bits = workloads.to_bf16_bits(x)
    got = vsa.score_full(to_dev(y), logits=bf16_tensor(bits), temperature=to_dev(tau))
    st = got["status"].cpu().numpy()
    assert list(st) == [4, 4, 0, 4, 0, 0], st
    ok = np.array([2, 4, 5])
    ref = oracle.score_full(oracle.logits_from_logits(bits[ok], "bf16"), tau[ok], y[ok])
    with np.errstate(over="ignore"):  # fp32 outputs: the oracle's values rounded to fp32
        for k in ("lse", "logprob", "entropy"):
            assert_close(k, got[k].cpu().numpy()[ok], ref[k].astype(np.float32).astype(np.float64))
    assert abs(float(got["entropy"][2]) - math.log(2)) < 1e-6 and abs(float(got["logprob"][2]) + math.log(2)) < 1e-6
    assert float(got["logprob"][4]) == -math.inf and float(got["logprob"][5]) == 0.0
