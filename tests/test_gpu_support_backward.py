"""GPU parity: the VJP of recorded-support scoring through the fused projection vs the fp64 oracle.

Tolerance, from the arithmetic: the kernel's dX (fp32) follows from fp32
support logits (dot products of H bf16 pairs), so each dX[t, j] is within a
small relative error of the size of its terms,
  M[t, j] = (|a_t| ([v_j = y_t] + p_j) + |b_t| p_j (|ln p_j| + H_S)) / tau_t;
the products then add fp32 roundings.  Element by element:
  |grad_hidden - ref| <= 1e-3 (M |W_S|)[t, h] + 1e-7
  |grad_weight - ref| <= 1e-3 (sum over pairs of M |bf16(hidden)|)[v, h] + 1e-7
Singleton, empty and bad rows must be exactly zero."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_common import bf16_tensor, say, to_dev, workload

pytestmark = pytest.mark.gpu
REL = 1e-3


@pytest.fixture(scope="module")
def vsa():
    import logprob_entropy_sampling_amd as m
    m.lib()
    return m


def _magnitudes(h64, w64, ids, tau, y, a, b):
    """M[t, j] of the module notes (0 at padding and on rows without gradient)."""
    T, width = ids.shape
    V = w64.shape[0]
    M = np.zeros((T, width))
    for t in range(T):
        pos = np.nonzero(ids[t] >= 0)[0]
        sup = ids[t, pos]
        if sup.size == 0 or (sup >= V).any() or len(np.unique(sup)) != sup.size or not (0 <= y[t] < V):
            continue
        z = (h64[t] @ w64[sup].T) / tau[t]
        lnp = z - (z.max() + np.log(np.sum(np.exp(z - z.max()))))
        p = np.exp(lnp)
        H = -np.sum(p * lnp)
        M[t, pos] = (abs(a[t]) * ((sup == y[t]) + p) + abs(b[t]) * p * (np.abs(lnp) + H)) / tau[t]
    return M


def _check(got, ref, M, h64, w64, ids, label):
    gh = got["grad_hidden"].cpu().numpy().astype(np.float64) if got.get("grad_hidden") is not None else None
    if gh is not None:
        bound = np.zeros_like(gh)
        for t in range(ids.shape[0]):
            pos = np.nonzero(M[t] > 0)[0]
            if pos.size:
                bound[t] = REL * (M[t, pos] @ np.abs(w64[ids[t, pos]]))
        bound += 1e-7
        err = np.abs(gh - ref["d_hidden"])
        say(f"  {label} grad_hidden: max |err| {err.max():.3e}, max err/bound {(err / bound).max():.3f}")
        assert (err <= bound).all(), np.unravel_index(int(np.argmax(err - bound)), err.shape)
    if got.get("grad_weight") is not None:
        gw = got["grad_weight"].cpu().numpy().astype(np.float64)
        V = gw.shape[0]
        bound = np.zeros((V, gw.shape[1]))
        for t in range(ids.shape[0]):
            for j in np.nonzero(M[t] > 0)[0]:
                bound[ids[t, j]] += REL * M[t, j] * np.abs(h64[t])
        bound += 1e-7
        err = np.abs(gw - ref["d_weight"])
        say(f"  {label} grad_weight: max |err| {err.max():.3e}, max err/bound {(err / bound).max():.3f}")
        assert (err <= bound).all(), np.unravel_index(int(np.argmax(err - bound)), err.shape)


def _inputs(rng, T, H, V, width, id_range=None):
    hb = workloads.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * (2.0 / np.sqrt(H))).astype(np.float32))
    r = id_range or V
    ids = np.full((T, width), -1, np.int64)
    y = np.empty(T, np.int64)
    for t in range(T):
        w = int(rng.integers(1, width + 1))
        row = rng.choice(r, w, replace=False)
        pos = np.sort(rng.choice(width, w, replace=False))  # padding anywhere
        ids[t, pos] = row
        y[t] = row[int(rng.integers(0, w))]
    # special rows: a singleton, an empty row, a repeated id, an id >= V, a target outside
    ids[0] = -1
    ids[0, width // 2] = 5
    y[0] = 5
    ids[1] = -1
    if width >= 2:
        ids[2, :2] = [7, 7]
        ids[3, :2] = [V + 4, 1]
        y[4] = int(np.setdiff1d(np.arange(r), ids[4])[0])
    tau = rng.uniform(0.6, 1.5, T).astype(np.float32)
    a = rng.normal(0, 1, T).astype(np.float32)
    b = rng.normal(0, 1, T).astype(np.float32)
    return hb, wb, ids, y, tau, a, b


@pytest.mark.parametrize("T,H,V,width,hdt,id_range", [
    (60, 256, 3000, 16, "bf16", 40),      # ids drawn from 40: every id in many rows (buckets of ~12 pairs)
    (40, 96, 1000, 8, "f32", None),       # an fp32 hidden state (rounded to bf16 first)
    (33, 40, 500, 64, "bf16", 100),       # H = 40
    (20, 1024, 20000, 1024, "bf16", None),  # the maximum width
])
def test_support_backward_matches_oracle(vsa, T, H, V, width, hdt, id_range):
    say(f"support backward: T={T} H={H} V={V} width {width} hidden {hdt}; singleton, empty, repeated, id >= V and "
        "outside-target rows")
    rng = np.random.default_rng(T * 31 + H + width)
    hb, wb, ids, y, tau, a, b = _inputs(rng, T, H, V, width, id_range)
    h_arg = hb if hdt == "bf16" else workloads.bf16_bits_to_f32(hb).copy()
    hid = bf16_tensor(hb) if hdt == "bf16" else to_dev(h_arg)
    w = bf16_tensor(wb)
    args = dict(hidden=hid, weight=w, grad_logprob=to_dev(a), grad_entropy=to_dev(b), temperature=to_dev(tau))
    got = vsa.score_support_backward(to_dev(y), to_dev(ids), **args)
    again = vsa.score_support_backward(to_dev(y), to_dev(ids), **args)
    assert torch.equal(got["grad_hidden"], again["grad_hidden"]) and torch.equal(got["grad_weight"], again["grad_weight"])
    ref = oracle.score_support_vjp(h_arg, hdt, wb, ids, tau, y, a, b)
    h64, w64 = oracle.widen_bf16(hb), oracle.widen_bf16(wb)
    M = _magnitudes(h64, w64, ids, tau.astype(np.float64), y, a.astype(np.float64), b.astype(np.float64))
    _check(got, ref, M, h64, w64, ids, f"T={T} H={H}")
    gh = got["grad_hidden"].cpu().numpy()
    for t in (0, 1, 2, 3):  # singleton, empty, repeated id, id >= V: exactly zero
        assert (gh[t] == 0).all(), t
    # one output at a time gives the same values
    only_h = vsa.score_support_backward(to_dev(y), to_dev(ids), want_weight=False, **args)
    only_w = vsa.score_support_backward(to_dev(y), to_dev(ids), want_hidden=False, **args)
    assert torch.equal(only_h["grad_hidden"], got["grad_hidden"])
    assert torch.equal(only_w["grad_weight"], got["grad_weight"])


def test_one_term_and_empty_width(vsa):
    say("support backward: only the entropy term, only the logprob term, and a width-0 support")
    rng = np.random.default_rng(9)
    T, H, V, width = 30, 64, 400, 12
    hb, wb, ids, y, tau, a, b = _inputs(rng, T, H, V, width, 50)
    h64, w64 = oracle.widen_bf16(hb), oracle.widen_bf16(wb)
    for aa, bb in ((None, b), (a, None)):
        got = vsa.score_support_backward(to_dev(y), to_dev(ids), hidden=bf16_tensor(hb), weight=bf16_tensor(wb),
                                         grad_logprob=None if aa is None else to_dev(aa),
                                         grad_entropy=None if bb is None else to_dev(bb), temperature=to_dev(tau))
        a0 = np.zeros(T, np.float32) if aa is None else aa
        b0 = np.zeros(T, np.float32) if bb is None else bb
        ref = oracle.score_support_vjp(hb, "bf16", wb, ids, tau, y, a0, b0)
        M = _magnitudes(h64, w64, ids, tau.astype(np.float64), y, a0.astype(np.float64), b0.astype(np.float64))
        _check(got, ref, M, h64, w64, ids, "one term")
    empty = torch.empty((T, 0), dtype=torch.int64, device="cuda")
    got = vsa.score_support_backward(to_dev(y), empty, hidden=bf16_tensor(hb), weight=bf16_tensor(wb),
                                     grad_logprob=to_dev(a), grad_entropy=to_dev(b))
    assert (got["grad_hidden"] == 0).all() and (got["grad_weight"] == 0).all()


def test_long_bucket(vsa):
    say("support backward: one id in 5000 rows (a bucket longer than the LDS sort), H=64, V=100")
    rng = np.random.default_rng(12)
    T, H, V = 5000, 64, 100
    hb = workloads.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * 0.25).astype(np.float32))
    ids = np.stack([np.full(T, 7), rng.integers(8, V, T)], axis=1).astype(np.int64)
    y = np.where(rng.random(T) < 0.5, ids[:, 0], ids[:, 1])
    tau = np.ones(T, np.float32)
    a, b = rng.normal(0, 1, T).astype(np.float32), rng.normal(0, 1, T).astype(np.float32)
    got = vsa.score_support_backward(to_dev(y), to_dev(ids), hidden=bf16_tensor(hb), weight=bf16_tensor(wb),
                                     grad_logprob=to_dev(a), grad_entropy=to_dev(b))
    again = vsa.score_support_backward(to_dev(y), to_dev(ids), hidden=bf16_tensor(hb), weight=bf16_tensor(wb),
                                       grad_logprob=to_dev(a), grad_entropy=to_dev(b))
    assert torch.equal(got["grad_weight"], again["grad_weight"])
    ref = oracle.score_support_vjp(hb, "bf16", wb, ids, tau, y, a, b)
    h64, w64 = oracle.widen_bf16(hb), oracle.widen_bf16(wb)
    M = _magnitudes(h64, w64, ids, tau.astype(np.float64), y, a.astype(np.float64), b.astype(np.float64))
    _check(got, ref, M, h64, w64, ids, "long bucket")


def test_full_size_replay_workload(vsa):
    say("support backward: the replay workload T=2048 H=7168 V=129280 width 64: every grad_hidden row, 48 "
        "grad_weight rows, untouched rows zero, the trace identity, determinism")
    c = workload(3)
    T, H, V = c["T"], c["H"], c["V"]
    rng = np.random.default_rng(13)
    a, b = rng.normal(0, 1, T).astype(np.float32), rng.normal(0, 1, T).astype(np.float32)
    hid, w = bf16_tensor(c["hidden"]), bf16_tensor(c["weight"])
    ids, y = c["support_ids"], c["targets"]
    args = dict(hidden=hid, weight=w, grad_logprob=to_dev(a), grad_entropy=to_dev(b))
    got = vsa.score_support_backward(to_dev(y), to_dev(ids), **args)
    again = vsa.score_support_backward(to_dev(y), to_dev(ids), **args)
    assert torch.equal(got["grad_hidden"], again["grad_hidden"]) and torch.equal(got["grad_weight"], again["grad_weight"])
    sup = ids[ids >= 0]
    uniq, counts = np.unique(sup, return_counts=True)
    pick = np.concatenate([uniq[np.argsort(-counts)[:16]], rng.choice(uniq, 16, replace=False),
                           rng.choice(np.setdiff1d(np.arange(V), uniq), 16, replace=False)])
    ref = oracle.score_support_vjp(c["hidden"], "bf16", c["weight"], ids, 1.0, y, a, b, weight_rows=pick)
    h64 = oracle.widen_bf16(c["hidden"])
    # the bounds of the module notes, on every grad_hidden row and on the picked grad_weight rows
    gh = got["grad_hidden"].cpu().numpy().astype(np.float64)
    gw = got["grad_weight"][torch.from_numpy(pick).cuda()].cpu().numpy().astype(np.float64)
    bh = np.zeros_like(gh)
    bw = np.zeros_like(gw)
    where = {int(v): i for i, v in enumerate(pick)}
    for t in range(T):
        pos = np.nonzero(ids[t] >= 0)[0]
        sup_t = ids[t, pos]
        if sup_t.size == 0:
            continue
        w_sup = oracle.widen_bf16(c["weight"][sup_t])
        z = h64[t] @ w_sup.T
        lnp = z - (z.max() + np.log(np.sum(np.exp(z - z.max()))))
        p = np.exp(lnp)
        Hs = -np.sum(p * lnp)
        Mt = abs(a[t]) * ((sup_t == y[t]) + p) + abs(b[t]) * p * (np.abs(lnp) + Hs)
        bh[t] = REL * (Mt @ np.abs(w_sup))
        for j, v in enumerate(sup_t):
            i = where.get(int(v))
            if i is not None:
                bw[i] += REL * Mt[j] * np.abs(h64[t])
    for name, g, r, bd in (("grad_hidden", gh, ref["d_hidden"], bh + 1e-7), ("grad_weight rows", gw, ref["d_weight"],
                                                                            bw + 1e-7)):
        err = np.abs(g - r)
        say(f"  {name}: max |err| {err.max():.3e}, max err/bound {(err / bd).max():.3f}")
        assert (err <= bd).all(), name
    assert (gw[32:] == 0).all()  # ids in no support
    # both products hold the same dX: sum(grad_hidden * hidden) = sum(grad_weight * W)
    lhs = float((got["grad_hidden"].double() * hid.double()).sum())
    rhs = float((got["grad_weight"].double() * w.double()).sum())
    scale = float((got["grad_hidden"].double() * hid.double()).abs().sum())
    say(f"  trace identity: {lhs:.6e} vs {rhs:.6e}")
    assert abs(lhs - rhs) <= 1e-4 * scale
