"""GPU parity: the VJP of full-vocabulary scoring through the fused projection vs the fp64 oracle.

Tolerance, from the arithmetic: the kernel rounds each logit gradient dX to
bf16 (relative 2^-9) before the two products, whose bf16 x bf16 terms are
exact and whose sums are fp32, so element by element
  |grad_hidden - ref| <= (2^-8 + 1e-4) (|dX| |W|)[t, h] + eps_t (M |W|)[t, h]
  |grad_weight - ref| <= (2^-8 + 1e-4) (|dX|^T |bf16(hidden)|)[v, h] + (eps M)^T |bf16(hidden)|
with |dX| the oracle's (the 1e-4 covers the fp32 sums and the forward's
fp32 logits inside p).  The second term covers the cancellation inside dX:
the kernel recomputes p from the forward's fp32 LSE, whose round trip through
natural units moves ln p by up to eps_t = 2^-20 (1 + |LSE_t|), so each term of
dX is off by that relative amount even where the terms cancel (a one-token
row: dX = a (1 - p) = 0 exactly, about 1e-7 a on the GPU); M[t, v] =
(|a_t| + |b_t| (|ln p_v| + H_t + 1)) p_v / tau_t is the size of those terms."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_common import bf16_tensor, say, to_dev, workload

pytestmark = pytest.mark.gpu
REL = 2.0 ** -8 + 1e-4


@pytest.fixture(scope="module")
def vsa():
    import logprob_entropy_sampling_amd as m
    m.lib()
    return m


def _close(label, got, ref, bound):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape)
    say(f"  {label}: max |err| {err.max():.3e}, max |err|/bound {(err / np.maximum(bound, 1e-30)).max():.3f}")
    assert (err <= bound).all(), f"{label}: gpu {got[worst]!r} oracle {ref[worst]!r} bound {bound[worst]!r} at {worst}"


def term_sizes(x, tau, y, a, b):
    """(M, eps) of the module notes, from the oracle's logits x [R, V]."""
    R, V = x.shape
    tau = np.broadcast_to(np.asarray(tau, np.float64), (R,))
    a = np.zeros(R) if a is None else np.abs(np.asarray(a, np.float64))
    b = np.zeros(R) if b is None else np.abs(np.asarray(b, np.float64))
    M = np.zeros((R, V))
    eps = np.zeros(R)
    for t in range(R):
        if not (0 <= y[t] < V) or not (tau[t] > 0):
            continue
        z = x[t] / tau[t]
        m = z.max()
        if not np.isfinite(m):
            continue
        lse = m + np.log(np.sum(np.exp(z - m)))
        lnp = z - lse
        p = np.exp(lnp)
        H = -np.sum(np.where(p > 0, p * lnp, 0.0))
        M[t] = (a[t] + b[t] * (np.abs(np.where(p > 0, lnp, 0.0)) + H + 1.0)) * p / tau[t]
        eps[t] = 2.0 ** -20 * (1.0 + abs(lse))
    return M, eps


def _case(vsa, T, H, V, chunk, hidden_dtype, seed, with_lp=True, with_ent=True, bad_rows=()):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((T, H)).astype(np.float32)
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * 0.08).astype(np.float32))
    tau = rng.uniform(0.6, 1.4, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    for r in bad_rows:
        y[r] = V + 3  # a bad target: the forward marks the row BAD, it gets no gradient
    a = rng.normal(0, 1, T).astype(np.float32) if with_lp else None
    b = rng.normal(0, 1, T).astype(np.float32) if with_ent else None
    if hidden_dtype == "bf16":
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
    again = vsa.score_full_backward(to_dev(y), fw["lse"], fw["entropy"], hidden=hid, weight=w,
                                    grad_logprob=None if a is None else to_dev(a),
                                    grad_entropy=None if b is None else to_dev(b), temperature=to_dev(tau),
                                    vocab_chunk=chunk)
    assert torch.equal(got["grad_hidden"], again["grad_hidden"]) and torch.equal(got["grad_weight"], again["grad_weight"])
    ref = oracle.score_full_vjp(h_arg, hidden_dtype, wb, tau, y, a, b)
    adx = np.abs(ref["d_logits"])
    h64 = oracle.widen_bf16(oracle.round_f32_to_bf16(h) if hidden_dtype == "f32" else h_arg)
    w64 = oracle.widen_bf16(wb)
    M, eps = term_sizes(h64 @ w64.T, tau, y, a, b)
    eM = eps[:, None] * M
    _close("grad_hidden", got["grad_hidden"].cpu().numpy(), ref["d_hidden"],
           REL * (adx @ np.abs(w64)) + eM @ np.abs(w64) + 1e-30)
    _close("grad_weight", got["grad_weight"].cpu().numpy(), ref["d_weight"],
           REL * (adx.T @ np.abs(h64)) + eM.T @ np.abs(h64) + 1e-30)
    for r in bad_rows:
        assert (got["grad_hidden"][r] == 0).all()
    return got


@pytest.mark.parametrize("T,H,V,chunk,hdt", [
    (300, 256, 5003, 1024, "bf16"),    # 5 vocabulary chunks, the last ragged; H: 64-wide K stages
    (77, 96, 700, 256, "f32"),         # T and every chunk ragged; H = 96: the 32-wide pipelined sweep
    (130, 40, 2000, 600, "bf16"),      # H = 40: the register-staged sweep; chunk rounded up to 768
    (513, 1024, 30000, 8192, "bf16"),  # 4 chunks of 8192 rows
    (77, 128, 700, 256, "f32"),        # G^T from the sweep itself: T odd (a token pair with one missing row)
    (150, 192, 1500, 512, "bf16"),     # an odd number of 64-wide stages: G^T from the transpose kernel
])
def test_backward_matches_oracle(vsa, T, H, V, chunk, hdt):
    say(f"backward: T={T} H={H} V={V} vocab_chunk={chunk} hidden {hdt}, logprob and entropy gradients, bad rows")
    _case(vsa, T, H, V, chunk, hdt, seed=T + H + V, bad_rows=(3, T - 1))


@pytest.mark.parametrize("lp,ent", [(True, False), (False, True)])
def test_backward_one_term(vsa, lp, ent):
    say(f"backward: only the {'logprob' if lp else 'entropy'} gradient")
    _case(vsa, 200, 128, 3000, 1024, "bf16", seed=7, with_lp=lp, with_ent=ent)


def test_backward_full_size(vsa):
    say("backward: the fused workload T=4096 H=4096 V=151936, vocab_chunk 8192 and V (one chunk): sampled rows, "
        "column sums, the trace identity, determinism")
    c = workload(4)
    T, V = c["T"], c["V"]
    rng = np.random.default_rng(44)
    a = rng.normal(0, 1, T).astype(np.float32)
    b = rng.normal(0, 1, T).astype(np.float32)
    hid, w = bf16_tensor(c["hidden"]), bf16_tensor(c["weight"])
    y = to_dev(c["targets"])
    fw = vsa.score_full(y, hidden=hid, weight=w)
    rows = np.array([0, 255, 256, 1500, 2047, 3000, 4095])
    x = oracle.logits_from_hidden(c["hidden"], "bf16", c["weight"], rows=rows)
    dx = oracle.logit_vjp(x, 1.0, c["targets"][rows], a[rows], b[rows])
    w64 = oracle.widen_bf16(c["weight"])
    ref = dx @ w64
    M, eps = term_sizes(x, 1.0, c["targets"][rows], a[rows], b[rows])
    bound = REL * (np.abs(dx) @ np.abs(w64)) + (eps[:, None] * M) @ np.abs(w64) + 1e-30
    h64 = oracle.widen_bf16(c["hidden"])
    first = None
    for chunk in (8192, V):
        say(f"  vocab_chunk {chunk}")
        got = vsa.score_full_backward(y, fw["lse"], fw["entropy"], hidden=hid, weight=w, grad_logprob=to_dev(a),
                                      grad_entropy=to_dev(b), vocab_chunk=chunk)
        again = vsa.score_full_backward(y, fw["lse"], fw["entropy"], hidden=hid, weight=w, grad_logprob=to_dev(a),
                                        grad_entropy=to_dev(b), vocab_chunk=chunk)
        assert torch.equal(got["grad_hidden"], again["grad_hidden"])
        assert torch.equal(got["grad_weight"], again["grad_weight"])
        del again
        # grad_hidden of rows spread over every token tile, against the oracle row by row
        _close(f"grad_hidden rows (chunk {chunk})", got["grad_hidden"].cpu().numpy()[rows], ref, bound)
        gw = got["grad_weight"]
        # every row of dX sums to 0, so the columns of grad_weight sum to 0 up to the rounding of its terms
        colsum = gw.sum(0, dtype=torch.float64).abs().cpu().numpy()
        scale = gw.abs().sum(0, dtype=torch.float64).cpu().numpy()
        assert (colsum <= 2.0 ** -7 * scale + 1e-6).all(), float((colsum / scale).max())
        assert torch.isfinite(gw).all() and torch.isfinite(got["grad_hidden"]).all()
        # both products hold the same dX: sum(grad_hidden * hidden) = sum(grad_weight * W) = sum(dX * logits)
        gh64 = got["grad_hidden"].cpu().numpy().astype(np.float64)
        lhs, lhs_abs = float((gh64 * h64).sum()), float(np.abs(gh64 * h64).sum())
        gw_cpu = gw.cpu().numpy()
        rhs = rhs_abs = 0.0
        for v0 in range(0, V, 16384):
            prod = gw_cpu[v0:v0 + 16384].astype(np.float64) * w64[v0:v0 + 16384]
            rhs += float(prod.sum())
            rhs_abs += float(np.abs(prod).sum())
        say(f"  trace identity: {lhs:.6e} vs {rhs:.6e}")
        assert abs(lhs - rhs) <= 1e-4 * (lhs_abs + rhs_abs), (lhs, rhs)
        if first is None:
            first = got
        else:  # the chunking changes only grad_hidden's summation order, and grad_weight not at all
            assert torch.equal(first["grad_weight"], got["grad_weight"])
            dh = float((first["grad_hidden"] - got["grad_hidden"]).abs().max())
            assert dh <= 1e-4 * float(got["grad_hidden"].abs().max()), dh
