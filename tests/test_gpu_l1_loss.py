"""GPU parity: the weighted L1 distillation loss and its draft-logit gradient vs the fp64 oracle.

Tolerances: l1, accept_rate and the loss's num / den / loss within the float
tolerance; the gradient element by element within 1e-4 * |g| + 1e-6 * G_t,
G_t the row's largest |gradient| (fp32 gradients: every term of
q_v (s_v - S) carries the fp32 rounding of q_v and of S, relative ~1e-6),
or one bf16 ulp more for bf16 gradients.  Rows with tied draft and target
probabilities (s_v = 0) are compared with the same bound.  Where p_v and q_v
agree to within the kernel's own error in them the sign s_v is a decision
either value of which is correct.  That error: the bf16 path scales logits by
log2(e) rounded to 16 bits (relative 4.9e-6, so each ln p_v moves by that
fraction of x_v - E_p[x]), plus the fp32 rounding of the exponent arguments
and row sums; so |ln p_v - ln q_v| <= 2^-16 (1 + |x_v - E_p[x]| +
|y_v - E_q[y]|) counts as a tie, where such an element may differ by the
flip, 2 q_v c_t (c_t = grad_scale w_t / den), and every element of its row by
the flip's change of S_t, q_u sum 2 q_v c_t."""

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


def sign_flip_bound(a64, b64, coef):
    """The extra bound of the module notes for near-tied p_v, q_v, per element
    ([R, V]); coef[t] = |grad_scale w_t / den|."""
    def softmax(x):
        m = x.max(axis=1, keepdims=True)
        e = np.exp(x - m)
        return e / e.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        p, q = softmax(np.asarray(a64, np.float64)), softmax(np.asarray(b64, np.float64))
        x, y = np.asarray(a64, np.float64), np.asarray(b64, np.float64)
        dev = np.abs(x - np.sum(p * x, axis=1, keepdims=True)) + np.abs(y - np.sum(q * y, axis=1, keepdims=True))
        near = np.abs(np.log(p) - np.log(q)) <= 2.0 ** -16 * (1.0 + dev)
    p, q = np.nan_to_num(p), np.nan_to_num(q)
    near = np.nan_to_num(near) & (p > 0) & (q > 0)
    flip = np.where(near, 2.0 * q, 0.0)
    coef = np.asarray(coef, np.float64)[:, None]
    return coef * (flip + q * flip.sum(axis=1, keepdims=True))


def _grad_close(label, got, ref, bf16=False, extra=None):
    got = np.asarray(got, np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{label}: NaN rows differ"
    fin = np.isfinite(ref).all(axis=1)
    g, r = got[fin], ref[fin]
    G = np.abs(r).max(axis=1, keepdims=True)
    bound = (2.0 ** -8 if bf16 else 1e-4) * np.abs(r) + 1e-6 * G
    if extra is not None:
        bound = bound + np.asarray(extra)[fin] * (1.0 + (2.0 ** -8 if bf16 else 1e-4))
    err = np.abs(g - r)
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape) if err.size else None
    say(f"  {label}: max |err| {err.max() if err.size else 0:.3e} over {err.size} values")
    assert (err <= bound).all(), f"{label}: gpu {g[worst]!r} oracle {r[worst]!r} at {worst}"


def _case(vsa, a, b, w, grad_scale, grad_dtype, label):
    dt = torch.bfloat16
    ta, tb = bf16_tensor(workloads.to_bf16_bits(a)), bf16_tensor(workloads.to_bf16_bits(b))
    a64 = oracle.logits_from_logits(workloads.to_bf16_bits(a), "bf16")
    b64 = oracle.logits_from_logits(workloads.to_bf16_bits(b), "bf16")
    got = vsa.l1_loss(ta, tb, weights=None if w is None else to_dev(np.asarray(w, np.float32)), grad_scale=grad_scale,
                      grad_dtype=grad_dtype or dt)
    ref = oracle.weighted_l1_loss(a64, b64, None if w is None else np.asarray(w, np.float32), grad_scale=grad_scale)
    assert_close(f"{label} l1", got["l1"].cpu().numpy(), ref["l1"])
    assert_close(f"{label} accept", got["accept_rate"].cpu().numpy(), ref["accept_rate"])
    loss = got["loss"].cpu().numpy()
    assert_close(f"{label} num/den/loss", loss, np.array([ref["num"], ref["den"], ref["loss"]]))
    _grad_close(f"{label} grad", got["grad"].float().cpu().numpy(), ref["grad"], bf16=(grad_dtype or dt) == dt)
    return got


@pytest.mark.parametrize("V,grad_dtype", [(1000, torch.float32), (30001, torch.bfloat16), (151936, torch.float32)])
def test_loss_and_gradient(vsa, V, grad_dtype):
    say(f"l1 loss: T=24 V={V}, weights with zeros, a masked NaN row, identical rows, grad {grad_dtype}")
    rng = np.random.default_rng(V)
    T = 24
    a = (rng.standard_normal((T, V)) * 2).astype(np.float32)
    b = (a + rng.standard_normal((T, V)) * rng.uniform(0.05, 3.0, (T, 1))).astype(np.float32)
    b[3] = a[3]                 # identical: zero distance, zero gradient
    a[5, 7] = np.nan            # a NaN row with weight 0: masked
    w = rng.uniform(0.0, 2.0, T).astype(np.float32)
    w[[2, 5]] = 0.0
    got = _case(vsa, a, b, w, 0.5, grad_dtype, f"V={V}")
    g = got["grad"].float().cpu().numpy()
    assert (g[3] == 0).all() and (g[2] == 0).all() and (g[5] == 0).all()


def test_unweighted_and_fp32_logits(vsa):
    say("l1 loss: no weights (every weight 1), fp32 logits and unaligned rows")
    rng = np.random.default_rng(5)
    T, V = 9, 4097
    a = (rng.standard_normal((T, V + 1)) * 2).astype(np.float32)
    b = (a + rng.standard_normal((T, V + 1))).astype(np.float32)
    ta, tb = to_dev(a)[:, :V], to_dev(b)[:, :V]  # ld = V + 1: the scalar paths
    got = vsa.l1_loss(ta, tb)
    ref = oracle.weighted_l1_loss(a[:, :V].astype(np.float64), b[:, :V].astype(np.float64))
    assert_close("l1", got["l1"].cpu().numpy(), ref["l1"])
    assert_close("loss", got["loss"].cpu().numpy(), np.array([ref["num"], ref["den"], ref["loss"]]))
    _grad_close("grad", got["grad"].cpu().numpy(), ref["grad"])


def test_ties_at_large_magnitude(vsa):
    # tied maxima far from zero (the accurate exponent form): target mass on 2
    # ids, draft on 4; the gradient is q_v (s_v - S) on those ids
    say("l1 loss: tied maxima at 2^60 and 2^100 (bf16)")
    V = 2000
    a = np.zeros((3, V), np.float32)
    b = np.zeros((3, V), np.float32)
    for t, mag in enumerate([3.0, 2.0 ** 60, 2.0 ** 100]):
        a[t] = mag / 2
        b[t] = mag / 2
        a[t, [10, 20]] = mag
        b[t, [10, 20, 30, 40]] = mag
    _case(vsa, a, b, None, 1.0, torch.float32, "large magnitude")


def test_full_size_workload(vsa):
    say("l1 loss: the transforms/draft workload T=2048 V=151936, every row vs the oracle (bf16 gradient)")
    c = workload(5)
    T = c["T"]
    w = np.random.default_rng(9).uniform(0.0, 1.0, T).astype(np.float32)
    ta, tb = bf16_tensor(c["logits"]), bf16_tensor(c["draft"])
    got = vsa.l1_loss(ta, tb, weights=to_dev(w))
    again = vsa.l1_loss(ta, tb, weights=to_dev(w))
    assert all(torch.equal(got[k], again[k]) for k in ("l1", "loss", "grad"))
    dist = vsa.l1_distance(ta, tb)
    assert torch.equal(got["l1"], dist["l1"]) or torch.allclose(got["l1"], dist["l1"], atol=2e-6)
    ref = oracle_by_rows(lambda r: oracle.l1_distance(oracle.logits_from_logits(c["logits"], "bf16", rows=r),
                                                      oracle.logits_from_logits(c["draft"], "bf16", rows=r)), T)
    assert_close("l1", got["l1"].cpu().numpy(), ref["l1"])
    num = float(np.sum(w.astype(np.float64) * ref["l1"]))
    den = float(np.sum(w.astype(np.float64)))
    assert_close("num/den/loss", got["loss"].cpu().numpy(), np.array([num, den, num / den]))
    # the gradient of 64 rows spread over the batch (the oracle's full [T, V] would be 2.5 GB)
    rows = np.linspace(0, T - 1, 64).astype(int)
    gr = got["grad"][torch.from_numpy(rows).to(ta.device)].float().cpu().numpy()
    sub = oracle.weighted_l1_loss(oracle.logits_from_logits(c["logits"], "bf16", rows=rows),
                                  oracle.logits_from_logits(c["draft"], "bf16", rows=rows), w[rows])
    _grad_close("grad rows", gr, sub["grad"] * (float(np.sum(w[rows].astype(np.float64))) / den), bf16=True)


@pytest.mark.parametrize("T", [1, 300, 1023])
def test_rows_split_over_workgroups(vsa, T):
    # every row is split over 2..8 workgroups, more on small batches
    # (partials merged in a fixed order): every row, the loss and the
    # gradient against the oracle, a bad row of nonzero weight included
    say(f"l1 loss: T={T} V=6000 (8, 4 and 2 workgroups per row), a NaN row of weight 1")
    rng = np.random.default_rng(T)
    V = 6000
    a = (rng.standard_normal((T, V)) * 3).astype(np.float32)
    b = (a + rng.standard_normal((T, V)) * rng.uniform(0.1, 2.0, (T, 1))).astype(np.float32)
    w = rng.uniform(0.0, 2.0, T).astype(np.float32)
    if T > 1:
        b[T // 2, 11] = np.nan
        w[T // 2] = 1.0
        w[T // 3] = 0.0
    got = _case(vsa, a, b, w, 2.0, torch.float32, f"T={T}")
    again = vsa.l1_loss(bf16_tensor(workloads.to_bf16_bits(a)), bf16_tensor(workloads.to_bf16_bits(b)),
                        weights=to_dev(w), grad_scale=2.0, grad_dtype=torch.float32)
    for k in ("l1", "accept_rate", "loss", "grad"):
        assert torch.equal(got[k].nan_to_num(7.0), again[k].nan_to_num(7.0)), k
