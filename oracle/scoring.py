"""fp64 reference definitions of the scoring op (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module.  It imports nothing from the HIP
library or its binding.

Notation (shared with the pages): row ``t``, vocabulary id ``v``, input logit
``x[t, v]`` (bf16/fp32 logits, or the projection of the hidden state onto
the LM-head weight), temperature ``tau_t > 0``, tempered logit
``z = x / tau``, target id ``y_t``.  Natural logarithms; entropy in nats.

Per-row status bits (one byte per row):

* ``ST_EMPTY_SUPPORT``          the recorded support holds no id >= 0
* ``ST_TARGET_OUTSIDE_SUPPORT`` the target is not in the support (logprob -inf)
* ``ST_BAD_INPUT``              invalid data: every float output is NaN
* ``ST_FULL_VOCAB_FALLBACK``    the synthetic-EOS full-vocabulary fallback was used
* ``ST_SUPPORT_TRUNCATED``      the dense support ids were cut at the capacity
"""

from __future__ import annotations

import numpy as np

ST_OK = 0
ST_EMPTY_SUPPORT = 0x01
ST_TARGET_OUTSIDE_SUPPORT = 0x02
ST_BAD_INPUT = 0x04
ST_FULL_VOCAB_FALLBACK = 0x08
ST_SUPPORT_TRUNCATED = 0x10

BORDERLINE = 1e-6  # rows whose cut quantity lies this close to top_p / min_p


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    A bf16 value is the upper half of an IEEE binary32 word, so shifting the
    16 bits into the top of a 32-bit word gives the same number as float32,
    and float32 -> float64 is exact.
    """
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_f32_to_bf16(x) -> np.ndarray:
    """float32 -> bf16 bit patterns with round-to-nearest-even.

    This is the cast of the hidden state to the LM-head weight dtype before
    the selected projection (SkyRL PR #2004, review's suggested
    ``_selected_hidden_projection``: ``hidden.to(lm_head_weight.dtype)``).
    Written from the IEEE rule: keep the top 16 bits, round the dropped 16
    bits to nearest, ties to the even kept pattern.  NaN stays NaN (quiet).
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    kept = u >> np.uint64(16)
    dropped = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    round_up = (dropped > half) | ((dropped == half) & ((kept & np.uint64(1)) == np.uint64(1)))
    out = (kept + round_up.astype(np.uint64)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = (kept[nan] | np.uint64(0x40)).astype(np.uint16)
    return out


# ---------------------------------------------------------------------------
# Logits (the input to every score)
# ---------------------------------------------------------------------------

def logits_from_logits(logits, dtype: str, rows=None) -> np.ndarray:
    """Materialised logits (bf16 bits or float32) -> float64 ``x[rows, :]``."""
    a = np.asarray(logits)
    if rows is not None:
        a = a[np.asarray(rows)]
    if dtype == "bf16":
        return widen_bf16(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def logits_from_hidden(hidden, hidden_dtype: str, weight_bits, rows=None, cols=None) -> np.ndarray:
    """``x[t, v] = sum_h bf16(hidden[t, h]) * W[v, h]`` in float64.

    The projection of xorl issue #71 section 1 ("chunked projection") and of
    the selected projection in SkyRL PR #2004: float32 hidden states are
    first cast to the weight dtype (bf16, round-to-nearest-even); the weight
    rows are vocabulary ids.  Products of two bf16 numbers are exact in
    float64, so up to the float64 summation this is the exact dot product.
    ``cols`` selects weight rows (vocabulary ids); ``rows`` selects tokens.
    """
    h = np.asarray(hidden)
    if rows is not None:
        h = h[np.asarray(rows)]
    if hidden_dtype == "f32":
        h64 = widen_bf16(round_f32_to_bf16(h))
    elif hidden_dtype == "bf16":
        h64 = widen_bf16(h)
    else:
        raise ValueError(hidden_dtype)
    w = np.asarray(weight_bits, dtype=np.uint16)
    if cols is not None:
        w = w[np.asarray(cols)]
    # Widening the whole weight to float64 at once would need 8 bytes per
    # entry; widen it in blocks of vocabulary rows (each output element is
    # still one float64 dot product over H).
    out = np.empty((h64.shape[0], w.shape[0]), dtype=np.float64)
    step = 16384
    for v0 in range(0, w.shape[0], step):
        out[:, v0:v0 + step] = h64 @ widen_bf16(w[v0:v0 + step]).T
    return out


# ---------------------------------------------------------------------------
# Helpers on one row of tempered logits
# ---------------------------------------------------------------------------

def _valid_tau(tau) -> bool:
    return bool(np.isfinite(tau) and tau > 0.0)


def _lse_and_entropy(z: np.ndarray):
    """Log-sum-exp and entropy of softmax(z) for one row (two-pass max shift).

    ``LSE = m + ln sum_v exp(z_v - m)`` with ``m = max_v z_v``;
    ``H = -sum_v p_v ln p_v`` with ``p_v = exp(z_v - LSE)`` and
    ``ln p_v = z_v - LSE``; a zero-probability entry (z = -inf) adds 0.
    Returns ``(nan, nan)`` when the row holds a NaN or +inf or is all -inf.
    """
    if z.size == 0 or np.isnan(z).any():
        return np.nan, np.nan
    m = z.max()
    if not np.isfinite(m):
        return np.nan, np.nan
    s = np.sum(np.exp(z - m))
    lse = m + np.log(s)
    lnp = z - lse
    p = np.exp(lnp)
    h = -np.sum(np.where(p > 0.0, p * np.where(np.isfinite(lnp), lnp, 0.0), 0.0))
    return lse, h


# ---------------------------------------------------------------------------
# O1: full-vocabulary scoring
# ---------------------------------------------------------------------------

def score_full(x, tau, targets) -> dict:
    """Full-vocabulary LSE, selected logprob and entropy of softmax(x / tau).

    The existing full-vocabulary path of SkyRL PR #2004 (Implementation: the
    path kept when replay is off) and the op of xorl issue #71 section 1
    (log-sum-exp over the vocabulary, then the selected logprob).  Temperature
    divides the finished dot product (SkyRL PR #2004, suggested
    ``_selected_hidden_projection``: ``... .sum(dim=-1) / temperature``).

    x: float64 [R, V]; tau: [R] (or scalar); targets: int [R].
    Returns float64 ``lse``, ``logprob``, ``entropy`` and uint8 ``status``.
    Rows with tau <= 0 / non-finite, a target outside [0, V), a NaN or +inf
    logit, or only -inf logits are ``ST_BAD_INPUT`` with NaN outputs.
    """
    x = np.asarray(x, dtype=np.float64)
    R, V = x.shape
    tau = np.broadcast_to(np.asarray(tau, dtype=np.float64), (R,))
    targets = np.asarray(targets, dtype=np.int64)
    lse = np.full(R, np.nan)
    logprob = np.full(R, np.nan)
    entropy = np.full(R, np.nan)
    status = np.zeros(R, dtype=np.uint8)
    for t in range(R):
        y = int(targets[t])
        if not _valid_tau(tau[t]) or not (0 <= y < V):
            status[t] = ST_BAD_INPUT
            continue
        z = x[t] / tau[t]
        l, h = _lse_and_entropy(z)
        if not np.isfinite(l):
            status[t] = ST_BAD_INPUT
            continue
        lse[t] = l
        logprob[t] = z[y] - l
        entropy[t] = h
    return {"lse": lse, "logprob": logprob, "entropy": entropy, "status": status}


# ---------------------------------------------------------------------------
# O2: recorded-support scoring
# ---------------------------------------------------------------------------

def score_support(logit_fn, V: int, ids, tau, targets, fallback=None) -> dict:
    """Logprob and entropy renormalised over a recorded sampler support.

    SkyRL PR #2004 (Problem; Implementation; last paragraph of the
    description): the support of row t is ``S_t = {ids[t, j] : ids[t, j] >= 0}``
    (dense padded ids, no CSR); the policy is restricted to ``S_t`` and
    renormalised, so ``logprob_S = z_y - LSE_S`` and
    ``H_S = -sum_{v in S} p_v ln p_v`` with ``p_v = exp(z_v - LSE_S)``.  A
    singleton support gives exactly zero entropy and zero logprob.

    Rows with no id >= 0 are ``ST_EMPTY_SUPPORT`` and are left out of the
    entropy (entropy 0).  When ``fallback[t]`` is set (a synthetic-EOS row)
    their logprob is the full-vocabulary one (``ST_FULL_VOCAB_FALLBACK``);
    otherwise it is 0.

    ``logit_fn(t, cols)`` returns float64 ``x[t, cols]``.  ``ST_BAD_INPUT``
    (NaN outputs): tau invalid, an id >= V, a repeated id, or - on a row that
    is scored - a target outside [0, V) or a support whose LSE is not finite.
    A target outside a non-empty support gives logprob -inf and
    ``ST_TARGET_OUTSIDE_SUPPORT``.
    """
    ids = np.asarray(ids, dtype=np.int64)
    R = ids.shape[0]
    tau = np.broadcast_to(np.asarray(tau, dtype=np.float64), (R,))
    targets = np.asarray(targets, dtype=np.int64)
    logprob = np.full(R, np.nan)
    entropy = np.full(R, np.nan)
    status = np.zeros(R, dtype=np.uint8)
    for t in range(R):
        row = ids[t]
        sup = row[row >= 0]
        if not _valid_tau(tau[t]) or (sup >= V).any() or len(np.unique(sup)) != len(sup):
            status[t] = ST_BAD_INPUT
            continue
        y = int(targets[t])
        if sup.size == 0:
            if fallback is not None and bool(fallback[t]):
                full = score_full(logit_fn(t, np.arange(V))[None, :], tau[t], [y])
                if full["status"][0] & ST_BAD_INPUT:
                    status[t] = ST_BAD_INPUT
                    continue
                logprob[t] = full["logprob"][0]
                status[t] = ST_EMPTY_SUPPORT | ST_FULL_VOCAB_FALLBACK
            else:
                logprob[t] = 0.0
                status[t] = ST_EMPTY_SUPPORT
            entropy[t] = 0.0
            continue
        if not (0 <= y < V):
            status[t] = ST_BAD_INPUT
            continue
        z = logit_fn(t, sup) / tau[t]
        l, h = _lse_and_entropy(z)
        if not np.isfinite(l):
            status[t] = ST_BAD_INPUT
            continue
        entropy[t] = h
        hit = np.nonzero(sup == y)[0]
        if hit.size:
            logprob[t] = z[hit[0]] - l
        else:
            logprob[t] = -np.inf
            status[t] = ST_TARGET_OUTSIDE_SUPPORT
    return {"logprob": logprob, "entropy": entropy, "status": status}


# ---------------------------------------------------------------------------
# O3: sampling transforms (temperature -> top-k -> top-p -> min-p)
# ---------------------------------------------------------------------------

def _rank_order(z: np.ndarray) -> np.ndarray:
    """Token ids sorted by tempered logit descending, ties by ascending id."""
    ids = np.arange(z.size)
    return np.lexsort((ids, -z))


def score_transforms(x, tau, top_k, top_p, min_p, targets, cap: int = 0) -> dict:
    """Scores over the top-k / top-p / min-p support of softmax(x / tau).

    The program named in xorl issue #71 section 3 - temperature, then stable
    token-id top-k, inclusive top-p, min-p against the original row max - up
    to (not including) the seeded Gumbel draw:

    1. ``z = x / tau``; order ``pi`` = ids by (z descending, id ascending).
    2. ``L_k = V`` if ``k <= 0`` or ``k >= V``, else ``k``.
    3. On the first ``L_k`` ranks, masses ``p'_j = exp(z_pi(j)) / sum`` over
       those ranks; exclusive prefix ``E_j = sum_{i<j} p'_i`` (sequential in
       rank order).  Inclusive top-p keeps rank j iff ``E_j < top_p`` (the
       token that crosses top_p is kept); ``top_p >= 1`` is the identity.
    4. Min-p keeps rank j iff ``exp(z_pi(j) - z_pi(0)) >= min_p`` - relative
       to the original (untruncated, unrenormalised) row max; ``min_p <= 0``
       disables it.
    5. Every filter keeps a prefix of ``pi``; the support is the shortest,
       ``S = pi[0:L]`` with ``L = min(L_k, L_p, L_m) >= 1``.

    Outputs per row: support-conditioned ``logprob`` / ``entropy`` (as in
    ``score_support``), ``status``, the support descriptor ``support_len = L``,
    ``threshold_logit = x_pi(L-1)`` (the input logit),
    ``threshold_ties = #{j < L : x_pi(j) == x_pi(L-1)}``, dense ids
    ``pi[0:min(L, cap)]`` padded with -1 (``ST_SUPPORT_TRUNCATED`` if
    ``cap > 0`` and ``L > cap``), and ``full_lse`` (the full-vocabulary LSE).
    Oracle-only extras: ``borderline_top_p`` (``top_p < 1`` and some
    ``E_j``, j <= L_k, within 1e-6 of top_p) and ``borderline_min_p``
    (``min_p > 0`` and some ``exp(z - z_max)`` within 1e-6 of min_p).

    ``ST_BAD_INPUT`` (NaN floats, support_len 0, ids -1): tau invalid,
    top_p NaN or <= 0, min_p NaN or > 1, target outside [0, V), or a row
    whose full LSE is not finite.
    """
    x = np.asarray(x, dtype=np.float64)
    R, V = x.shape
    tau = np.broadcast_to(np.asarray(tau, dtype=np.float64), (R,))
    top_k = np.broadcast_to(np.asarray(top_k, dtype=np.int64), (R,))
    top_p = np.broadcast_to(np.asarray(top_p, dtype=np.float64), (R,))
    min_p = np.broadcast_to(np.asarray(min_p, dtype=np.float64), (R,))
    targets = np.asarray(targets, dtype=np.int64)
    out = {
        "logprob": np.full(R, np.nan),
        "entropy": np.full(R, np.nan),
        "status": np.zeros(R, dtype=np.uint8),
        "support_len": np.zeros(R, dtype=np.int32),
        "threshold_logit": np.full(R, np.nan),
        "threshold_ties": np.zeros(R, dtype=np.int32),
        "support_ids": np.full((R, max(cap, 0)), -1, dtype=np.int64),
        "full_lse": np.full(R, np.nan),
        "borderline_top_p": np.zeros(R, dtype=bool),
        "borderline_min_p": np.zeros(R, dtype=bool),
    }
    for t in range(R):
        y = int(targets[t])
        p_top, p_min = top_p[t], min_p[t]
        if (not _valid_tau(tau[t]) or np.isnan(p_top) or p_top <= 0.0
                or np.isnan(p_min) or p_min > 1.0 or not (0 <= y < V)):
            out["status"][t] = ST_BAD_INPUT
            continue
        z = x[t] / tau[t]
        full_lse, _ = _lse_and_entropy(z)
        if not np.isfinite(full_lse):
            out["status"][t] = ST_BAD_INPUT
            continue
        out["full_lse"][t] = full_lse

        order = _rank_order(z)
        zs = z[order]
        k = int(top_k[t])
        L_k = V if (k <= 0 or k >= V) else k

        # inclusive top-p on the top-k renormalised masses
        e = np.exp(zs[:L_k] - zs[0])
        mass = e / np.sum(e)
        excl = np.concatenate(([0.0], np.cumsum(mass)))  # excl[j] = E_j, excl[L_k] = total
        if p_top >= 1.0:
            L_p = L_k
        else:
            L_p = int(np.count_nonzero(excl[:L_k] < p_top))
            out["borderline_top_p"][t] = bool(np.any(np.abs(excl - p_top) <= BORDERLINE))

        # min-p relative to the original row max
        if p_min <= 0.0:
            L_m = V
        else:
            rel = np.exp(zs - zs[0])
            L_m = int(np.count_nonzero(rel >= p_min))
            out["borderline_min_p"][t] = bool(np.any(np.abs(rel - p_min) <= BORDERLINE))

        L = min(L_k, L_p, L_m)
        sup = order[:L]
        out["support_len"][t] = L
        thr = x[t, order[L - 1]]
        out["threshold_logit"][t] = thr
        out["threshold_ties"][t] = int(np.count_nonzero(x[t, sup] == thr))
        if cap > 0:
            n = min(L, cap)
            out["support_ids"][t, :n] = sup[:n]
            if L > cap:
                out["status"][t] |= ST_SUPPORT_TRUNCATED

        lse_s, h_s = _lse_and_entropy(zs[:L])
        if not np.isfinite(lse_s):
            out["status"][t] = ST_BAD_INPUT
            out["support_len"][t] = 0
            out["threshold_logit"][t] = np.nan
            out["threshold_ties"][t] = 0
            out["support_ids"][t, :] = -1
            out["full_lse"][t] = np.nan
            continue
        out["entropy"][t] = h_s
        rank_y = int(np.nonzero(order == y)[0][0])
        if rank_y < L:
            out["logprob"][t] = z[y] - lse_s
        else:
            out["logprob"][t] = -np.inf
            out["status"][t] |= ST_TARGET_OUTSIDE_SUPPORT
    return out


# ---------------------------------------------------------------------------
# O4: draft/target softmax L1 distance
# ---------------------------------------------------------------------------

def l1_distance(x_target, x_draft) -> dict:
    """Per-row ``L1 = sum_v |softmax(x_target)_v - softmax(x_draft)_v|``.

    DeepSpec PR #87 (Purpose): the per-token probability distance computed
    once and shared by ``accept_rate = clamp(1 - 0.5 * L1, 0, 1)`` and the L1
    loss.  No temperature (the page applies none).  A row whose target or
    draft LSE is not finite gives NaN for both outputs.
    """
    a = np.asarray(x_target, dtype=np.float64)
    b = np.asarray(x_draft, dtype=np.float64)
    R = a.shape[0]
    l1 = np.full(R, np.nan)
    acc = np.full(R, np.nan)
    for t in range(R):
        la, _ = _lse_and_entropy(a[t])
        lb, _ = _lse_and_entropy(b[t])
        if not (np.isfinite(la) and np.isfinite(lb)):
            continue
        p = np.exp(a[t] - la)
        q = np.exp(b[t] - lb)
        d = np.sum(np.abs(p - q))
        l1[t] = d
        acc[t] = min(1.0, max(0.0, 1.0 - 0.5 * d))
    return {"l1": l1, "accept_rate": acc}
