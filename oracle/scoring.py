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


def round_f64_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit patterns, one rounding to nearest, ties to even.

    Written from the IEEE rule for an 8-bit significand: with
    x = m 2^e (0.5 <= |m| < 1), the unit in the last place is 2^(e - 8), but
    never below 2^-133, the spacing of the subnormal bf16 numbers; x is
    scaled by that power of two (exact), rounded to an integer, ties to
    even, and scaled back.  Magnitudes that round to 2^128 or beyond become
    infinities; NaN becomes the quiet NaN 0x7FC0; the sign of zero is kept.
    """
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    xs = np.where(nan, 0.0, x)
    _, e = np.frexp(xs)
    q = np.maximum(e - 8, -133)
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.ldexp(np.rint(np.ldexp(xs, -q)), q)
    y = np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, xs), y)
    bits = (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[nan] = np.uint16(0x7FC0)
    return bits


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

def bf16_logits_from_hidden(hidden, hidden_dtype: str, weight_bits, rows=None) -> np.ndarray:
    """The bf16 logits of the hidden/weight source for the sampling transforms.

    xorl issue #71 (section 3 and "Proposed direction" item 3) asks for the
    transform program on the chunked projection; it ranks bf16 logits.  The
    reading taken here: the logits it ranks are the projection rounded once
    to bf16 (nearest, ties to even), ``round_f64_to_bf16(logits_from_hidden)``.
    (A device computes the projection in fp32 first; the two agree wherever
    that fp32 sum is exact.)  Returns bf16 bit patterns ``[rows, V]``."""
    return round_f64_to_bf16(logits_from_hidden(hidden, hidden_dtype, weight_bits, rows=rows))


def _valid_tau(tau) -> bool:
    return bool(np.isfinite(tau) and tau > 0.0)


def _log_softmax(x: np.ndarray, tau: float = 1.0):
    """Log-softmax, log-sum-exp and entropy of softmax(x / tau) for one row.

    The plain definition, evaluated from shifted values so that no term is
    lost at any magnitude: with ``x_max = max_v x_v``,
    ``d_v = (x_v - x_max) / tau`` (the difference of two widened inputs is
    exact; the division rounds once), ``ln s = ln sum_v exp(d_v)``,
    ``ln p_v = d_v - ln s``, ``LSE = x_max / tau + ln s`` and
    ``H = -sum_v p_v ln p_v``.  (Forming ``z_v - LSE`` from the unshifted
    ``z = x / tau`` instead drops ``ln s`` below one float64 ulp of ``z``
    once ``|z|`` passes about 2^42.)  Since ``tau > 0``, ``x_max / tau`` is
    the maximum of ``z``.  A zero-probability entry (``x = -inf``) adds 0.
    Returns ``(lse, lnp, h)``; ``(nan, None, nan)`` when the row is empty,
    holds a NaN or +inf, or is all -inf.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0 or np.isnan(x).any():
        return np.nan, None, np.nan
    m = x.max()
    if not np.isfinite(m):
        return np.nan, None, np.nan
    d = (x - m) / tau
    ln_s = np.log(np.sum(np.exp(d)))
    lnp = d - ln_s
    p = np.exp(lnp)
    h = -np.sum(np.where(p > 0.0, p * np.where(np.isfinite(lnp), lnp, 0.0), 0.0))
    return m / tau + ln_s, lnp, h


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
        l, lnp, h = _log_softmax(x[t], tau[t])
        if not np.isfinite(l):
            status[t] = ST_BAD_INPUT
            continue
        lse[t] = l
        logprob[t] = lnp[y]
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
        l, lnp, h = _log_softmax(logit_fn(t, sup), tau[t])
        if not np.isfinite(l):
            status[t] = ST_BAD_INPUT
            continue
        entropy[t] = h
        hit = np.nonzero(sup == y)[0]
        if hit.size:
            logprob[t] = lnp[hit[0]]
        else:
            logprob[t] = -np.inf
            status[t] = ST_TARGET_OUTSIDE_SUPPORT
    return {"logprob": logprob, "entropy": entropy, "status": status}


# ---------------------------------------------------------------------------
# O3: sampling transforms (temperature -> top-k -> top-p -> min-p)
# ---------------------------------------------------------------------------

def _rank_order(x: np.ndarray) -> np.ndarray:
    """Token ids sorted by logit descending, ties by ascending id."""
    ids = np.arange(x.size)
    return np.lexsort((ids, -x))


def _transform_outputs(R: int, cap: int) -> dict:
    return {
        "logprob": np.full(R, np.nan),
        "entropy": np.full(R, np.nan),
        "status": np.zeros(R, dtype=np.uint8),
        "support_len": np.zeros(R, dtype=np.int32),
        "threshold_logit": np.full(R, np.nan),
        "threshold_ties": np.zeros(R, dtype=np.int32),
        "support_ids": np.full((R, max(cap, 0)), -1, dtype=np.int64),
    }


def _prefix_outputs(out: dict, t: int, x_row: np.ndarray, order: np.ndarray, L: int, tau: float, y: int,
                    cap: int) -> None:
    """Descriptor, dense ids and scores of the support ``pi[0:L]`` of row t.

    ``support_len = L``, ``threshold_logit = x_pi(L-1)``,
    ``threshold_ties = #{j < L : x_pi(j) == x_pi(L-1)}``, dense ids
    ``pi[0:min(L, cap)]`` padded with -1 (``ST_SUPPORT_TRUNCATED`` past the
    capacity), and the logprob / entropy renormalised over the support as in
    ``score_support`` (the support always holds the row maximum).
    """
    sup = order[:L]
    out["support_len"][t] = L
    thr = x_row[order[L - 1]]
    out["threshold_logit"][t] = thr
    out["threshold_ties"][t] = int(np.count_nonzero(x_row[sup] == thr))
    if cap > 0:
        n = min(L, cap)
        out["support_ids"][t, :n] = sup[:n]
        if L > cap:
            out["status"][t] |= ST_SUPPORT_TRUNCATED
    lse_s, lnp_s, h_s = _log_softmax(x_row[sup], tau)
    if not np.isfinite(lse_s):
        out["status"][t] = ST_BAD_INPUT
        out["support_len"][t] = 0
        out["threshold_logit"][t] = np.nan
        out["threshold_ties"][t] = 0
        out["support_ids"][t, :] = -1
        if "full_lse" in out:
            out["full_lse"][t] = np.nan
        return
    out["entropy"][t] = h_s
    rank_y = int(np.nonzero(order == y)[0][0])
    if rank_y < L:
        out["logprob"][t] = lnp_s[rank_y]
    else:
        out["logprob"][t] = -np.inf
        out["status"][t] |= ST_TARGET_OUTSIDE_SUPPORT


def score_prefix_support(x, tau, support_len, targets, cap: int = 0) -> dict:
    """Descriptor, dense ids and scores of a given support length per row.

    The last steps of the transform program (support = the first
    ``support_len[t]`` ranks of ``pi``, ids by logit descending, ties by
    ascending id; xorl issue #71 section 3) for a cut chosen by the caller.
    It serves rows whose top-p or min-p cut lies within the borderline band,
    where several cuts are equally correct: given the cut the kernel chose,
    everything else is fixed.  ``support_len[t]`` must lie in [1, V].
    """
    x = np.asarray(x, dtype=np.float64)
    R, V = x.shape
    tau = np.broadcast_to(np.asarray(tau, dtype=np.float64), (R,))
    targets = np.asarray(targets, dtype=np.int64)
    out = _transform_outputs(R, cap)
    for t in range(R):
        L = int(support_len[t])
        if not 1 <= L <= V:
            raise ValueError(f"row {t}: support_len {L} outside [1, {V}]")
        _prefix_outputs(out, t, x[t], _rank_order(x[t]), L, tau[t], int(targets[t]), cap)
    return out


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
    ``E_j``, j <= L_k, within 1e-6 of top_p), ``borderline_min_p``
    (``min_p > 0`` and some ``exp(z - z_max)`` within 1e-6 of min_p), and the
    band ``support_len_lo .. support_len_hi`` of the cut when top_p and min_p
    move by up to 1e-6 (a single value on a row that is not borderline).

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
    out = _transform_outputs(R, cap)
    out.update({
        "full_lse": np.full(R, np.nan),
        "borderline_top_p": np.zeros(R, dtype=bool),
        "borderline_min_p": np.zeros(R, dtype=bool),
        "support_len_lo": np.zeros(R, dtype=np.int32),
        "support_len_hi": np.zeros(R, dtype=np.int32),
    })
    for t in range(R):
        y = int(targets[t])
        p_top, p_min = top_p[t], min_p[t]
        if (not _valid_tau(tau[t]) or np.isnan(p_top) or p_top <= 0.0
                or np.isnan(p_min) or p_min > 1.0 or not (0 <= y < V)):
            out["status"][t] = ST_BAD_INPUT
            continue
        full_lse, _, _ = _log_softmax(x[t], tau[t])
        if not np.isfinite(full_lse):
            out["status"][t] = ST_BAD_INPUT
            continue
        out["full_lse"][t] = full_lse

        # tau > 0 keeps the order of x, so ranking x ranks z = x / tau exactly
        order = _rank_order(x[t])
        xs = x[t, order]
        d = (xs - xs[0]) / tau[t]  # z - z_max from the exact input difference
        k = int(top_k[t])
        L_k = V if (k <= 0 or k >= V) else k

        # inclusive top-p on the top-k renormalised masses
        e = np.exp(d[:L_k])
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
            rel = np.exp(d)
            L_m = int(np.count_nonzero(rel >= p_min))
            out["borderline_min_p"][t] = bool(np.any(np.abs(rel - p_min) <= BORDERLINE))

        L = min(L_k, L_p, L_m)
        _prefix_outputs(out, t, x[t], order, L, tau[t], y, cap)

        # the cut band: L when top_p and min_p move by up to BORDERLINE (one
        # value on every row that is not borderline)
        lo_p = hi_p = L_k
        if p_top < 1.0:
            lo_p = int(np.count_nonzero(excl[:L_k] < p_top - BORDERLINE))
            hi_p = int(np.count_nonzero(excl[:L_k] < p_top + BORDERLINE))
        lo_m = hi_m = V
        if p_min > 0.0:
            lo_m = int(np.count_nonzero(rel >= p_min + BORDERLINE))
            hi_m = int(np.count_nonzero(rel >= p_min - BORDERLINE))
        if out["status"][t] & ST_BAD_INPUT:
            continue
        out["support_len_lo"][t] = max(1, min(L_k, lo_p, lo_m))
        out["support_len_hi"][t] = min(L_k, hi_p, hi_m)
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
        la, lnp_a, _ = _log_softmax(a[t])
        lb, lnq_b, _ = _log_softmax(b[t])
        if not (np.isfinite(la) and np.isfinite(lb)):
            continue
        p = np.exp(lnp_a)
        q = np.exp(lnq_b)
        d = np.sum(np.abs(p - q))
        l1[t] = d
        acc[t] = min(1.0, max(0.0, 1.0 - 0.5 * d))
    return {"l1": l1, "accept_rate": acc}


# ---------------------------------------------------------------------------
# O5: weighted L1 distillation loss and its draft-logit gradient
# ---------------------------------------------------------------------------

def weighted_l1_loss(x_target, x_draft, weights=None, grad_scale: float = 1.0) -> dict:
    """The weighted L1 distillation loss built on the shared distance.

    DeepSpec PR #87 (Purpose; Test Plan): the per-token L1 distance, computed
    once, gives both ``accept_rate = clamp(1 - 0.5 * L1, 0, 1)`` and the
    weighted L1 loss, whose numerator and denominator are
    ``num = sum_t w_t L1_t`` and ``den = sum_t w_t``; the loss is
    ``num / den`` and its gradient flows into the draft logits (the target is
    a fixed reference).  With ``q = softmax(x_draft)``, ``p =
    softmax(x_target)`` and ``s_u = sign(q_u - p_u)`` (sign 0 where they are
    equal, as the subgradient of |.| is taken at 0):

        d L1_t / d x_draft[t, v] = q_v (s_v - sum_u s_u q_u)
        grad[t, v] = grad_scale * (w_t / den) * q_v (s_v - sum_u s_u q_u)

    Reading where the page is silent: a row of weight 0 adds nothing to num
    and has zero gradient even when its distance is NaN (a loss mask); a
    weight must be finite and >= 0.  ``weights`` None means 1 for every row.
    Returns ``l1``, ``accept_rate`` (per row, as ``l1_distance``), ``num``,
    ``den``, ``loss`` and ``grad`` (float64 [R, V]).
    """
    a = np.asarray(x_target, dtype=np.float64)
    b = np.asarray(x_draft, dtype=np.float64)
    R, V = a.shape
    w = np.ones(R) if weights is None else np.asarray(weights, dtype=np.float64)
    base = l1_distance(a, b)
    num = 0.0
    for t in range(R):
        if w[t] != 0.0:
            num += w[t] * base["l1"][t]
    den = float(np.sum(w))
    grad = np.zeros((R, V))
    for t in range(R):
        if w[t] == 0.0:
            continue
        la, lnp, _ = _log_softmax(a[t])
        lb, lnq, _ = _log_softmax(b[t])
        if not (np.isfinite(la) and np.isfinite(lb)):
            grad[t] = np.nan
            continue
        p, q = np.exp(lnp), np.exp(lnq)
        s = np.sign(q - p)
        grad[t] = grad_scale * (w[t] / den) * q * (s - np.sum(s * q))
    return {"l1": base["l1"], "accept_rate": base["accept_rate"], "num": num, "den": den,
            "loss": num / den if den != 0.0 else np.nan, "grad": grad}


# ---------------------------------------------------------------------------
# O6: the vector-Jacobian product of full-vocabulary scoring (fused source)
# ---------------------------------------------------------------------------

def logit_vjp(x, tau, targets, grad_logprob=None, grad_entropy=None) -> np.ndarray:
    """d(sum_t a_t logprob_t + b_t H_t) / d x[t, v] for full-vocabulary scores.

    xorl issue #71, section 1 (the op ends in "selected logprob + VJP") and
    SkyRL PR #2004 (gradients through logprob and entropy): with
    ``z = x / tau``, ``p = softmax(z)``, ``ln p_v = z_v - LSE`` and
    ``H = -sum p ln p``,

        d logprob / d z_v = [v = y] - p_v
        d H / d z_v       = -p_v (ln p_v + H)      (= -p_v (z_v - (LSE - H)))

    and ``d / d x = (d / d z) / tau``.  ``a`` = grad_logprob, ``b`` =
    grad_entropy ([R] each, None meaning 0).  A BAD_INPUT row of score_full
    (invalid tau or target, or an LSE that is not finite) gets a zero row.
    """
    x = np.asarray(x, dtype=np.float64)
    R, V = x.shape
    tau = np.broadcast_to(np.asarray(tau, dtype=np.float64), (R,))
    a = np.zeros(R) if grad_logprob is None else np.asarray(grad_logprob, dtype=np.float64)
    b = np.zeros(R) if grad_entropy is None else np.asarray(grad_entropy, dtype=np.float64)
    targets = np.asarray(targets, dtype=np.int64)
    out = np.zeros((R, V))
    for t in range(R):
        y = int(targets[t])
        if not _valid_tau(tau[t]) or not (0 <= y < V):
            continue
        lse, lnp, h = _log_softmax(x[t], tau[t])
        if not np.isfinite(lse):
            continue
        p = np.exp(lnp)
        plnp = np.where(p > 0.0, p * np.where(np.isfinite(lnp), lnp, 0.0), 0.0)
        dz = -a[t] * p - b[t] * (plnp + p * h)
        dz[y] += a[t]
        out[t] = dz / tau[t]
    return out


def score_support_vjp(hidden, hidden_dtype: str, weight_bits, ids, tau, targets, grad_logprob=None,
                      grad_entropy=None, weight_rows=None) -> dict:
    """Gradients of sum_t (a_t logprob_t + b_t H_t) of the recorded-support
    scores over the fused projection (``score_support`` with
    ``x = bf16(hidden) W^T``) with respect to the hidden state and the weight.

    SkyRL PR #2004 (Implementation: entropy and gradient tracking over the
    recorded support; the description: a singleton support has exactly zero
    entropy and zero entropy gradient): over ``S_t`` the scores are those of
    ``p = softmax(z_S)``, so for v in S_t

        d logprob / d z_v = [v = y] - p_v,   d H / d z_v = -p_v (ln p_v + H_S)

    and nothing outside S_t; ``d/dx = (d/dz) / tau``, then the chain rule
    through the projection: ``d_hidden[t] = sum_{v in S_t} dX[t, v] W[v]``,
    ``d_weight[v] = sum_{t : v in S_t} dX[t, v] bf16(hidden[t])``.
    Rows that get no gradient: BAD_INPUT rows of score_support, rows with an
    empty support (their scores are constants; a synthetic-EOS row's
    full-vocabulary logprob is score_full_vjp's), and - for the logprob term
    only - a target outside the support (its logprob is the constant -inf).

    ``weight_rows``: the vocabulary ids whose d_weight rows are returned
    (default every id).  Returns ``d_hidden`` [R, H], ``d_weight``
    [len(weight_rows), H] and ``d_support`` [R, width] (dX at each id's
    position, 0 at padding), float64."""
    h = np.asarray(hidden)
    h64 = widen_bf16(round_f32_to_bf16(h)) if hidden_dtype == "f32" else widen_bf16(h)
    w = np.asarray(weight_bits, dtype=np.uint16)
    V = w.shape[0]
    ids = np.asarray(ids, dtype=np.int64)
    R, width = ids.shape
    tau = np.broadcast_to(np.asarray(tau, dtype=np.float64), (R,))
    a = np.zeros(R) if grad_logprob is None else np.asarray(grad_logprob, dtype=np.float64)
    b = np.zeros(R) if grad_entropy is None else np.asarray(grad_entropy, dtype=np.float64)
    targets = np.asarray(targets, dtype=np.int64)
    rows = np.arange(V) if weight_rows is None else np.asarray(weight_rows, dtype=np.int64)
    where = {int(v): i for i, v in enumerate(rows)}
    d_hidden = np.zeros((R, h64.shape[1]))
    d_weight = np.zeros((rows.size, h64.shape[1]))
    d_support = np.zeros((R, width))
    for t in range(R):
        pos = np.nonzero(ids[t] >= 0)[0]
        sup = ids[t, pos]
        if not _valid_tau(tau[t]) or (sup >= V).any() or len(np.unique(sup)) != len(sup):
            continue
        y = int(targets[t])
        if sup.size == 0 or not (0 <= y < V):
            continue
        w_sup = widen_bf16(w[sup])
        lse, lnp, hs = _log_softmax(h64[t] @ w_sup.T, tau[t])
        if not np.isfinite(lse):
            continue
        p = np.exp(lnp)
        plnp = np.where(p > 0.0, p * np.where(np.isfinite(lnp), lnp, 0.0), 0.0)
        hit = np.nonzero(sup == y)[0]
        a_t = a[t] if hit.size else 0.0
        dz = -a_t * p - b[t] * (plnp + p * hs)
        if hit.size:
            dz[hit[0]] += a_t
        dx = dz / tau[t]
        d_support[t, pos] = dx
        d_hidden[t] = dx @ w_sup
        for j, v in enumerate(sup):
            i = where.get(int(v))
            if i is not None:
                d_weight[i] += dx[j] * h64[t]
    return {"d_hidden": d_hidden, "d_weight": d_weight, "d_support": d_support}


def score_full_vjp(hidden, hidden_dtype: str, weight_bits, tau, targets, grad_logprob=None,
                   grad_entropy=None) -> dict:
    """Gradients of sum_t (a_t logprob_t + b_t H_t) of the fused projection
    ``x = bf16(hidden) W^T`` with respect to the hidden state and the weight.

    ``d_hidden = dX W`` and ``d_weight = dX^T bf16(hidden)`` with
    ``dX = logit_vjp(x, ...)``: the chain rule through the projection (the
    cast of an fp32 hidden state to bf16 passes its gradient through
    unchanged, as the cast's own derivative is the identity).  float64.
    """
    h = np.asarray(hidden)
    h64 = widen_bf16(round_f32_to_bf16(h)) if hidden_dtype == "f32" else widen_bf16(h)
    w64 = widen_bf16(np.asarray(weight_bits, dtype=np.uint16))
    x = h64 @ w64.T
    dx = logit_vjp(x, tau, targets, grad_logprob, grad_entropy)
    return {"d_hidden": dx @ w64, "d_weight": dx.T @ h64, "d_logits": dx}
