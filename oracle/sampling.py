"""fp64 reference of the seeded Gumbel draw that ends the transform program
(test infrastructure only).

xorl issue #71, section 3, names the program
``temperature -> stable token-id top-k -> inclusive top-p -> min-p against
the original row max -> seeded Gumbel``; the pages name the last stage and
define neither its generator nor how its numbers are laid out.  The reading
taken here (the GPU kernel implements the same generator from the same
published definition; the two share no code):

* Generator: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC 2011): a counter of four 32-bit words is
  sent through ten rounds keyed by two 32-bit words.  Each round multiplies
  words 0 and 2 by 0xD2511F53 and 0xCD9E8D57 into 64-bit products and returns
  (hi(c2 * M1) ^ c1 ^ k0, lo(c2 * M1), hi(c0 * M0) ^ c3 ^ k1, lo(c0 * M0));
  the key grows by (0x9E3779B9, 0xBB67AE85) after every round.
* Layout: for row t, token v, seed s and offset o (both 64-bit), the key is
  (s mod 2^32, s div 2^32), the counter (v div 4, t, o mod 2^32, o div 2^32),
  and word (v mod 4) of the output is token v's 32-bit number r.
* Uniform: u = (r + 1/2) / 2^32, strictly inside (0, 1).
* Draw: the token of the transformed support S with the largest
  (x_v - x_max) / tau + G_v, G_v = -ln(-ln u_v) (the Gumbel-max draw from
  softmax over S; the shift by the row maximum changes no decision and keeps
  the sum exact at any magnitude); on equal scores the lower token id.
"""

from __future__ import annotations

import numpy as np

from .scoring import ST_BAD_INPUT, score_transforms

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key) -> np.ndarray:
    """Philox4x32-10 of counters ``[..., 4]`` under keys ``[..., 2]`` (uint32),
    the rounds written out as the published definition gives them."""
    c = np.asarray(counter, dtype=np.uint64) & _MASK32
    k = np.asarray(key, dtype=np.uint64) & _MASK32
    c0, c1, c2, c3 = (c[..., i] for i in range(4))
    k0, k1 = k[..., 0], k[..., 1]
    for _ in range(10):
        p0 = np.uint64(PHILOX_M0) * c0  # < 2^64: exact in uint64
        p1 = np.uint64(PHILOX_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
        k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def token_uniforms(row: int, V: int, seed: int, offset: int = 0) -> np.ndarray:
    """u_v for every token v of row ``row`` (float64, strictly inside (0, 1))."""
    n = (V + 3) // 4
    ctr = np.zeros((n, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(n, dtype=np.uint64)
    ctr[:, 1] = np.uint64(row & 0xFFFFFFFF)
    ctr[:, 2] = np.uint64(offset & 0xFFFFFFFF)
    ctr[:, 3] = np.uint64((offset >> 32) & 0xFFFFFFFF)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    r = philox4x32_10(ctr, np.broadcast_to(key, (n, 2))).reshape(-1)[:V]
    return (r.astype(np.float64) + 0.5) * 2.0 ** -32


def gumbel_draw(x_row, tau: float, support, row: int, seed: int, offset: int = 0) -> int:
    """The seeded Gumbel-max token of one row over the ids ``support``."""
    x_row = np.asarray(x_row, dtype=np.float64)
    sup = np.asarray(support, dtype=np.int64)
    u = token_uniforms(row, x_row.size, seed, offset)[sup]
    g = -np.log(-np.log(u))
    score = (x_row[sup] - x_row.max()) / tau + g
    best = score.max()
    return int(sup[score == best].min())


def sample_transforms(x, tau, top_k, top_p, min_p, seed: int, offset: int = 0, rows=None) -> dict:
    """Seeded draws from the transformed supports of rows ``rows`` of x.

    The support of each row is the transform program's (``score_transforms``),
    then the Gumbel-max draw as in the module notes.  ``rows`` gives the global
    row indices of x's rows (the counter's row word; default 0 .. R-1).
    Returns ``sampled`` (int64, -1 on a BAD_INPUT row), ``status``, and per
    row the draw's ``margin``: the gap between the best and second-best score
    (inf for a singleton support), which tells how close a draw was to another
    token."""
    x = np.asarray(x, dtype=np.float64)
    R, V = x.shape
    rows = np.arange(R) if rows is None else np.asarray(rows)
    tau = np.broadcast_to(np.asarray(tau, dtype=np.float64), (R,))
    desc = score_transforms(x, tau, top_k, top_p, min_p, np.zeros(R, dtype=np.int64), cap=0)
    sampled = np.full(R, -1, dtype=np.int64)
    margin = np.full(R, np.nan)
    for t in range(R):
        if desc["status"][t] & ST_BAD_INPUT:
            continue
        L = int(desc["support_len"][t])
        order = np.lexsort((np.arange(V), -x[t]))
        sup = order[:L]
        sampled[t] = gumbel_draw(x[t], tau[t], sup, int(rows[t]), seed, offset)
        u = token_uniforms(int(rows[t]), V, seed, offset)[sup]
        sc = np.sort((x[t, sup] - x[t].max()) / tau[t] - np.log(-np.log(u)))
        margin[t] = np.inf if L == 1 else sc[-1] - sc[-2]
    return {"sampled": sampled, "status": desc["status"] & ST_BAD_INPUT, "support_len": desc["support_len"],
            "margin": margin}
