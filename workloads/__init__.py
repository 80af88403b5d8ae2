"""Seeded synthetic inputs for the six scoring workloads.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests; it holds none of the scoring arithmetic (no log-sum-exp, no entropy,
no support selection).  Random numbers a method would draw (the sampled
target ids) are drawn here and passed in as inputs.

Each workload draws from ``numpy.random.Generator(PCG64(SeedSequence(seed)))``
with ``seed = 1000 + i`` (i = 1..6) and child streams spawned in a fixed order
(hidden, weight, logits, ids, targets, params, noise), so a workload and its
sizes determine every byte.  float32 -> bf16 uses round-to-nearest-even.

Workloads (sizes overridable for small parity cases):

1. ``tiny``: fused scoring, T=64, H=256, V=4096, fp32 hidden ~N(0,1), bf16
   W ~N(0, 0.05), uniform targets, tau=1; recorded support width 8 (rows 0..8
   have widths 0..8, the rest uniform on 0..8; distinct ids, -1 padded at the
   end; the target is in the support except on every 16th non-empty row;
   empty rows flagged synthetic-EOS).
2. ``logits_full``: T=512, V=151,936 bf16 logits ~N(0,2) with +8 added to 5
   distinct random ids per row, per-row tau ~U[0.6, 1.2), targets drawn by
   Gumbel-max from softmax(x / tau).
3. ``support_replay``: T=2048, H=7168, V=129,280, bf16 hidden ~N(0,1), bf16
   W ~N(0, 0.02), support ids [T, 64] (2% width 0, 5% width 1, the rest
   uniform on 2..64), distinct ids, target uniform among the row's ids, tau=1.
4. ``fused_full``: T=4096, H=4096, V=151,936, bf16 hidden ~N(0,1), bf16 W
   ~N(0, 0.02), uniform targets, tau=1, vocab chunk 8192.
5. ``transforms_l1``: T=2048, V=151,936 bf16 logits ~N(0,2); row t takes
   combination t mod 36 of top_k {0,20,50} x top_p {1.0,0.95,0.8} x min_p
   {0,0.05} x tau {0.7,1.0}; a uniform ``u[t]`` for drawing the in-support
   target by inverse CDF (done by the caller, who knows the support); draft
   logits = bf16(float32(x) + 0.5 N(0,1)).
6. ``transforms_hidden``: the transform program of workload 5 on a fused
   source, T=2048, H=4096, V=151,936, with hidden and W on grids that make
   every fp32 sum of the projection exact: hidden = k/4 and W = j/128 with
   k, j = round(4 N(0,1)) clipped to [-16, 16] (so x ~ N(0, 2), like workload
   5's logits; every product is a multiple of 2^-9 of magnitude <= 1/2, so
   any partial sum over H <= 65536 terms fits 24 bits); targets are the
   plain row argmax of the projected bf16 logits (computed by the caller).
"""

from __future__ import annotations

import hashlib

import numpy as np

NAMES = {1: "tiny", 2: "logits_full", 3: "support_replay", 4: "fused_full", 5: "transforms_l1",
         6: "transforms_hidden"}

FULL_SIZES = {
    1: dict(T=64, H=256, V=4096, W=8),
    2: dict(T=512, V=151936),
    3: dict(T=2048, H=7168, V=129280, W=64),
    4: dict(T=4096, H=4096, V=151936),
    5: dict(T=2048, V=151936),
    6: dict(T=2048, H=4096, V=151936),
}

_STREAMS = ("hidden", "weight", "logits", "ids", "targets", "params", "noise")


def _rngs(i: int) -> dict:
    ss = np.random.SeedSequence(1000 + i)
    return {name: np.random.Generator(np.random.PCG64(child))
            for name, child in zip(_STREAMS, ss.spawn(len(_STREAMS)))}


def to_bf16_bits(x) -> np.ndarray:
    """float32 array -> uint16 bf16 patterns, round-to-nearest-even (storage format)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u.astype(np.uint64) + bias) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng, shape, std) -> np.ndarray:
    """bf16(std * N(0,1)), generated in row blocks to bound the float32 temporary."""
    out = np.empty(shape, dtype=np.uint16)
    rows = shape[0]
    step = max(1, (1 << 26) // max(1, int(np.prod(shape[1:]))))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        blk = rng.standard_normal((r1 - r0,) + tuple(shape[1:]), dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        out[r0:r1] = to_bf16_bits(blk)
    return out


def _grid_bf16(rng, shape, unit) -> np.ndarray:
    """bf16(unit * k), k = round(4 N(0,1)) clipped to [-16, 16]: exact in bf16."""
    out = np.empty(shape, dtype=np.uint16)
    rows = shape[0]
    step = max(1, (1 << 26) // max(1, int(np.prod(shape[1:]))))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        k = np.rint(rng.standard_normal((r1 - r0,) + tuple(shape[1:]), dtype=np.float32) * np.float32(4.0))
        np.clip(k, -16, 16, out=k)
        out[r0:r1] = to_bf16_bits(k * np.float32(unit))
    return out


def _transform_params(T: int) -> dict:
    """Row t takes combination t mod 36 of top_k {0,20,50} x top_p {1,0.95,0.8}
    x min_p {0,0.05} x tau {0.7,1}."""
    combo = np.arange(T) % 36
    ks = np.array([0, 20, 50], dtype=np.int32)
    ps = np.array([1.0, 0.95, 0.8], dtype=np.float32)
    ms = np.array([0.0, 0.05], dtype=np.float32)
    ts = np.array([0.7, 1.0], dtype=np.float32)
    return {"top_k": ks[combo // 12], "top_p": ps[(combo // 4) % 3], "min_p": ms[(combo // 2) % 2],
            "temperature": ts[combo % 2]}


def _distinct_ids(rng, V: int, n: int, exclude: int = -1) -> np.ndarray:
    """n distinct ids uniform in [0, V), none equal to ``exclude``."""
    got = []
    seen = set()
    while len(got) < n:
        for v in rng.integers(0, V, size=2 * n + 4).tolist():
            if v != exclude and v not in seen:
                seen.add(v)
                got.append(v)
                if len(got) == n:
                    break
    return np.asarray(got, dtype=np.int64)


def _gumbel_targets(rng, logits_bits, tau) -> np.ndarray:
    """Gumbel-max draw of one id per row from softmax(x / tau) (float64)."""
    T, V = logits_bits.shape
    y = np.empty(T, dtype=np.int64)
    for t in range(T):
        u = rng.random(V)
        g = -np.log(-np.log(np.maximum(u, 1e-300)))
        y[t] = int(np.argmax(bf16_bits_to_f32(logits_bits[t]).astype(np.float64) / float(tau[t]) + g))
    return y


def make(i: int, **sizes) -> dict:
    """Inputs of workload ``i`` (1..5); keyword sizes override the full ones."""
    cfg = dict(FULL_SIZES[i])
    cfg.update(sizes)
    r = _rngs(i)
    out = {"workload": NAMES[i], "index": i, **cfg}
    T, V = cfg["T"], cfg["V"]

    if i == 1:
        H, Wd = cfg["H"], cfg["W"]
        out["kind"] = "hidden_weight"
        out["hidden"] = r["hidden"].standard_normal((T, H), dtype=np.float32)
        out["hidden_dtype"] = "f32"
        out["weight"] = _normal_bf16(r["weight"], (V, H), 0.05)
        out["targets"] = r["targets"].integers(0, V, size=T).astype(np.int64)
        out["temperature"] = np.ones(T, dtype=np.float32)
        widths = r["ids"].integers(0, Wd + 1, size=T)
        widths[: min(T, Wd + 1)] = np.arange(min(T, Wd + 1))
        ids = np.full((T, Wd), -1, dtype=np.int64)
        nonempty = 0
        for t in range(T):
            w = int(widths[t])
            if w == 0:
                continue
            nonempty += 1
            y = int(out["targets"][t])
            if nonempty % 16 == 0:  # every 16th non-empty row leaves the target out
                row = _distinct_ids(r["ids"], V, w, exclude=y)
            else:
                row = _distinct_ids(r["ids"], V, w - 1, exclude=y)
                pos = int(r["ids"].integers(0, w))
                row = np.insert(row, pos, y)
            ids[t, :w] = row
        out["support_ids"] = ids
        out["fallback"] = (widths == 0).astype(np.uint8)
        out["vocab_chunk"] = 8192

    elif i == 2:
        out["kind"] = "logits"
        x = r["logits"].standard_normal((T, V), dtype=np.float32)
        x *= np.float32(2.0)
        for t in range(T):
            x[t, _distinct_ids(r["ids"], V, 5)] += np.float32(8.0)
        out["logits"] = to_bf16_bits(x)
        del x
        out["logits_dtype"] = "bf16"
        out["temperature"] = r["params"].uniform(0.6, 1.2, size=T).astype(np.float32)
        out["targets"] = _gumbel_targets(r["targets"], out["logits"], out["temperature"])
        out["vocab_chunk"] = 8192

    elif i == 3:
        H, Wd = cfg["H"], cfg["W"]
        out["kind"] = "hidden_weight"
        out["hidden"] = _normal_bf16(r["hidden"], (T, H), 1.0)
        out["hidden_dtype"] = "bf16"
        out["weight"] = _normal_bf16(r["weight"], (V, H), 0.02)
        n_empty = int(round(0.02 * T))
        n_single = int(round(0.05 * T))
        widths = r["ids"].integers(2, Wd + 1, size=T)
        perm = r["ids"].permutation(T)
        widths[perm[:n_empty]] = 0
        widths[perm[n_empty:n_empty + n_single]] = 1
        ids = np.full((T, Wd), -1, dtype=np.int64)
        targets = np.empty(T, dtype=np.int64)
        for t in range(T):
            w = int(widths[t])
            if w == 0:
                targets[t] = int(r["targets"].integers(0, V))
                continue
            row = _distinct_ids(r["ids"], V, w)
            ids[t, :w] = row
            targets[t] = int(row[int(r["targets"].integers(0, w))])
        out["support_ids"] = ids
        out["targets"] = targets
        out["fallback"] = None
        out["temperature"] = np.ones(T, dtype=np.float32)

    elif i == 4:
        H = cfg["H"]
        out["kind"] = "hidden_weight"
        out["hidden"] = _normal_bf16(r["hidden"], (T, H), 1.0)
        out["hidden_dtype"] = "bf16"
        out["weight"] = _normal_bf16(r["weight"], (V, H), 0.02)
        out["targets"] = r["targets"].integers(0, V, size=T).astype(np.int64)
        out["temperature"] = np.ones(T, dtype=np.float32)
        out["vocab_chunk"] = 8192

    elif i == 5:
        out["kind"] = "logits"
        out["logits"] = _normal_bf16(r["logits"], (T, V), 2.0)
        out["logits_dtype"] = "bf16"
        out.update(_transform_params(T))
        out["u"] = r["targets"].random(T)
        # plain row argmax (lowest id among equal maxima): always inside any
        # top-k/top-p/min-p support; used where no support-aware draw is made
        out["targets"] = np.argmax(bf16_bits_to_f32(out["logits"]), axis=1).astype(np.int64)
        draft = np.empty((T, V), dtype=np.uint16)
        step = max(1, (1 << 26) // V)
        for r0 in range(0, T, step):
            r1 = min(T, r0 + step)
            noise = r["noise"].standard_normal((r1 - r0, V), dtype=np.float32)
            noise *= np.float32(0.5)
            noise += bf16_bits_to_f32(out["logits"][r0:r1])
            draft[r0:r1] = to_bf16_bits(noise)
        out["draft"] = draft
        out["support_cap"] = 64

    elif i == 6:
        H = cfg["H"]
        out["kind"] = "hidden_weight"
        out["hidden"] = _grid_bf16(r["hidden"], (T, H), 0.25)
        out["hidden_dtype"] = "bf16"
        out["weight"] = _grid_bf16(r["weight"], (V, H), 1.0 / 128)
        out.update(_transform_params(T))
        out["support_cap"] = 64
    return out


def digest(cfg: dict) -> dict:
    """SHA-256 (first 16 hex digits) of every array input of a workload."""
    out = {}
    for k, v in sorted(cfg.items()):
        if isinstance(v, np.ndarray):
            out[k] = hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
    return out
