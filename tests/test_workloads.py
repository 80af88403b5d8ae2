"""The seeded input generators: shapes, determinism and the stated recipes (CPU only)."""

import numpy as np

import workloads


def test_tiny_recipe():
    a = workloads.make(1)
    b = workloads.make(1)
    assert workloads.digest(a) == workloads.digest(b)
    T, H, V = 64, 256, 4096
    assert a["hidden"].shape == (T, H) and a["hidden"].dtype == np.float32
    assert a["weight"].shape == (V, H) and a["weight"].dtype == np.uint16
    ids = a["support_ids"]
    assert ids.shape == (T, 8) and ids.dtype == np.int64
    widths = (ids >= 0).sum(1)
    assert list(widths[:9]) == list(range(9))
    nonempty = 0
    for t in range(T):
        w = widths[t]
        assert (ids[t, :w] >= 0).all() and (ids[t, w:] == -1).all()
        assert len(set(ids[t, :w])) == w
        if w:
            nonempty += 1
            assert (a["targets"][t] in ids[t, :w]) == (nonempty % 16 != 0)
    np.testing.assert_array_equal(a["fallback"], (widths == 0).astype(np.uint8))


def test_support_replay_recipe_small():
    c = workloads.make(3, T=500, H=64, V=1000)
    widths = (c["support_ids"] >= 0).sum(1)
    assert (widths == 0).sum() == 10 and (widths == 1).sum() == 25
    assert widths.max() <= 64
    for t in range(500):
        w = widths[t]
        if w:
            assert c["targets"][t] in c["support_ids"][t, :w]
            assert len(set(c["support_ids"][t, :w])) == w


def test_logits_full_recipe_small():
    c = workloads.make(2, T=8, V=3000)
    x = workloads.bf16_bits_to_f32(c["logits"])
    assert ((x > 5.0).sum(1) >= 5).all()  # five boosted ids per row
    assert ((c["temperature"] >= 0.6) & (c["temperature"] < 1.2)).all()
    assert ((c["targets"] >= 0) & (c["targets"] < 3000)).all()


def test_transforms_recipe_small():
    c = workloads.make(5, T=72, V=500)
    assert set(c["top_k"].tolist()) == {0, 20, 50}
    f32 = lambda vals: {float(np.float32(v)) for v in vals}  # noqa: E731
    assert set(c["top_p"].tolist()) == f32([1.0, 0.95, 0.8])
    assert set(c["min_p"].tolist()) == f32([0.0, 0.05])
    assert set(c["temperature"].tolist()) == f32([0.7, 1.0])
    combos = {(int(c["top_k"][t]), float(c["top_p"][t]), float(c["min_p"][t]), float(c["temperature"][t]))
              for t in range(36)}
    assert len(combos) == 36
    assert c["draft"].shape == c["logits"].shape
    d = workloads.bf16_bits_to_f32(c["draft"]) - workloads.bf16_bits_to_f32(c["logits"])
    assert 0.4 < float(d.std()) < 0.6


def test_bf16_storage_rounding():
    import torch
    rng = np.random.default_rng(0)
    x = rng.normal(0, 1, 10000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(workloads.to_bf16_bits(x), ref)
