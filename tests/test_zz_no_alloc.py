"""GPU: vs_score_full_noalloc (no workspace; the library's per-GPU scratch
array) against vs_score_full on the same inputs, through the C ABI: two calls
in a row, the second with a smaller input, each bit-identical to the
workspace entry point (the same kernels), and within the float tolerance of
the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_common import assert_close, bf16_tensor, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsa():
    import logprob_entropy_sampling_amd as m
    m.lib()
    return m


def _case(rng, T, H, V, hidden_dtype):
    h = rng.standard_normal((T, H)).astype(np.float32)
    wb = workloads.to_bf16_bits((rng.standard_normal((V, H)) * 0.05).astype(np.float32))
    tau = rng.uniform(0.5, 1.5, T).astype(np.float32)
    y = rng.integers(0, V, T).astype(np.int64)
    if hidden_dtype == "bf16":
        hb = workloads.to_bf16_bits(h)
        return bf16_tensor(hb), hb, "bf16", wb, tau, y
    return to_dev(h), h, "f32", wb, tau, y


def test_noalloc_matches_workspace_entry_point(vsa):
    rng = np.random.default_rng(2024)
    # first call: 1536 rows, V = 60,000 (1.4 MB of partials, fp32 hidden adds its
    # bf16 copy); second call: smaller in every dimension
    for T, H, V, hdt in ((1536, 384, 60000, "f32"), (300, 128, 5003, "bf16")):
        say(f"noalloc: T={T} H={H} V={V} hidden {hdt}")
        hid, h_np, h_kind, wb, tau, y = _case(rng, T, H, V, hdt)
        w = bf16_tensor(wb)
        td, yd = to_dev(tau), to_dev(y)
        out = {k: torch.full((T,), -7.0, dtype=torch.float32, device=hid.device) for k in ("lse", "logprob", "entropy")}
        out["status"] = torch.full((T,), 0xEE, dtype=torch.uint8, device=hid.device)
        got = vsa.score_full_noalloc(yd, hidden=hid, weight=w, temperature=td, vocab_chunk=8192, out=out)
        ref = vsa.score_full(yd, hidden=hid, weight=w, temperature=td, vocab_chunk=8192)
        torch.cuda.synchronize()
        for k in ("lse", "logprob", "entropy", "status"):
            assert torch.equal(got[k], ref[k]), (T, k)
        x = oracle.logits_from_hidden(h_np, h_kind, wb)
        o = oracle.score_full(x, tau, y)
        assert np.array_equal(got["status"].cpu().numpy(), o["status"])
        for k in ("lse", "logprob", "entropy"):
            assert_close(k, got[k].cpu().numpy(), o[k])


def test_noalloc_logits_source_and_limit(vsa):
    say("noalloc: logits source (no scratch), and a request beyond the scratch array")
    c = workloads.make(2, T=6)
    lg = bf16_tensor(c["logits"])
    y, tau = to_dev(c["targets"]), to_dev(c["temperature"])
    a = vsa.score_full_noalloc(y, logits=lg, temperature=tau)
    b = vsa.score_full(y, logits=lg, temperature=tau)
    assert all(torch.equal(a[k], b[k]) for k in ("lse", "logprob", "entropy", "status"))
    assert vsa.noalloc_scratch_bytes() == 64 << 20
    # 2048 rows over V = 151,936 with an fp32 hidden state of H = 8192 need 19.5 MB of partials plus 33.5 MB
    # of bf16 copy: fits; T = 4096 would need 106 MB: VS_E_SCRATCH, nothing enqueued
    hid = torch.zeros((4096, 8192), dtype=torch.float32, device=lg.device)
    w = torch.zeros((151936, 8192), dtype=torch.bfloat16, device=lg.device)
    with pytest.raises(vsa.VsError) as e:
        vsa.score_full_noalloc(torch.zeros(4096, dtype=torch.int64, device=lg.device), hidden=hid, weight=w)
    assert e.value.code == 9
