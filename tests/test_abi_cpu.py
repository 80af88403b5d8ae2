"""The C ABI without a GPU: the library loads, exports every declared symbol,
the ctypes struct matches the C layout, and host-side validation rejects bad
arguments before anything is enqueued (fake device pointers are never read)."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vocabscore.h")


@pytest.fixture(scope="module")
def lib():
    from logprob_entropy_sampling_amd import _capi
    if not os.path.exists(_capi.LIB_PATH):
        from logprob_entropy_sampling_amd import build
        build.build()
    return _capi.load()


def test_every_declared_symbol_is_exported(lib):
    text = open(HEADER).read()
    names = sorted(set(re.findall(r"\b(vs_[a-z0-9_]+)\s*\(", text)))
    assert {"vs_score_full", "vs_score_support_ids", "vs_score_transforms", "vs_l1_distance",
            "vs_workspace_size", "vs_status_string", "vs_version"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], stdout=subprocess.PIPE, text=True).stdout
    exported = set(re.findall(r"\bT (vs_[a-z0-9_]+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_struct_layout_matches_c(lib):
    from logprob_entropy_sampling_amd import _capi
    prog = r'''
#include <stdio.h>
#include <stddef.h>
#include "vocabscore.h"
int main(void) {
  printf("%zu", sizeof(vs_source));
#define F(x) printf(" %zu", offsetof(vs_source, x));
  F(kind) F(logits) F(logits_dtype) F(ld_logits) F(hidden) F(hidden_dtype) F(ld_hidden) F(weight)
  F(weight_dtype) F(ld_weight) F(T) F(H) F(V) F(temperature) F(temperature_scalar)
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "p.c")
        exe = os.path.join(d, "p")
        open(src, "w").write(prog)
        subprocess.check_call(["gcc", "-I", os.path.dirname(HEADER), src, "-o", exe])
        vals = [int(v) for v in subprocess.check_output([exe]).split()]
    S = _capi.VsSource
    ours = [ctypes.sizeof(S)] + [getattr(S, f).offset for f, _ in S._fields_]
    assert vals == ours


def test_status_strings_and_version(lib):
    for code in range(10):
        s = lib.vs_status_string(code).decode()
        assert s and s != "unknown status code"
    assert lib.vs_status_string(99).decode() == "unknown status code"
    assert lib.vs_version() >= 10000


def test_sweep_timer_error_codes_without_a_bracket(lib):
    # no HIP call is made on these paths: disabling, and reading before any bracket was recorded
    assert lib.vs_sweep_timer(0) == 0
    assert lib.vs_sweep_timer_ms(None) == 1  # VS_E_NULL
    ms = ctypes.c_float(-1.0)
    assert lib.vs_sweep_timer_ms(ctypes.byref(ms)) == 5  # VS_E_PARAM: nothing recorded
    assert ms.value == -1.0


FAKE = 0x10000000  # never dereferenced: every call below fails validation first


def _src(**kw):
    from logprob_entropy_sampling_amd import _capi
    s = _capi.VsSource()
    s.kind = kw.get("kind", _capi.VS_SRC_LOGITS)
    s.logits = kw.get("logits", FAKE)
    s.logits_dtype = kw.get("logits_dtype", _capi.VS_BF16)
    s.ld_logits = kw.get("ld_logits", 1000)
    s.hidden = kw.get("hidden", FAKE)
    s.hidden_dtype = kw.get("hidden_dtype", _capi.VS_BF16)
    s.ld_hidden = kw.get("ld_hidden", 64)
    s.weight = kw.get("weight", FAKE)
    s.weight_dtype = kw.get("weight_dtype", _capi.VS_BF16)
    s.ld_weight = kw.get("ld_weight", 64)
    s.T = kw.get("T", 10)
    s.H = kw.get("H", 64)
    s.V = kw.get("V", 1000)
    s.temperature = kw.get("temperature", None)
    s.temperature_scalar = kw.get("temperature_scalar", 1.0)
    return s


def _full(lib, src, targets=FAKE, chunk=8192, logprob=FAKE, ws=FAKE, nws=1 << 40):
    return lib.vs_score_full(ctypes.byref(src) if src is not None else None, targets, chunk, FAKE, logprob, FAKE,
                             FAKE, ws, nws, None)


def test_score_full_validation(lib):
    from logprob_entropy_sampling_amd import _capi as C
    assert _full(lib, None) == C.VS_E_NULL
    assert _full(lib, _src(), targets=None) == C.VS_E_NULL
    assert _full(lib, _src(), logprob=None) == C.VS_E_NULL
    assert _full(lib, _src(logits=None)) == C.VS_E_NULL
    assert _full(lib, _src(T=0)) == C.VS_E_SHAPE
    assert _full(lib, _src(V=0)) == C.VS_E_SHAPE
    assert _full(lib, _src(V=1 << 31, ld_logits=1 << 31)) == C.VS_E_SHAPE
    assert _full(lib, _src(ld_logits=999)) == C.VS_E_SHAPE
    assert _full(lib, _src(logits_dtype=7)) == C.VS_E_DTYPE
    assert _full(lib, _src(logits=FAKE + 1)) == C.VS_E_ALIGN
    assert _full(lib, _src(logits=FAKE + 2, logits_dtype=C.VS_F32)) == C.VS_E_ALIGN
    assert _full(lib, _src(kind=5)) == C.VS_E_PARAM
    assert _full(lib, _src(temperature_scalar=0.0)) == C.VS_E_PARAM
    assert _full(lib, _src(temperature_scalar=float("nan"))) == C.VS_E_PARAM
    assert _full(lib, _src(), chunk=0) == C.VS_E_PARAM
    hw = dict(kind=C.VS_SRC_HIDDEN_WEIGHT)  # (a logits source needs no workspace at all)
    assert _full(lib, _src(**hw), ws=None) == C.VS_E_WORKSPACE
    assert _full(lib, _src(**hw), ws=FAKE + 16) == C.VS_E_WORKSPACE
    need = lib.vs_workspace_size(C.VS_OP_SCORE_FULL, ctypes.byref(_src(**hw)), 0)
    assert need > 0
    assert _full(lib, _src(**hw), nws=need - 1) == C.VS_E_WORKSPACE
    assert _full(lib, _src(hidden=None, **hw)) == C.VS_E_NULL
    assert _full(lib, _src(weight_dtype=C.VS_F32, **hw)) == C.VS_E_DTYPE
    assert _full(lib, _src(H=60, ld_hidden=64, ld_weight=64, **hw)) == C.VS_E_SHAPE
    assert _full(lib, _src(ld_hidden=32, **hw)) == C.VS_E_SHAPE
    assert _full(lib, _src(ld_weight=68, **hw)) == C.VS_E_ALIGN
    assert _full(lib, _src(hidden=FAKE + 8, **hw)) == C.VS_E_ALIGN
    assert _full(lib, _src(weight=FAKE + 2, **hw)) == C.VS_E_ALIGN


def test_support_validation(lib):
    from logprob_entropy_sampling_amd import _capi as C

    def call(src, ids=FAKE, width=8, ld=8, chunk=8192, ws=FAKE, nws=1 << 40):
        return lib.vs_score_support_ids(ctypes.byref(src), ids, width, ld, FAKE, None, chunk, FAKE, FAKE, FAKE, ws,
                                        nws, None)
    assert call(_src(), width=-1) == C.VS_E_SHAPE
    assert call(_src(), width=1025, ld=1025) == C.VS_E_SHAPE
    assert call(_src(), width=8, ld=7) == C.VS_E_SHAPE
    assert call(_src(), ids=None) == C.VS_E_NULL
    assert call(_src(), chunk=0) == C.VS_E_PARAM
    assert call(_src(kind=C.VS_SRC_HIDDEN_WEIGHT, H=16392, ld_hidden=16392, ld_weight=16392)) == C.VS_E_UNSUPPORTED
    assert call(_src(), nws=0) == C.VS_E_WORKSPACE


def test_transforms_validation(lib):
    from logprob_entropy_sampling_amd import _capi as C

    def call(src, topk=FAKE, cap=0, ws=None, nws=0):
        return lib.vs_score_transforms(ctypes.byref(src), topk, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, cap, FAKE, ws, nws, None)
    assert call(_src(logits_dtype=C.VS_F32)) == C.VS_E_UNSUPPORTED
    assert call(_src(), topk=None) == C.VS_E_NULL
    assert call(_src(), cap=-1) == C.VS_E_PARAM
    assert call(_src(), cap=4097, ws=FAKE, nws=1 << 40) == C.VS_E_UNSUPPORTED
    # a hidden/weight source: its bf16 logits are written block by block into the workspace
    hw = dict(kind=C.VS_SRC_HIDDEN_WEIGHT, H=4096, V=151936, ld_hidden=4096, ld_weight=4096)
    assert call(_src(T=100, **hw)) == C.VS_E_WORKSPACE
    assert call(_src(T=100, hidden=FAKE + 8, **hw)) == C.VS_E_ALIGN
    small = lib.vs_workspace_size(C.VS_OP_SCORE_TRANSFORMS, ctypes.byref(_src(T=100, **hw)), 0)
    block = lib.vs_workspace_size(C.VS_OP_SCORE_TRANSFORMS, ctypes.byref(_src(T=2048, **hw)), 0)
    big = lib.vs_workspace_size(C.VS_OP_SCORE_TRANSFORMS, ctypes.byref(_src(T=8192, **hw)), 0)
    logits_only = lib.vs_workspace_size(C.VS_OP_SCORE_TRANSFORMS,
                                        ctypes.byref(_src(T=100, V=151936, ld_logits=151936)), 0)
    assert small >= 100 * 151936 * 2 + logits_only
    assert big == block >= 2048 * 151936 * 2  # blocks of at most 2048 rows
    f32 = lib.vs_workspace_size(C.VS_OP_SCORE_TRANSFORMS,
                                ctypes.byref(_src(T=8192, hidden_dtype=C.VS_F32, **hw)), 0)
    assert f32 >= big + 8192 * 4096 * 2  # and the bf16 copy of an fp32 hidden state
    assert call(_src(T=100, **hw), ws=FAKE, nws=small - 1) == C.VS_E_WORKSPACE


def test_l1_validation(lib):
    from logprob_entropy_sampling_amd import _capi as C

    def call(t=FAKE, d=FAKE, dt=C.VS_BF16, T=4, V=100, lt=100, ldd=100, l1=FAKE):
        return lib.vs_l1_distance(t, d, dt, T, V, lt, ldd, l1, FAKE, FAKE, 1 << 40, None)
    assert call(t=None) == C.VS_E_NULL
    assert call(l1=None) == C.VS_E_NULL
    assert call(dt=3) == C.VS_E_DTYPE
    assert call(T=0) == C.VS_E_SHAPE
    assert call(ldd=99) == C.VS_E_SHAPE
    assert call(d=FAKE + 1) == C.VS_E_ALIGN


def test_workspace_sizes_scale(lib):
    from logprob_entropy_sampling_amd import _capi as C
    # a logits source is scored one row per workgroup with no partials
    assert lib.vs_workspace_size(C.VS_OP_SCORE_FULL, ctypes.byref(_src(T=100)), 0) == 0
    a = lib.vs_workspace_size(C.VS_OP_SCORE_SUPPORT, ctypes.byref(_src(T=100)), 8)
    b = lib.vs_workspace_size(C.VS_OP_SCORE_SUPPORT, ctypes.byref(_src(T=200)), 8)
    assert b > a > 0  # the fallback row list
    hw = _src(kind=C.VS_SRC_HIDDEN_WEIGHT, T=4096, H=4096, V=151936, ld_hidden=4096, ld_weight=4096)
    n = lib.vs_workspace_size(C.VS_OP_SCORE_FULL, ctypes.byref(hw), 0)
    assert n >= 4096 * 594 * 16  # one 16-byte partial per (row, 256-wide vocabulary tile)
    assert lib.vs_workspace_size(C.VS_OP_SCORE_FULL, None, 0) == 0


def test_noalloc_rejects_before_any_device_call(lib):
    from logprob_entropy_sampling_amd import _capi as C
    assert lib.vs_noalloc_scratch_bytes() == 64 << 20

    def call(src, targets=FAKE, logprob=FAKE):
        return lib.vs_score_full_noalloc(ctypes.byref(src) if src is not None else None, targets, 8192, FAKE,
                                         logprob, FAKE, FAKE, None)
    assert call(None) == C.VS_E_NULL
    assert call(_src(), targets=None) == C.VS_E_NULL  # a logits source needs no scratch
    assert call(_src(T=0)) == C.VS_E_SHAPE
    # the fused source's partials of 32768 rows over 151,936 ids (311 MB) exceed the 64 MiB array
    big = _src(kind=C.VS_SRC_HIDDEN_WEIGHT, T=32768, H=4096, V=151936, ld_hidden=4096, ld_weight=4096)
    assert lib.vs_workspace_size(C.VS_OP_SCORE_FULL, ctypes.byref(big), 0) > 64 << 20
    assert call(big) == C.VS_E_SCRATCH
    assert "scratch" in lib.vs_status_string(C.VS_E_SCRATCH).decode()


def test_sample_validation(lib):
    from logprob_entropy_sampling_amd import _capi as C

    def call(src, topk=FAKE, out=FAKE, ws=FAKE, nws=1 << 40):
        return lib.vs_sample_transforms(ctypes.byref(src), topk, FAKE, FAKE, 1, 0, out, None, None, None, None, ws,
                                        nws, None)
    assert call(_src(kind=C.VS_SRC_HIDDEN_WEIGHT), ws=None) == C.VS_E_WORKSPACE
    assert call(_src(logits_dtype=C.VS_F32)) == C.VS_E_UNSUPPORTED
    assert call(_src(), topk=None) == C.VS_E_NULL
    assert call(_src(), out=None) == C.VS_E_NULL
    assert call(_src(), ws=None) == C.VS_E_WORKSPACE
    need = lib.vs_workspace_size(C.VS_OP_SAMPLE_TRANSFORMS, ctypes.byref(_src(T=100, V=151936, ld_logits=151936)), 0)
    t = lib.vs_workspace_size(C.VS_OP_SCORE_TRANSFORMS, ctypes.byref(_src(T=100, V=151936, ld_logits=151936)), 0)
    assert need > t > 0
    assert call(_src(T=100, V=151936, ld_logits=151936), nws=need - 1) == C.VS_E_WORKSPACE


def test_support_backward_validation(lib):
    from logprob_entropy_sampling_amd import _capi as C

    def call(src, ids=FAKE, width=8, ld=8, gh=FAKE, gw=FAKE, ws=FAKE, nws=1 << 40):
        return lib.vs_score_support_backward(ctypes.byref(src), ids, width, ld, FAKE, FAKE, FAKE, gh, 64, gw, 64, ws,
                                             nws, None)
    hw = dict(kind=C.VS_SRC_HIDDEN_WEIGHT)
    assert call(_src()) == C.VS_E_UNSUPPORTED  # a logits source
    assert call(_src(**hw), ids=None) == C.VS_E_NULL
    assert call(_src(**hw), gh=None, gw=None) == C.VS_E_NULL
    assert call(_src(**hw), width=1025, ld=1025) == C.VS_E_SHAPE
    assert call(_src(**hw), width=8, ld=7) == C.VS_E_SHAPE
    assert call(_src(**hw), gh=FAKE + 2) == C.VS_E_ALIGN
    assert call(_src(H=16392, ld_hidden=16392, ld_weight=16392, **hw)) == C.VS_E_UNSUPPORTED
    assert call(_src(**hw), ws=None) == C.VS_E_WORKSPACE
    need = lib.vs_workspace_size(C.VS_OP_SCORE_SUPPORT_BACKWARD, ctypes.byref(_src(T=2048, V=129280, **hw)), 64)
    # dX and the pair list per (row, id), and three per-id arrays
    assert need >= 2048 * 64 * 8 + 3 * 129280 * 4
    assert call(_src(T=2048, V=129280, **hw), width=64, ld=64, nws=need - 1) == C.VS_E_WORKSPACE
    f32 = lib.vs_workspace_size(C.VS_OP_SCORE_SUPPORT_BACKWARD,
                                ctypes.byref(_src(T=2048, V=129280, hidden_dtype=C.VS_F32, **hw)), 64)
    assert f32 >= need + 2048 * 64 * 2


def test_l1_loss_validation(lib):
    from logprob_entropy_sampling_amd import _capi as C

    def call(t=FAKE, d=FAKE, dt=C.VS_BF16, T=4, V=100, l1=FAKE, loss=FAKE, grad=FAKE, gdt=C.VS_F32, ldg=100,
             scale=1.0, ws=FAKE, nws=1 << 40):
        return lib.vs_l1_loss(t, d, dt, T, V, V, V, None, scale, l1, None, loss, grad, gdt, ldg, ws, nws, None)
    assert call(loss=None) == C.VS_E_NULL
    assert call(l1=None) == C.VS_E_NULL
    assert call(gdt=7) == C.VS_E_DTYPE
    assert call(ldg=99) == C.VS_E_SHAPE
    assert call(grad=FAKE + 2) == C.VS_E_ALIGN
    assert call(scale=float("inf")) == C.VS_E_PARAM
    assert call(ws=None) == C.VS_E_WORKSPACE
    assert call(grad=None, ldg=0, gdt=7, ws=None) == C.VS_E_WORKSPACE  # no gradient: its dtype is not read


def test_backward_validation(lib):
    from logprob_entropy_sampling_amd import _capi as C
    hw = dict(kind=C.VS_SRC_HIDDEN_WEIGHT)

    def call(src, targets=FAKE, lse=FAKE, ent=FAKE, ge=None, chunk=8192, gh=FAKE, ldgh=64, gw=FAKE, ldgw=64,
             ws=FAKE, nws=1 << 40):
        return lib.vs_score_full_backward(ctypes.byref(src), targets, lse, ent, FAKE, ge, chunk, gh, ldgh, gw, ldgw,
                                          ws, nws, None)
    assert call(_src()) == C.VS_E_UNSUPPORTED  # a logits source
    assert call(_src(**hw), lse=None) == C.VS_E_NULL
    assert call(_src(**hw), ent=None, ge=FAKE) == C.VS_E_NULL
    assert call(_src(**hw), gh=None, gw=None) == C.VS_E_NULL
    assert call(_src(**hw), chunk=0) == C.VS_E_PARAM
    assert call(_src(**hw), ldgh=63) == C.VS_E_SHAPE
    assert call(_src(**hw), gw=FAKE + 2) == C.VS_E_ALIGN
    assert call(_src(**hw), ws=None) == C.VS_E_WORKSPACE
    big = _src(T=4096, H=4096, V=151936, ld_hidden=4096, ld_weight=4096, **hw)
    n = lib.vs_workspace_size(C.VS_OP_SCORE_FULL_BACKWARD, ctypes.byref(big), 8192)
    # hidden^T, G, G^T and one chunk of W^T, bf16
    assert n >= 2 * (4096 * 4096 + 4096 * 8192 + 8192 * 4096 + 4096 * 8192)
    # the chunk is capped at 2^23 vocabulary rows (the row stride of G): a larger one needs no more workspace
    huge = _src(T=16, H=64, V=(1 << 24) + 5, ld_hidden=64, ld_weight=64, **hw)
    capped = lib.vs_workspace_size(C.VS_OP_SCORE_FULL_BACKWARD, ctypes.byref(huge), 1 << 23)
    assert capped == lib.vs_workspace_size(C.VS_OP_SCORE_FULL_BACKWARD, ctypes.byref(huge), 1 << 30)
    assert capped > lib.vs_workspace_size(C.VS_OP_SCORE_FULL_BACKWARD, ctypes.byref(huge), 1 << 22)


def test_hidden_source_transforms_vocabulary_limit(lib):
    """The logits block of a hidden/weight source keeps a row stride (V rounded up to 8) of at most 2^23."""
    from logprob_entropy_sampling_amd import _capi as C
    hw = dict(kind=C.VS_SRC_HIDDEN_WEIGHT, T=4, H=64, ld_hidden=64, ld_weight=64)
    for V, rc in ((1 << 23, C.VS_E_WORKSPACE), ((1 << 23) + 1, C.VS_E_UNSUPPORTED)):
        src = _src(V=V, **hw)
        got = lib.vs_score_transforms(ctypes.byref(src), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, 0, FAKE, None, 0, None)
        assert got == rc, (V, got)
        got = lib.vs_sample_transforms(ctypes.byref(src), FAKE, FAKE, FAKE, 1, 0, FAKE, None, None, None, None, None,
                                       0, None)
        assert got == rc, (V, got)
