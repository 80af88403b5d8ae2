"""ctypes declarations of libvocabscore.so (mirrors include/vocabscore.h)."""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint64, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvocabscore.so")

(VS_OK, VS_E_NULL, VS_E_SHAPE, VS_E_DTYPE, VS_E_ALIGN, VS_E_PARAM, VS_E_WORKSPACE, VS_E_UNSUPPORTED, VS_E_DEVICE,
 VS_E_SCRATCH) = range(10)
VS_F32, VS_BF16 = 0, 1
VS_SRC_LOGITS, VS_SRC_HIDDEN_WEIGHT = 0, 1
(VS_OP_SCORE_FULL, VS_OP_SCORE_SUPPORT, VS_OP_SCORE_TRANSFORMS, VS_OP_L1_DISTANCE, VS_OP_SAMPLE_TRANSFORMS,
 VS_OP_L1_LOSS, VS_OP_SCORE_FULL_BACKWARD, VS_OP_SCORE_SUPPORT_BACKWARD) = range(8)

ROW_EMPTY_SUPPORT = 0x01
ROW_TARGET_OUTSIDE_SUPPORT = 0x02
ROW_BAD_INPUT = 0x04
ROW_FULL_VOCAB_FALLBACK = 0x08
ROW_SUPPORT_TRUNCATED = 0x10


class VsSource(ctypes.Structure):
    _fields_ = [
        ("kind", c_int32),
        ("logits", c_void_p),
        ("logits_dtype", c_int32),
        ("ld_logits", c_int64),
        ("hidden", c_void_p),
        ("hidden_dtype", c_int32),
        ("ld_hidden", c_int64),
        ("weight", c_void_p),
        ("weight_dtype", c_int32),
        ("ld_weight", c_int64),
        ("T", c_int64),
        ("H", c_int64),
        ("V", c_int64),
        ("temperature", c_void_p),
        ("temperature_scalar", c_float),
    ]


_SIGS = {
    "vs_version": (c_int32, []),
    "vs_status_string": (c_char_p, [c_int32]),
    "vs_workspace_size": (c_size_t, [c_int32, POINTER(VsSource), c_int64]),
    "vs_score_full": (c_int32, [POINTER(VsSource), c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_size_t, c_void_p]),
    "vs_score_support_ids": (c_int32, [POINTER(VsSource), c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_int64,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "vs_score_transforms": (c_int32, [POINTER(VsSource), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                                      c_size_t, c_void_p]),
    "vs_sample_transforms": (c_int32, [POINTER(VsSource), c_void_p, c_void_p, c_void_p, c_uint64, c_uint64, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "vs_l1_distance": (c_int32, [c_void_p, c_void_p, c_int32, c_int64, c_int64, c_int64, c_int64, c_void_p, c_void_p,
                                 c_void_p, c_size_t, c_void_p]),
    "vs_score_full_backward": (c_int32, [POINTER(VsSource), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                         c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_size_t, c_void_p]),
    "vs_score_full_noalloc": (c_int32, [POINTER(VsSource), c_void_p, c_int64, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p]),
    "vs_noalloc_scratch_bytes": (c_size_t, []),
    "vs_l1_loss": (c_int32, [c_void_p, c_void_p, c_int32, c_int64, c_int64, c_int64, c_int64, c_void_p, c_float,
                             c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int64, c_void_p, c_size_t, c_void_p]),
    "vs_score_support_backward": (c_int32, [c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_size_t, c_void_p]),
    "vs_sweep_timer": (c_int32, [c_int32]),
    "vs_sweep_timer_ms": (c_int32, [POINTER(c_float)]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library and declare every entry point's signature."""
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m logprob_entropy_sampling_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib
