"""ctypes mirror of include/quantwm.h.  Loading the library does not touch the GPU."""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libquantwm.so")

QWM_OK, QWM_ERR_ARG, QWM_ERR_UNSUPPORTED, QWM_ERR_WORKSPACE, QWM_ERR_HIP = 0, 1, 2, 3, 4
QWM_F32, QWM_BF16 = 0, 1
QWM_QSAC, QWM_PSAC, QWM_PSAC_KEEP = 1, 2, 4
QWM_OP_STATS, QWM_OP_CENTROIDS, QWM_OP_KEYS, QWM_OP_VALUES, QWM_OP_ATTENTION, QWM_OP_ATTENTION_ACTIVE = 0, 1, 2, 3, 4, 5
QWM_OP_KEEP_FULL = 6
QWM_LAYOUT_DENSE, QWM_LAYOUT_SPARSE, QWM_LAYOUT_OVERFLOW = 0, 1, -1
QWM_NOALLOC_MAX_HEADS, QWM_NOALLOC_MAX_TOKEN_HEADS = 64, 1 << 21

# every symbol include/quantwm.h declares
EXPORTS = ["qwm_update_query_stats", "qwm_build_centroids", "qwm_quantize_keys", "qwm_quantize_keys_noalloc",
           "qwm_quantize_keys_fullq",
           "qwm_quantize_values", "qwm_attention", "qwm_attention_merge", "qwm_attention_active", "qwm_decode_segment", "qwm_centroid_residual", "qwm_reference_top1", "qwm_two_level_scales", "qwm_psac_keep_full", "qwm_compact_coefficients",
           "qwm_coefficient_bytes", "qwm_workspace_bytes", "qwm_zeros_stride", "qwm_last_error", "qwm_abi_version"]


class Tokens(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("dtype", C.c_int32), ("H", C.c_int32), ("d", C.c_int32),
                ("reserved", C.c_int32), ("T", C.c_int64), ("stride_t", C.c_int64), ("stride_h", C.c_int64)]


class QStats(C.Structure):
    _fields_ = [("S", C.c_void_p), ("n", C.c_void_p), ("w", C.c_void_p), ("U", C.c_void_p),
                ("lam", C.c_void_p), ("energy", C.c_void_p), ("iters", C.c_void_p),
                ("H", C.c_int32), ("d", C.c_int32), ("r", C.c_int32), ("reserved", C.c_int32)]


class Packed(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("idx", C.c_void_p), ("scale", C.c_void_p), ("zeros", C.c_void_p),
                ("c", C.c_void_p), ("c_scale", C.c_void_p), ("T", C.c_int64), ("H", C.c_int32),
                ("r", C.c_int32)]


class Diag(C.Structure):
    _fields_ = [("nonfinite_rows", C.c_int64), ("exact_fallbacks", C.c_int64),
                ("scale_saturations", C.c_int64), ("layout_overflows", C.c_int64)]


class CDir(C.Structure):
    _fields_ = [("layout", C.c_int32), ("count", C.c_int32), ("offset", C.c_int64)]


class Segment(C.Structure):
    _fields_ = [("k_codes", C.c_void_p), ("k_idx", C.c_void_p), ("k_scale", C.c_void_p),
                ("k_zeros", C.c_void_p), ("k_c", C.c_void_p), ("k_c_scale", C.c_void_p),
                ("v_codes", C.c_void_p), ("v_idx", C.c_void_p), ("v_scale", C.c_void_p),
                ("v_zeros", C.c_void_p), ("k_centroids", C.c_void_p), ("v_centroids", C.c_void_p),
                ("U", C.c_void_p), ("T", C.c_int64), ("r", C.c_int32), ("reserved", C.c_int32),
                ("k_cdir", C.c_void_p), ("k_carena", C.c_void_p), ("k_scale2", C.c_void_p), ("v_scale2", C.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python bit_kv_cache_head_amd/build.py`")
    L = C.CDLL(LIB_PATH)
    P = C.c_void_p
    L.qwm_update_query_stats.argtypes = [P, P, C.c_int32, P, C.c_size_t, P]
    L.qwm_build_centroids.argtypes = [P, C.c_int32, C.c_int32, C.c_uint64, P, P, P, P, C.c_size_t, P]
    L.qwm_quantize_keys.argtypes = [P, P, P, P, C.c_int32, C.c_uint32, P, P, P, C.c_size_t, P]
    L.qwm_quantize_keys_noalloc.argtypes = [P, P, P, P, C.c_int32, C.c_uint32, P, P, P]
    L.qwm_quantize_keys_fullq.argtypes = [P, P, P, P, P, P, C.c_int32, C.c_uint32, P, P, P, C.c_size_t, P]
    L.qwm_quantize_values.argtypes = [P, P, P, P, P, C.c_size_t, P]
    L.qwm_attention.argtypes = [P, P, C.c_int32, C.c_float, P, P, P, P, C.c_size_t, P]
    L.qwm_attention_merge.argtypes = [P, P, P, P, C.c_int64, C.c_int32, P, P, P]
    L.qwm_attention_active.argtypes = [P, P, C.c_int32, P, P, C.c_float, P, P, P, P, C.c_size_t, P]
    L.qwm_decode_segment.argtypes = [P, C.c_int32, P, P, C.c_int64, C.c_int64, P]
    L.qwm_centroid_residual.argtypes = [P, P, P, P, C.c_int64, C.c_int64, P]
    L.qwm_reference_top1.argtypes = [P, P, P, P]
    L.qwm_two_level_scales.argtypes = [P, P, P, P, C.c_uint32, C.c_int32, P, P, P, P, P]
    L.qwm_psac_keep_full.argtypes = [P, P, P, P, P, P, P, P, P, C.c_size_t, P]
    L.qwm_compact_coefficients.argtypes = [P, P, P, C.c_int64, P, P, P]
    L.qwm_coefficient_bytes.argtypes = [C.c_int32, C.c_int64, C.c_int64, C.c_int32]
    L.qwm_coefficient_bytes.restype = C.c_int64
    L.qwm_workspace_bytes.argtypes = [C.c_int32, C.c_int64, C.c_int32, C.c_int64, C.c_int32]
    L.qwm_workspace_bytes.restype = C.c_size_t
    L.qwm_zeros_stride.argtypes = [C.c_int64]
    L.qwm_zeros_stride.restype = C.c_int64
    L.qwm_last_error.restype = C.c_char_p
    L.qwm_abi_version.restype = C.c_int32
    for name in ("qwm_update_query_stats", "qwm_build_centroids", "qwm_quantize_keys", "qwm_quantize_keys_noalloc",
                 "qwm_quantize_keys_fullq",
                 "qwm_quantize_values", "qwm_attention", "qwm_attention_merge", "qwm_attention_active",
                 "qwm_decode_segment", "qwm_centroid_residual", "qwm_reference_top1", "qwm_two_level_scales",
                 "qwm_psac_keep_full", "qwm_compact_coefficients"):
        getattr(L, name).restype = C.c_int
    return L


lib = _load()


class QwmError(RuntimeError):
    pass


def check(status: int):
    if status != QWM_OK:
        raise QwmError(f"libquantwm status {status}: {lib.qwm_last_error().decode(errors='replace')}")
