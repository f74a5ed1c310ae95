"""The C ABI: the library loads without a GPU, exports every declared symbol,
and rejects bad arguments on the host before any HIP call."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "quantwm.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qwm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    from bit_kv_cache_head_amd import _abi
    declared = _declared()
    assert declared, "no declarations found"
    assert sorted(_abi.EXPORTS) == declared
    for name in declared:
        assert hasattr(_abi.lib, name), name
    assert _abi.lib.qwm_abi_version() == 6


def test_struct_layouts_match_header_sizes():
    from bit_kv_cache_head_amd import _abi
    assert C.sizeof(_abi.Tokens) == 48
    assert C.sizeof(_abi.QStats) == 72
    assert C.sizeof(_abi.Packed) == 64
    assert C.sizeof(_abi.Segment) == 152
    assert C.sizeof(_abi.CDir) == 16
    assert C.sizeof(_abi.Diag) == 32


def test_sizes_and_strides():
    from bit_kv_cache_head_amd._abi import lib
    assert lib.qwm_zeros_stride(1) == 4
    assert lib.qwm_zeros_stride(8) == 4
    assert lib.qwm_zeros_stride(9) == 8
    assert lib.qwm_zeros_stride(1560) == 780
    assert lib.qwm_workspace_bytes(0, 1560, 12, 0, 0) == 0
    k = lib.qwm_workspace_bytes(2, 1560, 12, 0, 0)
    assert k >= 12 * 256 * 4 * 2 + 12 * 1560 * 4          # B_j split per centroid + fallback worklist
    assert lib.qwm_workspace_bytes(1, 1560, 12, 0, 0) > k       # Lloyd adds assignment + shuffle
    # attention: the segment descriptors, fp16 centroid tables for every (segment, head),
    # plus split partials; one split: descriptors, tables and basis fragments only
    assert lib.qwm_workspace_bytes(4, 64, 1, 16, 1) == 256 + 2 * 256 * 128 * 2 + 32 * 128 * 2   # basis rows up to rank 32
    big = lib.qwm_workspace_bytes(4, 39000, 12, 1560, 25)
    assert big >= 25 * 12 * 2 * 256 * 128 * 2
    assert lib.qwm_workspace_bytes(4, 39000, 12, 1560, 0) == 0


def _tok(ptr=0x1000, T=16, H=2, d=128, dtype=1, st=256, sh=128):
    from bit_kv_cache_head_amd._abi import Tokens
    return Tokens(C.c_void_p(ptr), dtype, H, d, 0, T, st, sh)


@pytest.mark.parametrize("case,code", [
    (dict(d=64), 2), (dict(dtype=7), 2), (dict(H=0), 1), (dict(ptr=0), 1), (dict(ptr=0x1004), 1),
    (dict(st=100), 1), (dict(T=-1), 1),
])
def test_key_argument_validation(case, code):
    """Errors come back before any device access (pointers here are never dereferenced)."""
    from bit_kv_cache_head_amd._abi import lib, Packed
    t = _tok(**case)
    out = Packed(C.c_void_p(0x2000), C.c_void_p(0x3000), C.c_void_p(0x4000), C.c_void_p(0x5000),
                 C.c_void_p(0x6000), C.c_void_p(0x7000), t.T, t.H, 8)
    st = lib.qwm_quantize_keys(C.byref(t), C.c_void_p(0x8000), None, None, 8, 3, C.byref(out), None,
                               None, 0, None)
    assert st == code
    assert lib.qwm_last_error()


def test_other_validation_paths():
    from bit_kv_cache_head_amd._abi import lib, Packed, QStats
    t = _tok()
    out = Packed(C.c_void_p(0x2000), C.c_void_p(0x3000), C.c_void_p(0x4000), C.c_void_p(0x5000),
                 C.c_void_p(0x6000), C.c_void_p(0x7000), t.T, t.H, 8)
    # M out of range, unknown flags, workspace missing
    assert lib.qwm_quantize_keys(C.byref(t), C.c_void_p(0x8000), None, None, 0, 1, C.byref(out), None,
                                 None, 0, None) == 1
    assert lib.qwm_quantize_keys(C.byref(t), C.c_void_p(0x8000), None, None, 8, 8, C.byref(out), None,
                                 None, 0, None) == 1
    assert lib.qwm_quantize_keys(C.byref(t), C.c_void_p(0x8000), None, None, 8, 3, C.byref(out), None,
                                 None, 0, None) == 3
    assert b"workspace" in lib.qwm_last_error()
    # shape mismatch between tokens and packed chunk
    bad = Packed(C.c_void_p(0x2000), C.c_void_p(0x3000), C.c_void_p(0x4000), C.c_void_p(0x5000),
                 C.c_void_p(0x6000), C.c_void_p(0x7000), t.T + 1, t.H, 8)
    assert lib.qwm_quantize_values(C.byref(t), C.c_void_p(0x8000), C.byref(bad), None, None, 0, None) == 1
    # Lloyd: seeded start needs >= 256 tokens; centroid count must be 256
    assert lib.qwm_build_centroids(C.byref(t), 256, 3, 0, None, C.c_void_p(0x9000), None, None, 0, None) == 1
    assert lib.qwm_build_centroids(C.byref(t), 128, 3, 0, None, C.c_void_p(0x9000), None, None, 0, None) == 2
    # stats: rank must be 8, H must match
    qs = QStats(C.c_void_p(0x1000), C.c_void_p(0x2000), C.c_void_p(0x3000), C.c_void_p(0x4000),
                C.c_void_p(0x5000), C.c_void_p(0x6000), None, t.H, 128, 4, 0)
    assert lib.qwm_update_query_stats(C.byref(t), C.byref(qs), 1, None, 0, None) == 2
    qs.r, qs.H = 8, 3
    assert lib.qwm_update_query_stats(C.byref(t), C.byref(qs), 1, None, 0, None) == 1
    # attention: segments, scale
    segs = _segs(3)
    assert lib.qwm_attention(C.byref(t), None, 1, C.c_float(0.1), C.c_void_p(0x1000), None, None,
                             None, 0, None) == 1
    assert lib.qwm_attention(C.byref(t), segs, 0, C.c_float(0.1), C.c_void_p(0x1000),
                             None, None, None, 0, None) == 1
    assert lib.qwm_attention(C.byref(t), segs, 3, C.c_float(-1.0), C.c_void_p(0x1000),
                             None, None, None, 0, None) == 1
    # valid descriptors but no workspace: the workspace check comes last
    assert lib.qwm_attention(C.byref(t), segs, 3, C.c_float(0.1), C.c_void_p(0x1000),
                             None, None, None, 0, None) == 3


def _segs(n, T=100):
    """Host descriptors with aligned (never dereferenced) device addresses."""
    from bit_kv_cache_head_amd._abi import Segment
    arr = (Segment * n)()
    for i in range(n):
        s = arr[i]
        base = 0x100000 * (i + 1)
        for k, name in enumerate(["k_codes", "k_idx", "k_scale", "k_zeros", "k_c", "k_c_scale", "v_codes",
                                  "v_idx", "v_scale", "v_zeros", "k_centroids", "v_centroids", "U"]):
            setattr(s, name, base + 0x1000 * k)
        s.T = T
        s.r = 8
    return arr


@pytest.mark.parametrize("field,value,code", [
    ("T", 0, 1), ("T", 1 << 26, 1), ("T", -5, 1), ("k_codes", 0, 1), ("v_centroids", 0, 1),
    ("k_codes", 0x100004, 1), ("k_scale", 0x100002, 1), ("U", 0x100008, 1), ("k_c", 0x100004, 1),
    ("r", 12, 2), ("r", 0, 2),
])
def test_attention_segment_validation(field, value, code):
    """Every host descriptor is checked before any HIP call: a bad segment T,
    a null array or a misaligned pointer in segment 1 of 3 is QWM_ERR_ARG."""
    from bit_kv_cache_head_amd._abi import lib
    t = _tok()
    segs = _segs(3)
    setattr(segs[1], field, value)
    ws = C.c_void_p(0x10000000)
    args = (C.c_float(0.1), C.c_void_p(0x1000), None, None, ws, 1 << 40, None)
    assert lib.qwm_attention(C.byref(t), segs, 3, *args) == code
    assert b"segment 1" in lib.qwm_last_error()
    ka = _tok(ptr=0x2000, T=8)
    assert lib.qwm_attention_active(C.byref(t), segs, 3, C.byref(ka), C.byref(ka), *args) == code


def test_attention_total_keys_limit():
    """Keys are summed on the host: 2^31 or more in all is refused."""
    from bit_kv_cache_head_amd._abi import lib
    t = _tok()
    segs = _segs(40, T=(1 << 26) - 1)
    assert lib.qwm_attention(C.byref(t), segs, 40, C.c_float(0.1), C.c_void_p(0x1000), None, None,
                             C.c_void_p(0x10000000), 1 << 40, None) == 2
    assert b"2^31" in lib.qwm_last_error()


def test_reference_top1_validation():
    from bit_kv_cache_head_amd._abi import lib
    q = _tok(dtype=1)
    k = _tok(ptr=0x2000, dtype=1, T=100)
    assert lib.qwm_reference_top1(C.byref(q), C.byref(_tok(ptr=0x2000, dtype=0)), C.c_void_p(0x3000), None) == 2
    assert lib.qwm_reference_top1(C.byref(q), C.byref(_tok(ptr=0x2000, H=3)), C.c_void_p(0x3000), None) == 1
    assert lib.qwm_reference_top1(C.byref(q), C.byref(k), None, None) == 1
    assert b"top1" in lib.qwm_last_error()


def test_attention_merge_validation():
    from bit_kv_cache_head_amd._abi import lib
    p = [C.c_void_p(a) for a in (0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000)]
    # null part, bad sizes, lse aliasing a part's lse, misaligned buffer: rejected before any device access
    assert lib.qwm_attention_merge(None, p[1], p[2], p[3], 10, 2, p[4], p[5], None) == 1
    assert lib.qwm_attention_merge(p[0], p[1], p[2], p[3], 0, 2, p[4], p[5], None) == 1
    assert lib.qwm_attention_merge(p[0], p[1], p[2], p[3], 10, 0, p[4], p[5], None) == 1
    assert lib.qwm_attention_merge(p[0], p[1], p[2], p[3], 10, 2, p[4], p[1], None) == 1
    assert b"alias" in lib.qwm_last_error()
    assert lib.qwm_attention_merge(p[0], p[1], p[2], p[3], 10, 2, C.c_void_p(0x4002), p[5], None) == 1
