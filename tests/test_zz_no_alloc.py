"""qwm_quantize_keys_noalloc (the key quantizer for callers that cannot
allocate: its scratch is a static device array) against qwm_quantize_keys on
the same inputs: two calls in a row, the second smaller, both bit-identical to
the workspace entry point; sizes past the limits are refused on the host."""
import ctypes as C
import sys

import numpy as np
import pytest

import datagen

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _packed_equal(a, b):
    for name in ("codes", "idx", "scale", "zeros", "c", "c_scale"):
        x, y = getattr(a, name), getattr(b, name)
        assert bool((x == y).all()), name


def test_noalloc_keys_match_workspace_call():
    import torch
    import bit_kv_cache_head_amd as qwm
    from gpu_helpers import dev_tokens
    assert torch.cuda.is_available()
    # (tokens, heads): a 480p-shaped chunk, then a smaller ragged one
    for T, H, seed in ((1560, 12, 3), (300, 4, 4)):
        _log(f"no-alloc keys T={T} H={H}")
        w = datagen.make_workload("480p", heads=list(range(H)), n_chunks=1, chunk=T)
        K = dev_tokens(w.K, "bf16")
        st = qwm.QueryStats(H)
        qwm.update_query_stats(dev_tokens(w.Q, "bf16"), st, compute_basis=True)
        table = qwm.build_centroids(K, 2, seed=seed)
        for flags in (qwm.QWM_QSAC | qwm.QWM_PSAC, qwm.QWM_QSAC | qwm.QWM_PSAC | qwm.QWM_PSAC_KEEP, 0):
            d_ref, d_new = qwm.new_diag(), qwm.new_diag()
            ref = qwm.quantize_keys(K, table, st.w, st.U, M=8, flags=flags, diag=d_ref)
            new = qwm.quantize_keys_noalloc(K, table, st.w, st.U, M=8, flags=flags, diag=d_new)
            torch.cuda.synchronize()
            _packed_equal(ref, new)
            assert d_ref.tolist() == d_new.tolist()
            _log(f"  flags={flags} identical (diag {d_new.tolist()})")


def test_noalloc_keys_limits():
    from bit_kv_cache_head_amd._abi import lib, Tokens, Packed, QWM_NOALLOC_MAX_HEADS, QWM_NOALLOC_MAX_TOKEN_HEADS
    for H, T in ((QWM_NOALLOC_MAX_HEADS + 1, 16), (16, QWM_NOALLOC_MAX_TOKEN_HEADS // 16 + 1)):
        t = Tokens(C.c_void_p(0x1000), 1, H, 128, 0, T, 128 * H, 128)
        out = Packed(C.c_void_p(0x2000), C.c_void_p(0x3000), C.c_void_p(0x4000), C.c_void_p(0x5000),
                     C.c_void_p(0x6000), C.c_void_p(0x7000), T, H, 8)
        assert lib.qwm_quantize_keys_noalloc(C.byref(t), C.c_void_p(0x8000), None, None, 8, 3, C.byref(out),
                                             None, None) == 2
        assert b"token-heads" in lib.qwm_last_error()
