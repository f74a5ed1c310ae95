"""Python binding of libquantwm (the QuantWM 2-bit KV-cache hot path on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
libquantwm.so.  PyTorch provides device memory and the current stream.  The
library must be built first (python bit_kv_cache_head_amd/build.py); importing
this package raises if it is missing.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

from ._abi import (lib, LIB_PATH, QWM_OK, QWM_F32, QWM_BF16, QWM_QSAC, QWM_PSAC, QWM_PSAC_KEEP, QWM_OP_STATS,
                   QWM_OP_CENTROIDS, QWM_OP_KEYS, QWM_OP_VALUES, QWM_OP_ATTENTION, QWM_OP_ATTENTION_ACTIVE,
                   QWM_OP_KEEP_FULL, QWM_LAYOUT_DENSE, QWM_LAYOUT_SPARSE, Tokens, QStats, Packed, Diag, Segment, CDir,
                   check)

D, NC, R, GROUP = 128, 256, 8, 64

__all__ = ["QueryStats", "PackedChunk", "Workspace", "update_query_stats", "build_centroids",
           "quantize_keys", "quantize_values", "attention", "segment_array", "SegmentArray", "zeros_stride",
           "QWM_QSAC", "QWM_PSAC", "QWM_PSAC_KEEP", "LIB_PATH", "new_diag"]


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return C.c_void_p(0 if t is None else t.data_ptr())


def _tokens(x: torch.Tensor) -> Tokens:
    """Descriptor of a [T, H, d] tensor (bf16 or fp32, channel stride 1)."""
    if x.dim() != 3:
        raise ValueError("token tensor must be [T, H, d]")
    if not x.is_cuda:
        raise ValueError("token tensor must be on the GPU")
    if x.stride(2) != 1:
        raise ValueError("channel stride must be 1")
    dt = {torch.bfloat16: QWM_BF16, torch.float32: QWM_F32}.get(x.dtype)
    if dt is None:
        raise ValueError("token dtype must be bfloat16 or float32")
    T, H, d = x.shape
    return Tokens(C.c_void_p(x.data_ptr()), dt, H, d, 0, T, x.stride(0), x.stride(1))


def zeros_stride(T: int) -> int:
    return int(lib.qwm_zeros_stride(T))


class Workspace:
    """Grow-only device scratch buffers (256-byte aligned by the caching
    allocator), one per stream: calls enqueued on different streams may run
    concurrently and must not share scratch memory."""

    def __init__(self):
        self.bufs = {}

    def get(self, nbytes: int, device) -> tuple:
        if nbytes == 0:
            return C.c_void_p(0), 0
        key = (device, torch.cuda.current_stream(device).cuda_stream)
        buf = self.bufs.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
            self.bufs[key] = buf
        return C.c_void_p(buf.data_ptr()), buf.numel()


_WS = Workspace()


def new_diag(device="cuda") -> torch.Tensor:
    """Device counters: [nonfinite_rows, exact_fallbacks, scale_saturations, layout_overflows] int64."""
    return torch.zeros(4, dtype=torch.int64, device=device)


class QueryStats:
    """Per-head running Query statistics and principal basis (device tensors);
    r = PSAC rank (8, or 16 / 32 for the rank ablation)."""

    def __init__(self, H: int, device="cuda", r: int = R):
        self.H, self.r = H, r
        self.S = torch.zeros(H, D, D, dtype=torch.float64, device=device)
        self.n = torch.zeros(H, dtype=torch.int64, device=device)
        self.w = torch.ones(H, D, dtype=torch.float32, device=device)
        self.U = torch.zeros(H, D, r, dtype=torch.bfloat16, device=device)
        self.lam = torch.zeros(H, r, dtype=torch.float32, device=device)
        self.energy = torch.zeros(H, dtype=torch.float32, device=device)
        self.iters = torch.zeros(H, dtype=torch.int32, device=device)

    def reset(self):
        """Back to the cold start (no Queries seen)."""
        self.S.zero_()
        self.n.zero_()
        self.w.fill_(1.0)
        self.U.zero_()

    def desc(self) -> QStats:
        return QStats(_ptr(self.S), _ptr(self.n), _ptr(self.w), _ptr(self.U), _ptr(self.lam),
                      _ptr(self.energy), _ptr(self.iters), self.H, D, self.r, 0)


class PackedChunk:
    """One packed chunk: codes [H,T,32] u8, idx [H,T] u8, scale [H,T,2] fp16 bits,
    zeros [H, zstride] u8, c [H,T,8] i8 and c_scale [H,T] fp16 bits (keys)."""

    def __init__(self, T: int, H: int, keys: bool, device="cuda", r: int = R):
        self.T, self.H, self.keys, self.r = T, H, keys, r
        self.scale_q = self.scale2 = None      # two-level scales (two_level_scales)
        self.cdir = self.carena = None         # compacted coefficients (compact_coefficients)
        self.codes = torch.empty(H, T, D // 4, dtype=torch.uint8, device=device)
        self.idx = torch.empty(H, T, dtype=torch.uint8, device=device)
        self.scale = torch.empty(H, T, 2, dtype=torch.int16, device=device)
        self.zeros = torch.zeros(H, zeros_stride(T), dtype=torch.uint8, device=device)
        self.c = torch.empty(H, T, r, dtype=torch.int8, device=device) if keys else None
        self.c_scale = torch.empty(H, T, dtype=torch.int16, device=device) if keys else None

    def desc(self) -> Packed:
        return Packed(_ptr(self.codes), _ptr(self.idx), _ptr(self.scale), _ptr(self.zeros),
                      _ptr(self.c), _ptr(self.c_scale), self.T, self.H, self.r)

    def nbytes(self) -> int:
        """Bytes the chunk keeps: codes, indices, zero-points, its scales
        (fp16, or INT8 codes plus the second level) and its coefficients
        (dense, or as compacted)."""
        tot = self.codes.numel() + self.idx.numel() + self.zeros.numel()
        tot += 2 * self.scale.numel() if self.scale2 is None else self.scale_q.numel() + 2 * self.scale2.numel()
        if self.keys:
            if self.cdir is None:
                tot += self.c.numel() + 2 * self.c_scale.numel()
            else:
                tot += sum(self.coefficient_bytes())
        return tot

    def coefficient_bytes(self) -> list:
        """Per head: bytes of the compacted coefficients (host read of the directory)."""
        d = self.cdir.cpu().numpy().view(np.int64).reshape(self.H, 2)
        out = []
        for h in range(self.H):
            layout, count = int(d[h, 0] & 0xFFFFFFFF), int(d[h, 0] >> 32)
            layout = layout - (1 << 32) if layout >= 1 << 31 else layout
            out.append(int(lib.qwm_coefficient_bytes(layout, self.T, count, self.r)) if layout >= 0 else 0)
        return out

    def layouts(self) -> list:
        """Per head: (layout, kept count, arena offset) of the compacted coefficients."""
        d = self.cdir.cpu().numpy().view(np.int64).reshape(self.H, 2)
        res = []
        for h in range(self.H):
            lo = int(d[h, 0] & 0xFFFFFFFF)
            res.append((lo - (1 << 32) if lo >= 1 << 31 else lo, int(d[h, 0] >> 32), int(d[h, 1])))
        return res


def update_query_stats(q: torch.Tensor, st: QueryStats, compute_basis: bool = True):
    td = _tokens(q)
    check(lib.qwm_update_query_stats(C.byref(td), C.byref(st.desc()), int(compute_basis),
                                     C.c_void_p(0), 0, _stream()))


def build_centroids(x: torch.Tensor, iters: int, seed: int = 0, init: torch.Tensor | None = None,
                    out: torch.Tensor | None = None, diag: torch.Tensor | None = None) -> torch.Tensor:
    """[H, 256, 128] bf16 centroid table by `iters` Lloyd iterations."""
    td = _tokens(x)
    if out is None:
        out = torch.empty(td.H, NC, D, dtype=torch.bfloat16, device=x.device)
    ws, nb = _WS.get(lib.qwm_workspace_bytes(QWM_OP_CENTROIDS, td.T, td.H, 0, 0), x.device)
    check(lib.qwm_build_centroids(C.byref(td), NC, iters, C.c_uint64(seed), _ptr(init), _ptr(out),
                                  _ptr(diag), ws, nb, _stream()))
    return out


def quantize_keys(k: torch.Tensor, centroids: torch.Tensor, w: torch.Tensor | None, U: torch.Tensor | None,
                  M: int = 8, flags: int = QWM_QSAC | QWM_PSAC, out: PackedChunk | None = None,
                  diag: torch.Tensor | None = None) -> PackedChunk:
    td = _tokens(k)
    if out is None:
        out = PackedChunk(td.T, td.H, True, k.device, r=R if U is None else U.shape[2])
    ws, nb = _WS.get(lib.qwm_workspace_bytes(QWM_OP_KEYS, td.T, td.H, 0, 0), k.device)
    check(lib.qwm_quantize_keys(C.byref(td), _ptr(centroids), _ptr(w), _ptr(U), M, flags,
                                C.byref(out.desc()), _ptr(diag), ws, nb, _stream()))
    return out


def quantize_keys_noalloc(k: torch.Tensor, centroids: torch.Tensor, w: torch.Tensor | None, U: torch.Tensor | None,
                          M: int = 8, flags: int = QWM_QSAC | QWM_PSAC, out: PackedChunk | None = None,
                          diag: torch.Tensor | None = None) -> PackedChunk:
    """quantize_keys without a workspace: the library's static device scratch
    (at most 64 heads and 2^21 token-heads per call; calls that overlap on one
    device race)."""
    td = _tokens(k)
    if out is None:
        out = PackedChunk(td.T, td.H, True, k.device, r=R if U is None else U.shape[2])
    check(lib.qwm_quantize_keys_noalloc(C.byref(td), _ptr(centroids), _ptr(w), _ptr(U), M, flags,
                                        C.byref(out.desc()), _ptr(diag), _stream()))
    return out


def quantize_keys_fullq(k: torch.Tensor, centroids: torch.Tensor, S: torch.Tensor, n: torch.Tensor,
                        w: torch.Tensor | None, U: torch.Tensor | None, M: int = 8,
                        flags: int = QWM_QSAC | QWM_PSAC, out: PackedChunk | None = None,
                        diag: torch.Tensor | None = None) -> PackedChunk:
    """QSAC with candidates by the full Query second-moment matrix S / n
    (S [H, 128, 128] fp64, n [H] int64, as QueryStats keeps them)."""
    td = _tokens(k)
    if S.dtype != torch.float64 or tuple(S.shape) != (td.H, D, D) or not S.is_contiguous():
        raise ValueError("S must be a contiguous [H, 128, 128] float64 tensor")
    if n.dtype != torch.int64 or tuple(n.shape) != (td.H,):
        raise ValueError("n must be an [H] int64 tensor")
    if out is None:
        out = PackedChunk(td.T, td.H, True, k.device, r=R if U is None else U.shape[2])
    ws, nb = _WS.get(lib.qwm_workspace_bytes(QWM_OP_KEYS, td.T, td.H, 0, 0), k.device)
    check(lib.qwm_quantize_keys_fullq(C.byref(td), _ptr(centroids), _ptr(S), _ptr(n), _ptr(w), _ptr(U), M, flags,
                                      C.byref(out.desc()), _ptr(diag), ws, nb, _stream()))
    return out


def quantize_values(v: torch.Tensor, centroids: torch.Tensor, out: PackedChunk | None = None,
                    diag: torch.Tensor | None = None) -> PackedChunk:
    td = _tokens(v)
    if out is None:
        out = PackedChunk(td.T, td.H, False, v.device)
    ws, nb = _WS.get(lib.qwm_workspace_bytes(QWM_OP_VALUES, td.T, td.H, 0, 0), v.device)
    check(lib.qwm_quantize_values(C.byref(td), _ptr(centroids), C.byref(out.desc()), _ptr(diag),
                                  ws, nb, _stream()))
    return out


def centroid_residual(x: torch.Tensor, centroids: torch.Tensor, idx: torch.Tensor,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 [T, H, 128]: every token minus its assigned centroid (idx [H, T] u8)."""
    td = _tokens(x)
    if out is None:
        out = torch.empty(td.T, td.H, D, dtype=torch.float32, device=x.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (td.T, td.H, D) or out.stride(2) != 1:
        raise ValueError("residual output must be [T, H, 128] fp32 with contiguous rows")
    check(lib.qwm_centroid_residual(C.byref(td), _ptr(centroids), _ptr(idx), _ptr(out), out.stride(0),
                                    out.stride(1), _stream()))
    return out


def prq_quantize(x: torch.Tensor, stages: int, iters: int = 10, seed: int = 0):
    """QVG's progressive residual quantization of the tokens x [T, H, 128]:
    stages 1 .. S-1 each cluster the current residual (256 centroids, seeded
    Lloyd, seed + s - 1), take every token's nearest centroid and pass on the
    fp32 residual; the last stage codes that residual as values are coded.
    Returns ([(table, idx [H, T] u8)] for the first S - 1 stages, the last
    stage's table, its PackedChunk)."""
    if stages < 1:
        raise ValueError("stages must be >= 1")
    e = x
    first = []
    for s in range(stages - 1):
        Cs = build_centroids(e, iters, seed=seed + s)
        pk = quantize_values(e, Cs)              # idx: the nearest centroid of every token
        first.append((Cs, pk.idx))
        e = centroid_residual(e, Cs, pk.idx)
    C_last = build_centroids(e, iters, seed=seed + stages - 1)
    return first, C_last, quantize_values(e, C_last)


def two_level_scales(x: torch.Tensor, centroids: torch.Tensor, chunk: PackedChunk, w: torch.Tensor | None = None,
                     U: torch.Tensor | None = None, flags: int = QWM_QSAC | QWM_PSAC,
                     diag: torch.Tensor | None = None) -> PackedChunk:
    """Convert a quantized chunk (the x and table it was quantized with; for
    keys also its w, U and flags) to two-level group scales: INT8 step codes
    chunk.scale_q [H, T, 2] under fp16 second-level scales chunk.scale2 [H, 2];
    codes, zero-points (and C) re-encoded in place."""
    td = _tokens(x)
    chunk.scale_q = torch.empty(chunk.H, chunk.T, 2, dtype=torch.uint8, device=x.device)
    chunk.scale2 = torch.empty(chunk.H, 2, dtype=torch.int16, device=x.device)
    check(lib.qwm_two_level_scales(C.byref(td), _ptr(centroids), _ptr(w), _ptr(U), flags, int(chunk.keys),
                                   C.byref(chunk.desc()), _ptr(chunk.scale_q), _ptr(chunk.scale2), _ptr(diag),
                                   _stream()))
    return chunk


def psac_keep_full(k: torch.Tensor, centroids: torch.Tensor, st: "QueryStats", U: torch.Tensor,
                   chunk: PackedChunk) -> PackedChunk:
    """The keep test with the full second moment S / n of st on a key chunk
    quantized without QWM_PSAC_KEEP (coefficients dropped in place)."""
    td = _tokens(k)
    ws, nb = _WS.get(lib.qwm_workspace_bytes(QWM_OP_KEEP_FULL, td.T, td.H, chunk.r, 0), k.device)
    check(lib.qwm_psac_keep_full(C.byref(td), _ptr(centroids), _ptr(st.S), _ptr(st.n), _ptr(U), C.byref(chunk.desc()),
                                 _ptr(chunk.scale_q), _ptr(chunk.scale2), ws, nb, _stream()))
    return chunk


def compact_coefficients(chunk: PackedChunk, arena: torch.Tensor | None = None, used: torch.Tensor | None = None,
                         diag: torch.Tensor | None = None) -> PackedChunk:
    """Store the chunk's coefficients per head in the smaller of the dense and
    sparse layouts (chunk.cdir [H] directory, chunk.carena the arena).  Without
    an arena, one sized for the dense layout of every head is allocated."""
    H, T, r = chunk.H, chunk.T, chunk.r
    if arena is None:
        arena = torch.empty(H * int(lib.qwm_coefficient_bytes(QWM_LAYOUT_DENSE, T, T, r)), dtype=torch.uint8,
                            device=chunk.c.device)
    if used is None:
        used = torch.zeros(1, dtype=torch.int64, device=chunk.c.device)
    chunk.cdir = torch.empty(H * 16, dtype=torch.uint8, device=chunk.c.device)
    chunk.carena = arena
    check(lib.qwm_compact_coefficients(C.byref(chunk.desc()), _ptr(chunk.cdir), _ptr(arena), arena.numel(),
                                       _ptr(used), _ptr(diag), _stream()))
    return chunk


def _segment(kp, vp, kc, vc, U) -> Segment:
    s = Segment()
    s.k_codes, s.k_idx, s.k_scale, s.k_zeros = (kp.codes.data_ptr(), kp.idx.data_ptr(),
                                                kp.scale.data_ptr(), kp.zeros.data_ptr())
    s.k_c, s.k_c_scale = kp.c.data_ptr(), kp.c_scale.data_ptr()
    s.v_codes, s.v_idx, s.v_scale, s.v_zeros = (vp.codes.data_ptr(), vp.idx.data_ptr(),
                                                vp.scale.data_ptr(), vp.zeros.data_ptr())
    s.k_centroids, s.v_centroids = kc.data_ptr(), vc.data_ptr()
    s.U = 0 if U is None else U.data_ptr()
    s.T = kp.T
    s.r = kp.r
    if kp.cdir is not None:
        s.k_cdir, s.k_carena = kp.cdir.data_ptr(), kp.carena.data_ptr()
    if kp.scale2 is not None:
        s.k_scale, s.k_scale2 = kp.scale_q.data_ptr(), kp.scale2.data_ptr()
    if vp.scale2 is not None:
        s.v_scale, s.v_scale2 = vp.scale_q.data_ptr(), vp.scale2.data_ptr()
    return s


def decode_segment(kp, vp, kc, vc, U, k_out: torch.Tensor | None = None, v_out: torch.Tensor | None = None):
    """BF16 reconstruction of one packed chunk: (K_hat, V_hat) [T, H, 128] bf16
    (written into k_out / v_out, e.g. views of a larger buffer, when given)."""
    T, H = kp.T, kp.H
    if k_out is None:
        k_out = torch.empty(T, H, D, dtype=torch.bfloat16, device=kp.codes.device)
    if v_out is None:
        v_out = torch.empty(T, H, D, dtype=torch.bfloat16, device=kp.codes.device)
    for o in (k_out, v_out):
        if o.dtype != torch.bfloat16 or tuple(o.shape) != (T, H, D) or o.stride(2) != 1:
            raise ValueError("decode outputs must be [T, H, 128] bf16 with contiguous rows")
    if k_out.stride() != v_out.stride():
        raise ValueError("decode outputs must share strides")
    seg = _segment(kp, vp, kc, vc, U)
    check(lib.qwm_decode_segment(C.byref(seg), H, _ptr(k_out), _ptr(v_out), k_out.stride(0), k_out.stride(1),
                                 _stream()))
    return k_out, v_out


class SegmentArray:
    """Host array of segment descriptors for attention (the library validates
    them, sums their keys and copies them to the device itself).  `segments`:
    list of (k: PackedChunk, v: PackedChunk, k_centroids, v_centroids, U or None).
    Keep the chunks alive while the array is in use."""

    def __init__(self, segments):
        self.n = len(segments)
        self.arr = (Segment * max(self.n, 1))()
        self.total = 0
        for i, (kp, vp, kc, vc, U) in enumerate(segments):
            self.arr[i] = _segment(kp, vp, kc, vc, U)
            self.total += kp.T

    def ptr(self):
        return C.cast(self.arr, C.c_void_p) if self.n else C.c_void_p(0)


def segment_array(segments) -> SegmentArray:
    return SegmentArray(segments)


def attention(q: torch.Tensor, segs: SegmentArray | None, scale: float | None = None,
              want_lse: bool = False, want_top1: bool = False, active: tuple | None = None):
    """out [Tq, H, 128] fp32 (+ lse [H, Tq], top1 [H, Tq] int32).  `active`:
    (K, V) of the BF16 active chunk, [Ta, H, 128] bf16 each (segs may then be
    None)."""
    td = _tokens(q)
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    n_segs = 0 if segs is None else segs.n
    total = 0 if segs is None else segs.total
    sp = C.c_void_p(0) if segs is None else segs.ptr()
    out = torch.empty(td.T, td.H, D, dtype=torch.float32, device=q.device)
    lse = torch.empty(td.H, td.T, dtype=torch.float32, device=q.device) if want_lse else None
    top1 = torch.empty(td.H, td.T, dtype=torch.int32, device=q.device) if want_top1 else None
    if active is None:
        ws, nb = _WS.get(lib.qwm_workspace_bytes(QWM_OP_ATTENTION, total, td.H, td.T, n_segs), q.device)
        check(lib.qwm_attention(C.byref(td), sp, n_segs, C.c_float(scale),
                                _ptr(out), _ptr(lse), _ptr(top1), ws, nb, _stream()))
    else:
        ka, va = _tokens(active[0]), _tokens(active[1])
        ws, nb = _WS.get(lib.qwm_workspace_bytes(QWM_OP_ATTENTION_ACTIVE, total + ka.T, td.H, td.T, n_segs),
                         q.device)
        check(lib.qwm_attention_active(C.byref(td), sp, n_segs, C.byref(ka), C.byref(va),
                                       C.c_float(scale), _ptr(out), _ptr(lse), _ptr(top1), ws, nb, _stream()))
    return out, lse, top1


def attention_merge(out_a: torch.Tensor, lse_a: torch.Tensor, out_b: torch.Tensor, lse_b: torch.Tensor,
                    out: torch.Tensor | None = None, want_lse: bool = False):
    """Log-sum-exp merge of two attention results over disjoint key sets:
    out [Tq, H, 128] fp32 (+ lse [H, Tq])."""
    Tq, H = out_a.shape[0], out_a.shape[1]
    for t in (out_a, out_b):
        if t.dtype != torch.float32 or tuple(t.shape) != (Tq, H, D) or not t.is_contiguous():
            raise ValueError("outputs must be contiguous [Tq, H, 128] float32")
    for t in (lse_a, lse_b):
        if t.dtype != torch.float32 or tuple(t.shape) != (H, Tq) or not t.is_contiguous():
            raise ValueError("lse must be contiguous [H, Tq] float32")
    if out is None:
        out = torch.empty_like(out_a)
    lse = torch.empty(H, Tq, dtype=torch.float32, device=out_a.device) if want_lse else None
    check(lib.qwm_attention_merge(_ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), Tq, H, _ptr(out), _ptr(lse),
                                  _stream()))
    return out, lse


def reference_top1(q: torch.Tensor, k: torch.Tensor) -> torch.Tensor:
    """top1 [H, Tq] int32: argmax over all keys k [Tk, H, 128] (bf16) of q . k."""
    tq, tk = _tokens(q), _tokens(k)
    top1 = torch.empty(tq.H, tq.T, dtype=torch.int32, device=q.device)
    check(lib.qwm_reference_top1(C.byref(tq), C.byref(tk), _ptr(top1), _stream()))
    return top1
