"""Refinements of the stored format (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Three storage refinements of QuantWM's packed cache:

  * the per-chunk choice between a dense and a sparse layout of the PSAC
    coefficients, sparse indices included (QuantWM v2 App. D.1);
  * group scales stored as INT8 codes under an FP16 second-level scale
    (rainbus digest, method step (3): "组缩放INT8+FP16二级缩放");
  * the keep test of the coefficients with the full Query second moment:
    they stay only if they lower the Query-weighted error e^T M_h e (method
    step (4), and the method section's objective e^T M_h e).

Readings (the pages give the ingredients, not the byte layout):

  Sparse layout, per (chunk, head): a key keeps coefficients iff its
  coefficient scale is nonzero.  A bitmap with one bit per key (64-key
  words, key 64 w + b at bit b of word w), the number of kept keys before
  each word (u32), then the kept keys' INT8 rows and fp16 scales in key
  order.  Dense: every key's row and scale.  Each section starts on a
  16-byte boundary.  The chunk keeps whichever is smaller (dense on a tie).

  Two-level scales, per (chunk, head, group g): the second-level scale s2_g
  is the smallest power of two p (at least 2^-24, the smallest fp16 step)
  with 255 p >= max_t s_{t,g}, the group's largest fp16 step; each token's
  code is q = ceil(s / s2_g), at most 255 and never past 65504 / s2_g; the
  effective step is q s2_g.  A power of two keeps every effective step an
  exact fp16 value (q has at most 8 significant bits), so dequantization and
  the exact-quotient code decisions stay exact; rounding the code up keeps
  the coded interval covering the residual range.  The residual codes,
  zero-points and the PSAC error are then those of the effective step.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import FP16_MAX, rne_quotient

WORD = 64          # keys per bitmap word
ALIGN = 16         # byte alignment of every section


def _al(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


def dense_bytes(T: int, r: int) -> int:
    return _al(T * r) + _al(T * 2)


def sparse_bytes(T: int, count: int, r: int) -> int:
    nw = (T + WORD - 1) // WORD
    return _al(nw * 8) + _al(nw * 4) + _al(count * r) + _al(count * 2)


def choose_layout(T: int, count: int, r: int) -> str:
    return "sparse" if sparse_bytes(T, count, r) < dense_bytes(T, r) else "dense"


def pack_coefficients(Cq: np.ndarray, cs_bits: np.ndarray) -> dict:
    """One (chunk, head)'s coefficients in the chosen layout.  Cq [T][r] int8,
    cs_bits [T] uint16 (fp16 bits).  Returns layout, count, bytes and the
    sections (bitmap, prefix for the sparse layout; c, cs)."""
    Cq = np.asarray(Cq, np.int8)
    cs_bits = np.asarray(cs_bits, np.uint16)
    T, r = Cq.shape
    kept = cs_bits != 0
    count = int(kept.sum())
    layout = choose_layout(T, count, r)
    if layout == "dense":
        return {"layout": layout, "count": count, "bytes": dense_bytes(T, r), "c": Cq.copy(), "cs": cs_bits.copy()}
    nw = (T + WORD - 1) // WORD
    bitmap = np.zeros(nw, np.uint64)
    for t in np.nonzero(kept)[0]:
        bitmap[t // WORD] |= np.uint64(1) << np.uint64(t % WORD)
    per_word = np.array([int(kept[w * WORD:(w + 1) * WORD].sum()) for w in range(nw)], np.int64)
    prefix = np.concatenate([[0], np.cumsum(per_word)[:-1]]).astype(np.uint32)
    return {"layout": layout, "count": count, "bytes": sparse_bytes(T, count, r), "bitmap": bitmap,
            "prefix": prefix, "c": Cq[kept].copy(), "cs": cs_bits[kept].copy()}


def unpack_coefficients(p: dict, T: int, r: int):
    """Dense (Cq [T][r], cs_bits [T]) from either layout: dropped keys read as
    zero coefficients with a zero scale."""
    if p["layout"] == "dense":
        return np.asarray(p["c"], np.int8), np.asarray(p["cs"], np.uint16)
    Cq = np.zeros((T, r), np.int8)
    cs = np.zeros(T, np.uint16)
    for t in range(T):
        w, b = divmod(t, WORD)
        word = int(p["bitmap"][w])
        if (word >> b) & 1:
            e = int(p["prefix"][w]) + bin(word & ((1 << b) - 1)).count("1")
            Cq[t] = p["c"][e]
            cs[t] = p["cs"][e]
    return Cq, cs


def second_level_scale(m: float) -> float:
    """Smallest power of two p >= 2^-24 with 255 p >= m (m >= 0 the group's largest step)."""
    if m <= 0.0:
        return 0.0
    e = max(-24, math.ceil(math.log2(m / 255.0)))
    while 255.0 * math.ldexp(1.0, e) < m:      # guard the float log
        e += 1
    while e > -24 and 255.0 * math.ldexp(1.0, e - 1) >= m:
        e -= 1
    return math.ldexp(1.0, e)


def two_level_scales(s: np.ndarray):
    """Group steps s [T][G] (fp16 values) -> (codes q [T][G] uint8, second-level
    scales s2 [G], effective steps q s2 [T][G])."""
    s = np.asarray(s, np.float64)
    T, G = s.shape
    q = np.zeros((T, G), np.int64)
    s2 = np.zeros(G)
    for g in range(G):
        p = second_level_scale(float(s[:, g].max()) if T else 0.0)
        s2[g] = p
        if p > 0.0:
            qq = np.ceil(s[:, g] / p)                 # exact: p is a power of two
            q[:, g] = np.minimum(qq, math.floor(FP16_MAX / p)).astype(np.int64)
    return q.astype(np.uint8), s2, q * s2[None, :]


def encode_with_steps(r: np.ndarray, steps: np.ndarray):
    """INT2 codes of residuals r [T][d] with given group steps [T][G] (the
    codec of the packed format with the step fixed): z = clamp(rne(-lo/s), 0, 3),
    q = clamp(rne(r/s) + z, 0, 3); a zero step codes the group as zeros.
    Returns (q [T][d], z [T][G], r_hat [T][d])."""
    from .quantize import group_ranges, GROUP
    T, d = r.shape
    G = d // GROUP
    lo, _, _ = group_ranges(r)
    s = np.asarray(steps, np.float64)
    zero = s == 0.0
    s_safe = np.where(zero, 1.0, s)
    z = np.where(zero, 0, np.clip(rne_quotient(-lo, s_safe), 0, 3))
    rg = np.asarray(r, np.float64).reshape(T, G, GROUP)
    qq = np.clip(rne_quotient(rg, s_safe[..., None]) + z[..., None], 0, 3)
    qq = np.where(zero[..., None], 0, qq)
    r_hat = s[..., None] * (qq - z[..., None])
    return qq.reshape(T, d).astype(np.uint8), z.astype(np.uint8), r_hat.reshape(T, d)


def psac_keep_full(E: np.ndarray, Cq: np.ndarray, cs: np.ndarray, U_bf16: np.ndarray, Mq: np.ndarray):
    """The keep test with the full Query second moment M (method step (4)):
    keep iff (e - D)^T M (e - D) < e^T M e, D = (c_s C_q) U^T.  Returns
    (keep [T], error after, error before)."""
    E = np.asarray(E, np.float64)
    Dm = (np.asarray(cs, np.float64)[:, None] * np.asarray(Cq, np.float64)) @ np.asarray(U_bf16, np.float64).T
    Mq = np.asarray(Mq, np.float64)
    before = np.einsum("tc,cd,td->t", E, Mq, E)
    A = E - Dm
    after = np.einsum("tc,cd,td->t", A, Mq, A)
    return after < before, after, before


def requantize_two_level(X: np.ndarray, C: np.ndarray, base: dict, U_bf16=None, w=None, flags: int = 3):
    """Two-level form of one head's chunk from its single-level result `base`
    (quantize_keys / quantize_values: the centroid choice and the fp16 steps
    are kept).  X [T][d], C [n_c][d] bf16-valued.  For keys (U_bf16 given and
    the PSAC flag set) the coefficients are those of the new error E =
    X - (mu + r_hat), with the diagonal keep test under PSAC_KEEP (weights w
    under QSAC, else 1)."""
    from .quantize import residual, psac_coefficients, psac_keep, QSAC, PSAC, PSAC_KEEP
    from .formats import pack_codes, pack_zeros, fp16_bits
    X = np.asarray(X, np.float64)
    idx = np.asarray(base["idx"], np.int64)
    mu = np.asarray(C, np.float64)[idx]
    r = residual(X, mu)
    q_s, s2, steps = two_level_scales(base["scale"])
    q, z, r_hat = encode_with_steps(r, steps)
    out = {"idx": base["idx"], "q": q, "zero": z, "scale_q": q_s, "scale2": s2, "steps": steps, "r_hat": r_hat,
           "codes": pack_codes(q), "zeros": pack_zeros(z), "scale2_bits": fp16_bits(s2)}
    T = X.shape[0]
    if U_bf16 is not None and (flags & PSAC):
        E = X - (mu + r_hat)
        Cq, cs, Craw = psac_coefficients(E, U_bf16)
        if flags & PSAC_KEEP:
            wk = np.ones(X.shape[1]) if (w is None or not (flags & QSAC)) else np.asarray(w, np.float32).astype(np.float64)
            keep, _, _ = psac_keep(E, Cq, cs, U_bf16, wk)
            Cq = np.where(keep[:, None], Cq, 0).astype(np.int8)
            cs = np.where(keep, cs, 0.0)
        out.update(Cq=Cq, c_scale=cs, c_scale_bits=fp16_bits(cs), E=E)
    elif "Cq" in base:
        rr = base["Cq"].shape[1]
        out.update(Cq=np.zeros((T, rr), np.int8), c_scale=np.zeros(T), c_scale_bits=np.zeros(T, np.uint16))
    return out
