"""QSAC Key quantization, INT2 residual codec, PSAC coefficients and Value
quantization (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows QuantWM (arXiv 2609.26425 v2) and the rainbus digest of it:
  * affine b-bit code with scale s and zero-point z shared by a group
    (preliminaries "低比特KV缓存量化"; v2 Sec. 2), here b = 2, groups of 64
    channels (method step (2)), codes packed four per byte, uint8 centroid
    index, INT2 zero-points (method step (3); App. D.1);
  * QSAC (Sec. 4.1; method section ¶2 and step (2)): Query-aware distance
    d_Q(k, mu) = sum_c w_c (k_c - mu_c)^2, keep the top-M candidates, score each
    by S = sum_g (sum_{c in g} w_c) R_g^2 with R_g the dynamic range of the
    residual in group g, take the minimum.  Nearest-centroid assignment is the
    sensitivity-free special case;
  * PSAC (Sec. 4.2; method step (4)): E = K - K0_hat, C = E U_r stored in
    INT8, K_hat = K0_hat + C U_r^T;
  * Values: nearest centroid plus the INT2 residual, no compensation.

Readings where the pages leave a step open (all deliberate):
  * r = fl32(k - mu) (float32 subtraction);
  * R_g = max(0, max r) - min(0, min r), so the coded interval always holds 0
    (integer zero-points);
  * s_g = smallest fp16 h with 3h >= R_g; z_g = rne(-lo_g / s_g) clamped to
    [0, 3]; q_c = clamp(rne(r_c / s_g) + z_g, 0, 3), with rne the round-half-
    to-even of the exact quotient; s_g = 0 gives z = q = 0;
  * M candidates ordered by (d_Q, index); final choice by (S, index);
  * C is computed against the stored bf16 basis; one fp16 scale per token:
    c_s = smallest fp16 h with 127h >= max_j |C_j|, C_q = clamp(rne(C / c_s),
    -127, 127), c_s = 0 gives C_q = 0.
"""
from __future__ import annotations

import numpy as np

from .formats import (bf16_rne, fp16_up_div, rne_quotient, pack_codes, pack_zeros,
                      fp16_bits)

GROUP = 64
QSAC = 1
PSAC = 2
PSAC_KEEP = 4   # the PSAC keep test (QuantWM method step (4))
QSAC_FULL = 8   # QSAC candidates by the full Query second-moment matrix (QuantWM App. C.4 ablation)


def weighted_dists(K: np.ndarray, C: np.ndarray, w: np.ndarray, block: int = 64) -> np.ndarray:
    """d_Q [T][n_c] = sum_c w_c (k_c - mu_c)^2 in float64 (direct form)."""
    K = np.asarray(K, np.float64)
    C = np.asarray(C, np.float64)
    w = np.asarray(w, np.float64)
    out = np.empty((K.shape[0], C.shape[0]))
    for s in range(0, K.shape[0], block):
        diff = K[s:s + block, None, :] - C[None, :, :]
        out[s:s + block] = np.sum(diff * diff * w, axis=2)
    return out


def full_dists(K: np.ndarray, C: np.ndarray, Mq: np.ndarray, block: int = 32) -> np.ndarray:
    """d_full [T][n_c] = (k - mu)^T Mq (k - mu) in float64, direct form: the
    quadratic form that the full-matrix ablation of QSAC (QuantWM App. C.4)
    puts in place of the diagonal-weighted distance."""
    K = np.asarray(K, np.float64)
    C = np.asarray(C, np.float64)
    Mq = np.asarray(Mq, np.float64)
    out = np.empty((K.shape[0], C.shape[0]))
    for s in range(0, K.shape[0], block):
        diff = K[s:s + block, None, :] - C[None, :, :]
        out[s:s + block] = np.sum((diff @ Mq) * diff, axis=2)
    return out


def second_moment(S: np.ndarray, n: int) -> np.ndarray:
    """M_h = S_h / n_h, the mean of q q^T (identity before any Query, the
    cold start's w = 1)."""
    S = np.asarray(S, np.float64)
    return S / float(n) if n > 0 else np.eye(S.shape[0])


def residual(k32: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """r = fl32(k - mu), element-wise float32 subtraction."""
    return np.asarray(k32, np.float32) - np.asarray(mu, np.float32)


def group_ranges(r: np.ndarray):
    """lo_g = min(0, min r), hi_g = max(0, max r), R_g = hi_g - lo_g (exact in float64).
    r [..., d] -> arrays [..., G]."""
    G = r.shape[-1] // GROUP
    rg = np.asarray(r, np.float64).reshape(r.shape[:-1] + (G, GROUP))
    lo = np.minimum(0.0, rg.min(axis=-1))
    hi = np.maximum(0.0, rg.max(axis=-1))
    return lo, hi, hi - lo


def qsac_score(R: np.ndarray, W: np.ndarray) -> np.ndarray:
    """S = sum_g W_g R_g^2 (float64)."""
    return np.sum(W * R * R, axis=-1)


def encode_residual(r: np.ndarray):
    """INT2 codec of residuals r [T][d] (float32 values).

    Returns codes q [T][d] (0..3), scales s [T][G] (fp16 values), zero-points
    z [T][G] (0..3), the dequantized residual r_hat [T][d] and a count of
    saturated scales.
    """
    T, d = r.shape
    G = d // GROUP
    lo, hi, R = group_ranges(r)
    s, sat = fp16_up_div(R, 3.0)
    zero = s == 0.0
    s_safe = np.where(zero, 1.0, s)
    z = np.clip(rne_quotient(-lo, s_safe), 0, 3)
    z = np.where(zero, 0, z)
    rg = np.asarray(r, np.float64).reshape(T, G, GROUP)
    qq = rne_quotient(rg, s_safe[..., None]) + z[..., None]
    qq = np.clip(qq, 0, 3)
    qq = np.where(zero[..., None], 0, qq)
    r_hat = s[..., None] * (qq - z[..., None])
    return (qq.reshape(T, d).astype(np.uint8), s, z.astype(np.uint8),
            r_hat.reshape(T, d), int(np.sum(sat)))


def psac_coefficients(E: np.ndarray, U_bf16: np.ndarray):
    """C = E U (float64, against the stored bf16 basis), then symmetric INT8 with
    one fp16 scale per token.  Returns (C_q int8 [T][r], c_s [T], C float64)."""
    C = np.asarray(E, np.float64) @ np.asarray(U_bf16, np.float64)
    m = np.max(np.abs(C), axis=1)
    cs, _ = fp16_up_div(m, 127.0)
    zero = cs == 0.0
    cs_safe = np.where(zero, 1.0, cs)
    Cq = np.clip(rne_quotient(C, cs_safe[:, None]), -127, 127)
    Cq = np.where(zero[:, None], 0, Cq)
    return Cq.astype(np.int8), cs, C


def psac_keep(E: np.ndarray, Cq: np.ndarray, cs: np.ndarray, U_bf16: np.ndarray, w: np.ndarray):
    """PSAC keep test (QuantWM method step (4)): a token keeps its coefficients
    only if the compensation lowers its Query-weighted error
    sum_c w_c e_c^2, i.e. iff sum_c w_c D_c (D_c - 2 E_c) < 0 with
    D = (c_s C_q) U^T (the difference of the errors with and without it).
    Returns (keep [T] bool, that criterion [T], sum_c w_c E_c^2 [T])."""
    E = np.asarray(E, np.float64)
    Dm = (np.asarray(cs, np.float64)[:, None] * np.asarray(Cq, np.float64)) @ np.asarray(U_bf16, np.float64).T
    w = np.asarray(w, np.float64)
    crit = np.sum(w * Dm * (Dm - 2.0 * E), axis=1)
    return crit < 0.0, crit, np.sum(w * E * E, axis=1)


def select_qsac(K: np.ndarray, C: np.ndarray, w: np.ndarray, M: int, Mq: np.ndarray | None = None):
    """QSAC: top-M candidates by (d_Q, j), then argmin by (S, j).

    With Mq (the full Query second-moment matrix, App. C.4 ablation) the
    candidates come from the quadratic form (k - mu)^T Mq (k - mu) instead of
    d_Q; the score S keeps the diagonal weights w (the rest of the pipeline is
    unchanged in that ablation).

    Returns idx [T] and the per-token score table used (for diagnostics):
    dict(dq [T][n_c], cand [T][M], S [T][M]).
    """
    K = np.asarray(K)
    dq = weighted_dists(K, C, w) if Mq is None else full_dists(K, C, Mq)
    cand = np.argsort(dq, axis=1, kind="stable")[:, :M]
    W = np.asarray(w, np.float64).reshape(-1, GROUP).sum(axis=1)
    k32 = np.asarray(K, np.float32)
    C32 = np.asarray(C, np.float32)
    S = np.empty(cand.shape)
    for m in range(M):
        r = k32 - C32[cand[:, m]]
        _, _, R = group_ranges(r)
        S[:, m] = qsac_score(R, W)
    # argmin by (S, j): lexsort sorts by the last key first
    idx = np.empty(K.shape[0], np.int64)
    for t in range(K.shape[0]):
        order = np.lexsort((cand[t], S[t]))
        idx[t] = cand[t, order[0]]
    return idx, {"dq": dq, "cand": cand, "S": S}


def select_nearest(X: np.ndarray, C: np.ndarray):
    """argmin_j (||x - mu_j||^2, j) in float64."""
    d = weighted_dists(X, C, np.ones(X.shape[1]))
    return np.argmin(d, axis=1), d


def quantize_keys(K: np.ndarray, C: np.ndarray, w: np.ndarray | None, U_bf16: np.ndarray | None,
                  M: int = 8, flags: int = QSAC | PSAC, Mq: np.ndarray | None = None) -> dict:
    """One head: K [T][d] (bf16- or fp32-valued), centroid table C [n_c][d]
    (bf16-valued), w [d] float32 or None (w = 1), U_bf16 [d][r] or None (no PSAC).

    flags & QSAC: QSAC choice with weights w (w = 1 when None); otherwise the
    nearest centroid (w is then ignored).  flags & PSAC with a basis: PSAC
    coefficients; otherwise C = 0.  flags & PSAC_KEEP: the keep test drops the
    coefficients (C = 0, c_s = 0) of tokens they do not help, with the channel
    weights of the centroid choice (w under QSAC, else 1).  flags & QSAC_FULL
    (with QSAC): candidates by the full matrix Mq [d][d] (second_moment()).
    """
    K = np.asarray(K, np.float64)
    T, d = K.shape
    if flags & QSAC:
        ww = np.ones(d, np.float32) if w is None else np.asarray(w, np.float32)
        if flags & QSAC_FULL:
            if Mq is None:
                raise ValueError("QSAC_FULL needs the second-moment matrix Mq")
            idx, info = select_qsac(K, C, ww, M, Mq=Mq)
        else:
            idx, info = select_qsac(K, C, ww, M)
    else:
        idx, dq = select_nearest(K, C)
        info = {"dq": dq}
    r = residual(K, np.asarray(C)[idx])
    q, s, z, r_hat, n_sat = encode_residual(r)
    r_rank = 8 if U_bf16 is None else U_bf16.shape[1]
    keep_info = None
    if (flags & PSAC) and U_bf16 is not None:
        E = K - (np.asarray(C, np.float64)[idx] + r_hat)
        Cq, cs, Craw = psac_coefficients(E, U_bf16)
        if flags & PSAC_KEEP:
            wk = np.ones(d) if (w is None or not (flags & QSAC)) else np.asarray(w, np.float32).astype(np.float64)
            keep, crit, base = psac_keep(E, Cq, cs, U_bf16, wk)
            Cq = np.where(keep[:, None], Cq, 0).astype(np.int8)
            cs = np.where(keep, cs, 0.0)
            keep_info = {"keep": keep, "crit": crit, "base": base}
    else:
        Cq = np.zeros((T, r_rank), np.int8)
        cs = np.zeros(T)
        Craw = None
    return {"idx": idx.astype(np.uint8), "q": q, "scale": s, "zero": z, "r_hat": r_hat,
            "Cq": Cq, "c_scale": cs, "C_raw": Craw, "info": info, "saturated": n_sat, "keep": keep_info,
            # packed storage
            "codes": pack_codes(q), "zeros": pack_zeros(z),
            "scale_bits": fp16_bits(s), "c_scale_bits": fp16_bits(cs)}


def quantize_values(V: np.ndarray, C: np.ndarray) -> dict:
    """One head: nearest centroid + INT2 residual, no compensation."""
    V = np.asarray(V, np.float64)
    idx, dq = select_nearest(V, C)
    r = residual(V, np.asarray(C)[idx])
    q, s, z, r_hat, n_sat = encode_residual(r)
    return {"idx": idx.astype(np.uint8), "q": q, "scale": s, "zero": z, "r_hat": r_hat,
            "info": {"dq": dq}, "saturated": n_sat,
            "codes": pack_codes(q), "zeros": pack_zeros(z), "scale_bits": fp16_bits(s)}


def dequant_keys(idx, q, s, z, Cq, cs, C, U_bf16) -> np.ndarray:
    """K_hat = mu_idx + s (q - z) + (c_s C_q) U^T, exact in float64."""
    K0 = dequant_values(idx, q, s, z, C)
    if U_bf16 is None:
        return K0
    Chat = np.asarray(cs, np.float64)[:, None] * np.asarray(Cq, np.float64)
    return K0 + Chat @ np.asarray(U_bf16, np.float64).T


def dequant_values(idx, q, s, z, C) -> np.ndarray:
    T = len(idx)
    d = np.asarray(C).shape[1]
    G = d // GROUP
    mu = np.asarray(C, np.float64)[np.asarray(idx, np.int64)]
    qq = np.asarray(q, np.float64).reshape(T, G, GROUP)
    rh = np.asarray(s, np.float64)[..., None] * (qq - np.asarray(z, np.float64)[..., None])
    return mu + rh.reshape(T, d)


def bf16_table(C) -> np.ndarray:
    return bf16_rne(C)
