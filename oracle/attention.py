"""Attention over the compressed cache, and top-1 token selection (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Attention logits L = Q K^T / sqrt(d); a Key error e perturbs them by
Q e^T / sqrt(d) (rainbus digest "注意力logits与时空token选择"; QuantWM v2
Sec. 3.3).  PSAC restores the Key error along the principal Query subspace,
so logits = Q K0_hat^T + (Q U_r) C^T (digest, method section ¶1), i.e. the
attention reads K_hat = K0_hat + C U_r^T.  Every Query attends to every key of
every cached chunk (no mask).  The top-1 token of a Query is the argmax of its
logits; the shift ratio compares it between the quantized and the original
bf16 Keys (Sec. 5.3).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_rne
from .quantize import dequant_keys, dequant_values


def softmax_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Float64 softmax(scale * Q K^T) V with max subtraction.

    Returns (O [Tq][d], lse [Tq] = log sum_j exp(scale * l_j), top1 [Tq]).
    """
    Q = np.asarray(Q, np.float64)
    L = Q @ np.asarray(K, np.float64).T
    top1 = np.argmax(L, axis=1)
    Z = scale * L
    m = Z.max(axis=1, keepdims=True)
    P = np.exp(Z - m)
    s = P.sum(axis=1, keepdims=True)
    O = (P / s) @ np.asarray(V, np.float64)
    lse = (m + np.log(s))[:, 0]
    return O, lse, top1


def segment_kv(seg: dict):
    """Dequantize one cached chunk of one head.  seg holds the per-head arrays:
    k_idx, k_q, k_scale, k_zero, k_Cq, k_cs, k_centroids, U (or None),
    v_idx, v_q, v_scale, v_zero, v_centroids.

    A BF16 chunk (the active chunk, kept unquantized until it completes:
    QuantWM App. D.1) holds k_bf16 and v_bf16 instead, [T][d] arrays of its
    bf16 values; attention reads them as they are."""
    if "k_bf16" in seg:
        return np.asarray(seg["k_bf16"], np.float64), np.asarray(seg["v_bf16"], np.float64)
    K = dequant_keys(seg["k_idx"], seg["k_q"], seg["k_scale"], seg["k_zero"],
                     seg["k_Cq"], seg["k_cs"], seg["k_centroids"], seg.get("U"))
    V = dequant_values(seg["v_idx"], seg["v_q"], seg["v_scale"], seg["v_zero"],
                       seg["v_centroids"])
    return K, V


def decode_segment(seg: dict):
    """BF16 reconstruction of one packed chunk of one head, the decoder of
    QuantWM App. D.1 / Fig. 9: every element of K_hat and V_hat (exact in
    float64) rounded once to bf16, nearest-even."""
    K, V = segment_kv(seg)
    return bf16_rne(K), bf16_rne(V)


def cache_attention(Q: np.ndarray, segments: list, scale: float):
    """One head: Q [Tq][d] attends to the concatenation of all segments."""
    Ks, Vs = zip(*[segment_kv(s) for s in segments])
    return softmax_attention(Q, np.concatenate(Ks), np.concatenate(Vs), scale)


def top1(Q: np.ndarray, K: np.ndarray) -> np.ndarray:
    """argmax_j q . k_j (lowest j on ties), float64."""
    return np.argmax(np.asarray(Q, np.float64) @ np.asarray(K, np.float64).T, axis=1)


def shift_rate(top_a: np.ndarray, top_b: np.ndarray) -> float:
    """Fraction of Queries whose top-1 token differs."""
    top_a = np.asarray(top_a)
    return float(np.mean(top_a != np.asarray(top_b))) if top_a.size else 0.0
