"""Seeded Lloyd (k-means) centroid tables (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

QuantWM builds on QVG's centroid-residual representation: Keys (and Values)
are clustered with K-means into 256 centroids kept in BF16 (QuantWM v2 Sec. 2;
rainbus digest "质心-残差量化"; QVG summary Sec. 2A).  QVG starts each chunk's
k-means from the previous chunk's result (QVG summary Sec. 2C).

Readings: Forgy initialisation with 256 distinct tokens drawn by a partial
Fisher-Yates shuffle driven by SplitMix64 (Steele, Lea & Flood, OOPSLA 2014),
seeded with seed + (head << 32); Euclidean assignment with ties to the lowest
centroid index; new centroid = bf16(mean of its members), computed in float64;
an empty cluster keeps its centroid.

Tokens with a NaN or infinite channel take no part in the table: the
quantizers store them as index 0 with zero codes (a degenerate case the
pages leave open), so they are never Forgy picks (the shuffle goes on past
them; slots left without a finite token hold zeros) and never members of a
cluster.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_rne

_MASK64 = (1 << 64) - 1


class SplitMix64:
    """SplitMix64: a Weyl sequence with increment 0x9E3779B97F4A7C15 followed
    by the variant-13 mixing function (two xor-shift-multiply rounds and a final
    xor-shift)."""

    def __init__(self, seed: int):
        self.state = seed & _MASK64

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & _MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        return z ^ (z >> 31)


def forgy_indices(N: int, n_c: int, seed: int, head: int, finite=None) -> np.ndarray:
    """First n_c picks of a Fisher-Yates shuffle of range(N): pick i swaps slot i
    with slot i + (next() mod (N - i)).  With a boolean mask `finite`, picks of
    rows outside it are dropped and the shuffle goes on until n_c finite rows
    are picked or the range is exhausted; missing picks are -1."""
    if N < n_c:
        raise ValueError("fewer tokens than centroids")
    rng = SplitMix64(seed + (head << 32))
    perm = list(range(N))
    picks = []
    i = 0
    while len(picks) < n_c and i < N:
        j = i + rng.next() % (N - i)
        perm[i], perm[j] = perm[j], perm[i]
        if finite is None or finite[perm[i]]:
            picks.append(perm[i])
        i += 1
    picks += [-1] * (n_c - len(picks))
    return np.array(picks, dtype=np.int64)


def finite_rows(X: np.ndarray) -> np.ndarray:
    """Rows whose every channel is finite."""
    return np.all(np.isfinite(np.asarray(X, np.float64)), axis=1)


def sq_dists(X: np.ndarray, C: np.ndarray, block: int = 256) -> np.ndarray:
    """[N][n_c] squared Euclidean distances, direct form sum_c (x_c - mu_c)^2, float64."""
    X = np.asarray(X, np.float64)
    C = np.asarray(C, np.float64)
    out = np.empty((X.shape[0], C.shape[0]))
    for s in range(0, X.shape[0], block):
        diff = X[s:s + block, None, :] - C[None, :, :]
        out[s:s + block] = np.sum(diff * diff, axis=2)
    return out


def assign(X: np.ndarray, C: np.ndarray) -> np.ndarray:
    """Nearest centroid; np.argmin returns the lowest index among equal minima."""
    return np.argmin(sq_dists(X, C), axis=1)


def update_means(X: np.ndarray, a: np.ndarray, C: np.ndarray) -> np.ndarray:
    X = np.asarray(X, np.float64)
    out = np.array(C, dtype=np.float64, copy=True)
    for j in range(C.shape[0]):
        members = X[a == j]
        if members.shape[0] > 0:
            out[j] = bf16_rne(np.sum(members, axis=0) / members.shape[0])
    return out


def lloyd(X: np.ndarray, n_c: int = 256, iters: int = 10, seed: int = 0, head: int = 0,
          init: np.ndarray | None = None, return_history: bool = False):
    """Centroid table [n_c][d] (bf16-valued float64) after `iters` Lloyd iterations.

    init=None: Forgy seeding; otherwise warm start from the given table.
    """
    X = np.asarray(X, np.float64)
    fin = finite_rows(X)
    if init is None:
        idx = forgy_indices(X.shape[0], n_c, seed, head, finite=None if fin.all() else fin)
        C = np.zeros((n_c, X.shape[1]))
        C[idx >= 0] = bf16_rne(X[idx[idx >= 0]])
    else:
        C = np.array(init, dtype=np.float64, copy=True)
    Xf = X[fin]
    hist = []
    for _ in range(iters):
        a = assign(Xf, C)
        if return_history:
            hist.append((C.copy(), a.copy()))
        C = update_means(Xf, a, C)
    if return_history:
        return C, hist
    return C
