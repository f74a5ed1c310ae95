"""Progressive residual quantization, QVG's codec (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

QVG, the prior art QuantWM builds on, first subtracts cluster centroids from
the tokens, which leaves small residuals centred on zero (Semantic-Aware
Smoothing, QVG summary Sec. 2A), then quantizes that residual over several
coarse-to-fine stages, each one working on what the previous stage left, and
stores only every stage's centroids and codes (Progressive Residual
Quantization, Sec. 2B).

Reading (the summary fixes no further detail): stage s = 1 .. S-1 clusters
the current residual e^{s-1} (e^0 = the tokens) into 256 bf16 centroids by
seeded Lloyd (seed + s - 1), gives each token its nearest centroid a^s and
leaves e^s = fl32(e^{s-1} - C^s[a^s]); the last stage codes e^{S-1} as a
Value chunk is coded: its own Lloyd table, nearest centroid, INT2 residual.
S = 1 is QuantWM's nearest-centroid codec.  The reconstruction sums every
stage's centroid and the last stage's dequantized residual.
"""
from __future__ import annotations

import numpy as np

from .lloyd import assign, lloyd
from .quantize import dequant_values, quantize_values, residual


def prq_quantize(X: np.ndarray, stages: int, iters: int, seed: int, head: int = 0):
    """One head, tokens X [T][d].  Returns (list of (C^s, a^s) for the first
    S - 1 stages, C^S, the last stage's value codes, e^{S-1})."""
    e = np.asarray(X, np.float32)
    first = []
    for s in range(stages - 1):
        C = lloyd(e.astype(np.float64), 256, iters, seed=seed + s, head=head)
        a = assign(e.astype(np.float64), C)
        first.append((C, a.astype(np.uint8)))
        e = residual(e, C[a])
    C_last = lloyd(e.astype(np.float64), 256, iters, seed=seed + stages - 1, head=head)
    last = quantize_values(e.astype(np.float64), C_last)
    return first, C_last, last, e


def prq_reconstruct(first, C_last, last) -> np.ndarray:
    """Sum of every stage's centroid plus the last stage's dequantized residual, float64."""
    X = dequant_values(last["idx"], last["q"], last["scale"], last["zero"], C_last)
    for C, a in first:
        X = X + np.asarray(C, np.float64)[np.asarray(a, np.int64)]
    return X
