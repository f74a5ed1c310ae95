"""Query statistics and the principal Query basis (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows QuantWM (arXiv 2609.26425 v2):
  * per head h the second moment of all previously seen Queries,
    M_h = (1/N) sum q q^T, kept incrementally without storing the Queries
    (rainbus digest "二阶Query统计与低秩分解"; App. D.1);
  * channel sensitivity w_{h,c} = (M_h)_{cc}, the diagonal approximation of
    E_Q[(q^T e)^2] = e^T M_h e (method section; App. C.4);
  * cold start: before any Query has been seen, w = 1 and there is no basis
    (method step (1); App. C.3);
  * M_h = U Lambda U^T, U_r = the top r = 8 eigenvectors, stored in BF16
    (Sec. 4.2; method step (4); Sec. 5.1).
The eigen-decomposition is a cyclic Jacobi iteration in float64.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import bf16_rne


def update(S: np.ndarray, n: int, Q: np.ndarray):
    """S [d][d] float64 running sum of q q^T, n = Queries seen, Q [T][d].

    Returns (S + Q^T Q, n + T).  The products of bf16 / fp32 inputs are exact
    in float64; the sum is a plain float64 matrix product.
    """
    Q = np.asarray(Q, dtype=np.float64)
    return S + Q.T @ Q, n + Q.shape[0]


def channel_weights(S: np.ndarray, n: int) -> np.ndarray:
    """w_c = diag(S)/n rounded to float32 (w = 1 while n == 0)."""
    d = S.shape[0]
    if n == 0:
        return np.ones(d, np.float32)
    return (np.diag(S) / float(n)).astype(np.float32)


def jacobi_eigh(A: np.ndarray, tol: float = 1e-14, max_sweeps: int = 60):
    """Cyclic (row-by-row) Jacobi eigen-decomposition of a symmetric matrix.

    Each step zeroes one off-diagonal pair (p, q) with a plane rotation whose
    angle solves the 2x2 symmetric eigenproblem; sweeps repeat until the
    off-diagonal Frobenius norm is <= tol * ||A||_F.
    Returns (eigenvalues, eigenvectors as columns), unsorted.
    """
    A = np.array(A, dtype=np.float64, copy=True)
    n = A.shape[0]
    V = np.eye(n)
    normA = np.linalg.norm(A)
    if normA == 0.0:
        return np.zeros(n), V
    for _ in range(max_sweeps):
        off = np.linalg.norm(A - np.diag(np.diag(A)))
        if off <= tol * normA:
            break
        for p in range(n - 1):
            for q in range(p + 1, n):
                apq = A[p, q]
                if apq == 0.0:
                    continue
                theta = (A[q, q] - A[p, p]) / (2.0 * apq)
                if abs(theta) > 1e150:       # theta^2 would overflow: t ~ 1/(2 theta)
                    t = 0.5 / theta
                else:
                    t = (1.0 if theta >= 0 else -1.0) / (abs(theta) + math.sqrt(theta * theta + 1.0))
                c = 1.0 / math.sqrt(t * t + 1.0)
                s = t * c
                # A <- J^T A J with J = rotation in the (p, q) plane
                ap = A[:, p].copy()
                aq = A[:, q].copy()
                A[:, p] = c * ap - s * aq
                A[:, q] = s * ap + c * aq
                ap = A[p, :].copy()
                aq = A[q, :].copy()
                A[p, :] = c * ap - s * aq
                A[q, :] = s * ap + c * aq
                A[p, q] = A[q, p] = 0.0
                vp = V[:, p].copy()
                vq = V[:, q].copy()
                V[:, p] = c * vp - s * vq
                V[:, q] = s * vp + c * vq
    return np.diag(A).copy(), V


def principal_basis(S: np.ndarray, n: int, r: int = 8):
    """Top-r eigenpairs of M = S/n.

    Order: eigenvalues descending.  Sign: the largest-magnitude entry of each
    eigenvector (lowest index on ties) is made positive.
    Returns dict(U [d][r] float64, U_bf16 [d][r] bf16-valued float64,
                 lam [r], energy = sum(top r)/trace).
    """
    if n == 0:
        raise ValueError("no Queries seen yet: cold start has no basis")
    M = S / float(n)
    lam, V = jacobi_eigh(M)
    order = np.argsort(-lam, kind="stable")
    lam = lam[order]
    V = V[:, order]
    U = V[:, :r].copy()
    for j in range(r):
        i = int(np.argmax(np.abs(U[:, j])))
        if U[i, j] < 0:
            U[:, j] = -U[:, j]
    energy = float(np.sum(lam[:r]) / np.sum(lam))
    return {"U": U, "U_bf16": bf16_rne(U), "lam": lam[:r].copy(), "energy": energy,
            "lam_all": lam}
