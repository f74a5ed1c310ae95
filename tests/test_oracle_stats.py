"""Pins of the oracle's Query statistics and principal basis: the expected-
perturbation identity, a library eigensolver, closed forms of the synthetic
spectrum."""
import numpy as np
import pytest

import datagen
from oracle import stats
from oracle.formats import bf16_rne


def test_second_moment_identity():
    """E_Q[(q^T e)^2] = e^T M e for the running mean M (QuantWM's sensitivity identity)."""
    rng = np.random.default_rng(0)
    Q1 = rng.standard_normal((50, 128))
    Q2 = rng.standard_normal((70, 128)) * 2
    S, n = stats.update(np.zeros((128, 128)), 0, Q1)
    S, n = stats.update(S, n, Q2)
    assert n == 120
    M = S / n
    allq = np.concatenate([Q1, Q2])
    for _ in range(5):
        e = rng.standard_normal(128)
        direct = np.mean([(q @ e) ** 2 for q in allq])
        assert abs(direct - e @ M @ e) <= 1e-12 * direct


def test_channel_weights_diag_and_cold_start():
    rng = np.random.default_rng(1)
    Q = rng.standard_normal((33, 128))
    S, n = stats.update(np.zeros((128, 128)), 0, Q)
    w = stats.channel_weights(S, n)
    assert w.dtype == np.float32
    want = np.array([np.mean(Q[:, c] ** 2) for c in range(128)])
    np.testing.assert_allclose(w, want, rtol=1e-7)
    np.testing.assert_array_equal(stats.channel_weights(np.zeros((128, 128)), 0), np.ones(128))


@pytest.mark.parametrize("seed", [0, 1])
def test_jacobi_matches_lapack(seed):
    rng = np.random.default_rng(seed)
    n = 40
    B = rng.standard_normal((n, n))
    A = B @ B.T + np.diag(np.arange(n))
    lam, V = stats.jacobi_eigh(A)
    order = np.argsort(lam)
    lam, V = lam[order], V[:, order]
    ref_l, ref_V = np.linalg.eigh(A)
    np.testing.assert_allclose(lam, ref_l, rtol=1e-12, atol=1e-12 * np.abs(ref_l).max())
    dots = np.abs(np.sum(V * ref_V, axis=0))
    np.testing.assert_allclose(dots, 1.0, atol=1e-10)
    assert np.linalg.norm(A @ V - V * lam) <= 1e-12 * np.linalg.norm(A)
    assert np.linalg.norm(V.T @ V - np.eye(n)) <= 1e-12
    assert abs(lam.sum() - np.trace(A)) <= 1e-12 * abs(np.trace(A))


def test_jacobi_diagonal_gives_unit_vectors():
    d = np.array([3.0, 1.0, 7.0, 2.0])
    lam, V = stats.jacobi_eigh(np.diag(d))
    np.testing.assert_array_equal(lam, d)
    np.testing.assert_array_equal(V, np.eye(4))


def test_principal_basis_order_sign_energy():
    """A matrix with a known eigen-basis: order by eigenvalue, sign rule, bf16 copy."""
    rng = np.random.default_rng(2)
    Uh = datagen.haar_orthogonal(rng, 128)
    lam = datagen.query_spectrum(0.65)
    n = 1000
    S = (Uh * lam) @ Uh.T * n
    out = stats.principal_basis(S, n, r=8)
    np.testing.assert_allclose(out["lam"], lam[:8], rtol=1e-10)
    for j in range(8):
        u = out["U"][:, j]
        assert abs(abs(u @ Uh[:, j]) - 1.0) < 1e-9
        i = np.argmax(np.abs(u))
        assert u[i] > 0
    np.testing.assert_array_equal(out["U_bf16"], bf16_rne(out["U"]))
    # energy of the geometric spectrum equals its closed form (1 - rho^8)/(1 - rho^128)
    assert abs(out["energy"] - 0.65) < 1e-9
    with pytest.raises(ValueError):
        stats.principal_basis(np.zeros((128, 128)), 0)


def test_principal_basis_sample_energy_in_pages_band():
    """Sample second moment of generated Queries keeps ~the requested top-8 share."""
    w = datagen.make_workload("tiny", n_queries=4096)
    S, n = stats.update(np.zeros((128, 128)), 0, w.Q[:, 0])
    e = np.linalg.eigvalsh(S / n)[::-1]
    frac = e[:8].sum() / e.sum()
    assert 0.60 < frac < 0.71
