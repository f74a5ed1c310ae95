"""Pins of the oracle's QSAC choice, INT2 codec and PSAC coefficients: scipy
distances, hand-derived golden values, brute force, closed forms and exact
identities."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.spatial.distance import cdist

import datagen
from oracle import lloyd
from oracle import quantize as Qz
from oracle import stats
from oracle.formats import bf16_rne, unpack_zeros, unpack_codes

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _table(rng, n_c=16, d=128, scale=1.0):
    return bf16_rne(rng.standard_normal((n_c, d)) * scale)


def test_weighted_distance_is_scipy():
    rng = np.random.default_rng(0)
    K = bf16_rne(rng.standard_normal((20, 128)))
    C = _table(rng)
    np.testing.assert_allclose(Qz.weighted_dists(K, C, np.ones(128)), cdist(K, C, "sqeuclidean"),
                               rtol=1e-13)
    w = rng.uniform(0.1, 5.0, 128).astype(np.float32)
    # scipy's standardized Euclidean distance divides by V = 1/w
    ref = cdist(K, C, "seuclidean", V=1.0 / w.astype(np.float64)) ** 2
    np.testing.assert_allclose(Qz.weighted_dists(K, C, w), ref, rtol=1e-12)


def test_qsac_golden_uniform_weights():
    g = json.load(open(os.path.join(GOLD, "qsac_tiny.json")))["cases"][0]
    K = np.zeros((1, 128))
    C = np.zeros((2, 128))
    C[0, 0] = 1.0
    C[1, :] = 0.125
    idx, info = Qz.select_qsac(K, C, np.ones(128, np.float32), M=2)
    assert idx[0] == g["qsac_M2"]
    np.testing.assert_array_equal(info["S"][0][np.argsort(info["cand"][0])], g["S"])
    np.testing.assert_array_equal(info["dq"][0], g["dq"])
    assert Qz.select_qsac(K, C, np.ones(128, np.float32), M=1)[0][0] == g["qsac_M1"]
    assert Qz.select_nearest(K, C)[0][0] == g["nearest"]
    out = Qz.quantize_keys(K, C, None, None, M=2, flags=Qz.QSAC)
    np.testing.assert_array_equal(out["scale"][0], g["qsac_scale"])
    np.testing.assert_array_equal(out["scale_bits"][0], g["qsac_scale_bits"])
    np.testing.assert_array_equal(out["zero"][0], g["qsac_zero"])
    assert np.all(out["q"] == g["qsac_codes_all"])
    assert np.all(out["r_hat"] == g["qsac_r_hat"])
    assert out["zeros"][0] & 0xF == 15
    near = Qz.quantize_keys(K, C, None, None, M=2, flags=0)
    assert near["idx"][0] == g["nearest"]
    np.testing.assert_array_equal(near["scale"][0], g["nearest_scale"])
    np.testing.assert_array_equal(near["scale_bits"][0], g["nearest_scale_bits"])
    np.testing.assert_array_equal(near["zero"][0], g["nearest_zero"])
    assert list(near["codes"][0, :2]) == g["nearest_code_bytes_head"]
    assert np.all(near["codes"][0, 2:16] == 255) and np.all(near["codes"][0, 16:] == 0)


def test_qsac_golden_weights_flip():
    g = json.load(open(os.path.join(GOLD, "qsac_tiny.json")))["cases"][1]
    K = np.zeros((1, 128))
    C = np.zeros((2, 128))
    C[0, 0] = 1.0
    C[1, 64] = 0.5
    w = np.ones(128, np.float32)
    w[64:] = 16
    idx, info = Qz.select_qsac(K, C, w, M=2)
    assert idx[0] == g["qsac_M2"]
    np.testing.assert_array_equal(info["dq"][0], g["dq"])
    np.testing.assert_array_equal(info["S"][0][np.argsort(info["cand"][0])], g["S"])
    assert Qz.select_qsac(K, C, np.ones(128, np.float32), M=2)[0][0] == g["qsac_M2_uniform"]
    assert Qz.select_nearest(K, C)[0][0] == g["nearest"]


def _S_bruteforce(k, mu, w):
    """QSAC score by plain Python: residual in float32, ranges, group weight sums."""
    r = (np.float32(1) * k.astype(np.float32)) - mu.astype(np.float32)
    S = 0.0
    for g in range(2):
        seg = [float(x) for x in r[64 * g:64 * g + 64]]
        R = max(0.0, max(seg)) - min(0.0, min(seg))
        S += math.fsum(float(x) for x in w[64 * g:64 * g + 64]) * R * R
    return S


def test_qsac_full_candidate_set_is_argmin_of_S():
    """M = n_c: QSAC returns the centroid with the smallest S (ties -> lowest j)."""
    rng = np.random.default_rng(1)
    C = _table(rng, n_c=24, scale=0.3)
    K = bf16_rne(C[rng.integers(0, 24, 30)] + 0.3 * rng.standard_normal((30, 128)))
    w = rng.uniform(0.2, 3, 128).astype(np.float32)
    idx, _ = Qz.select_qsac(K, C, w, M=24)
    for t in range(30):
        S = [_S_bruteforce(K[t], C[j], w) for j in range(24)]
        best = min(range(24), key=lambda j: (S[j], j))
        assert idx[t] == best


def test_qsac_M1_is_weighted_nearest_and_uniform_is_euclidean():
    rng = np.random.default_rng(2)
    C = _table(rng, n_c=32)
    K = bf16_rne(rng.standard_normal((50, 128)))
    w = rng.uniform(0.2, 3, 128).astype(np.float32)
    idx, _ = Qz.select_qsac(K, C, w, M=1)
    ref = cdist(K, C, "seuclidean", V=1.0 / w.astype(np.float64)).argmin(axis=1)
    np.testing.assert_array_equal(idx, ref)
    np.testing.assert_array_equal(Qz.select_nearest(K, C)[0], cdist(K, C, "sqeuclidean").argmin(1))


def test_qsac_score_bounds_distance():
    """S_j >= d_Q(j) for every candidate (|r_c| <= R_g and w >= 0)."""
    w = datagen.make_workload("tiny", chunk=600)
    K = w.K[:, 0]
    rng = np.random.default_rng(3)
    C = bf16_rne(K[rng.choice(600, 64, replace=False)])
    ww = rng.uniform(0.0, 4, 128).astype(np.float32)
    idx, info = Qz.select_qsac(K, C, ww, M=8)
    dq_c = np.take_along_axis(info["dq"], info["cand"], axis=1)
    assert np.all(info["S"] >= dq_c * (1 - 1e-12))


def test_codec_invariants_and_error_bound():
    rng = np.random.default_rng(4)
    r = (rng.standard_normal((400, 128)) * np.exp(rng.uniform(-6, 3, (400, 1)))).astype(np.float32)
    r[0] = 0.0                       # zero range -> s = 0
    r[1, :64] = 0.25                 # one-signed groups
    r[2, 64:] = -1.5
    q, s, z, r_hat, nsat = Qz.encode_residual(r)
    assert nsat == 0
    assert q.min() >= 0 and q.max() <= 3 and z.min() >= 0 and z.max() <= 3
    err = np.abs(r.astype(np.float64) - r_hat).reshape(400, 2, 64)
    assert np.all(err <= s[..., None] / 2)
    assert np.all(s[0] == 0) and np.all(q[0] == 0) and np.all(z[0] == 0)
    # s is the smallest fp16 with 3s >= R (checked exactly on a sample)
    lo = np.minimum(0, r.astype(np.float64).reshape(400, 2, 64).min(-1))
    hi = np.maximum(0, r.astype(np.float64).reshape(400, 2, 64).max(-1))
    for t in range(0, 400, 7):
        for g in range(2):
            R = Fraction(hi[t, g]) - Fraction(lo[t, g])
            sv = Fraction(s[t, g])
            assert 3 * sv >= R
            if s[t, g] > 0:
                prev = Fraction(float(np.nextafter(np.float16(s[t, g]), np.float16(0))))
                assert 3 * prev < R
                assert z[t, g] == min(3, max(0, round(-Fraction(lo[t, g]) / sv)))


def test_codec_mse_matches_uniform_noise_model():
    """Uniform residuals: MSE = R^2 / [12 (2^b - 1)^2] with b = 2 (the pages'
    INT2 error model), within statistical error; the stored scale is within
    2^-10 of R/3."""
    rng = np.random.default_rng(5)
    n = 6000
    a = -rng.uniform(0.05, 2.0, (n, 2, 1))          # each group: uniform on [a, b], a < 0 < b
    b = rng.uniform(0.05, 2.0, (n, 2, 1))
    r = (a + (b - a) * rng.uniform(0, 1, (n, 2, 64))).reshape(n, 128).astype(np.float32)
    q, s, z, r_hat, _ = Qz.encode_residual(r)
    lo, hi, R = Qz.group_ranges(r)
    mse = np.mean((r.astype(np.float64) - r_hat) ** 2)
    model = np.mean(R ** 2) / (12 * (2 ** 2 - 1) ** 2)
    assert abs(mse / model - 1) < 0.03
    assert np.all(s >= R / 3) and np.all(s <= R / 3 * (1 + 2 ** -10))


def test_psac_full_rank_restores_keys_exactly():
    """r = d, float64 orthonormal U, unquantized C: K0_hat + C U^T = K."""
    rng = np.random.default_rng(6)
    K = bf16_rne(rng.standard_normal((40, 128)))
    C = _table(rng, n_c=8)
    out = Qz.quantize_keys(K, C, None, None, M=4, flags=Qz.QSAC)
    K0 = Qz.dequant_values(out["idx"], out["q"], out["scale"], out["zero"], C)
    U = datagen.haar_orthogonal(rng, 128)
    E = K - K0
    Cf = E @ U
    np.testing.assert_allclose(K0 + Cf @ U.T, K, rtol=0, atol=1e-12 * np.abs(K).max())


def test_psac_gain_identity():
    """With eigenvectors U_r of M and unquantized C: e'^T M e' = e^T M e - sum_j lam_j (u_j^T e)^2."""
    rng = np.random.default_rng(7)
    Uh = datagen.haar_orthogonal(rng, 128)
    lam = datagen.query_spectrum(0.65)
    M = (Uh * lam) @ Uh.T
    Ur = Uh[:, :8]
    for _ in range(5):
        e = rng.standard_normal(128)
        e2 = e - Ur @ (Ur.T @ e)
        lhs = e2 @ M @ e2
        rhs = e @ M @ e - np.sum(lam[:8] * (Ur.T @ e) ** 2)
        assert abs(lhs - rhs) <= 1e-12 * (e @ M @ e)
        assert lhs <= e @ M @ e


def test_psac_int8_scale_and_codes_exact():
    rng = np.random.default_rng(8)
    E = rng.standard_normal((60, 128)) * np.exp(rng.uniform(-8, 2, (60, 1)))
    E[0] = 0
    U = bf16_rne(datagen.haar_orthogonal(rng, 128)[:, :8])
    Cq, cs, C = Qz.psac_coefficients(E, U)
    np.testing.assert_allclose(C, E @ U, rtol=0, atol=0)
    assert np.all(Cq[0] == 0) and cs[0] == 0
    assert Cq.min() >= -127 and Cq.max() <= 127
    for t in range(1, 60):
        m = max(abs(Fraction(x)) for x in C[t])
        c = Fraction(cs[t])
        assert 127 * c >= m and 127 * Fraction(float(np.nextafter(np.float16(cs[t]), np.float16(0)))) < m
        for j in range(8):
            assert Cq[t, j] == max(-127, min(127, round(Fraction(C[t, j]) / c)))


def test_logit_identity():
    """Q K_hat^T = Q K0_hat^T + (Q U) (c_s C_q)^T, to 1e-12 relative."""
    w = datagen.make_workload("tiny", chunk=300, n_queries=50)
    K, Qm = w.K[:, 0].astype(np.float64), w.Q[:, 0].astype(np.float64)
    rng = np.random.default_rng(9)
    C = bf16_rne(K[rng.choice(300, 32, replace=False)])
    S, n = stats.update(np.zeros((128, 128)), 0, Qm)
    basis = stats.principal_basis(S, n)
    U = basis["U_bf16"]
    out = Qz.quantize_keys(K, C, stats.channel_weights(S, n), U, M=8)
    Khat = Qz.dequant_keys(out["idx"], out["q"], out["scale"], out["zero"], out["Cq"],
                           out["c_scale"], C, U)
    K0 = Qz.dequant_values(out["idx"], out["q"], out["scale"], out["zero"], C)
    lhs = Qm @ Khat.T
    rhs = Qm @ K0.T + (Qm @ U) @ (out["c_scale"][:, None] * out["Cq"]).T
    assert np.linalg.norm(lhs - rhs) <= 1e-12 * np.linalg.norm(lhs)
    # PSAC shrinks the Query-weighted key error on average
    M = S / n
    e0 = K - K0
    e1 = K - Khat
    assert np.mean(np.einsum("ti,ij,tj->t", e1, M, e1)) < np.mean(np.einsum("ti,ij,tj->t", e0, M, e0))


def test_values_are_nearest_plus_codec():
    rng = np.random.default_rng(10)
    C = _table(rng, n_c=20)
    V = bf16_rne(C[rng.integers(0, 20, 64)] + 0.1 * rng.standard_normal((64, 128)))
    out = Qz.quantize_values(V, C)
    np.testing.assert_array_equal(out["idx"], cdist(V, C, "sqeuclidean").argmin(1))
    np.testing.assert_array_equal(unpack_codes(out["codes"], 128), out["q"])
    np.testing.assert_array_equal(unpack_zeros(out["zeros"], 64), out["zero"])
    Vh = Qz.dequant_values(out["idx"], out["q"], out["scale"], out["zero"], C)
    err = np.abs(V - Vh).reshape(64, 2, 64)
    assert np.all(err <= out["scale"][..., None] / 2)


def test_psac_keep_test():
    """The keep test (method step (4)): with it, no token's Query-weighted error
    sum_c w_c e_c^2 (e = k - K_hat) is above the error without compensation,
    and the criterion equals the difference of the two errors, computed
    directly (brute force) for every token."""
    w = datagen.make_workload("480p", heads=[0], n_chunks=1, chunk=400)
    K, Q = w.K[:, 0].astype(np.float64), w.Q[:, 0].astype(np.float64)
    C = lloyd.lloyd(K, 256, 2, seed=3)
    S, n = stats.update(np.zeros((128, 128)), 0, Q)
    U = stats.principal_basis(S, n)["U_bf16"]
    wt = stats.channel_weights(S, n)
    full = Qz.quantize_keys(K, C, wt, U, M=8, flags=Qz.QSAC | Qz.PSAC)
    kept = Qz.quantize_keys(K, C, wt, U, M=8, flags=Qz.QSAC | Qz.PSAC | Qz.PSAC_KEEP)
    assert np.array_equal(full["idx"], kept["idx"]) and np.array_equal(full["q"], kept["q"])
    info = kept["keep"]
    w64 = np.asarray(wt, np.float32).astype(np.float64)
    mu = np.asarray(C, np.float64)[np.asarray(full["idx"], np.int64)]
    E = K - (mu + full["r_hat"])
    D = (full["c_scale"][:, None] * full["Cq"].astype(np.float64)) @ np.asarray(U, np.float64).T
    err_with = np.sum(w64 * (E - D) ** 2, axis=1)
    err_without = np.sum(w64 * E ** 2, axis=1)
    np.testing.assert_allclose(info["crit"], err_with - err_without, rtol=1e-9, atol=1e-9 * err_without.max())
    assert np.array_equal(info["keep"], err_with < err_without)
    # dropped tokens store zeros; kept ones their coefficients unchanged
    assert np.all(kept["Cq"][~info["keep"]] == 0) and np.all(kept["c_scale"][~info["keep"]] == 0)
    assert np.array_equal(kept["Cq"][info["keep"]], full["Cq"][info["keep"]])
    # the error with the stored coefficients never exceeds the uncompensated one
    Dk = (kept["c_scale"][:, None] * kept["Cq"].astype(np.float64)) @ np.asarray(U, np.float64).T
    assert np.all(np.sum(w64 * (E - Dk) ** 2, axis=1) <= err_without * (1 + 1e-12))
    assert 0 < info["keep"].sum() < len(K) or info["keep"].all()


# ---- full-matrix candidate distance (QuantWM App. C.4 ablation) ----

def _spd(rng, d=128, rank=12):
    A = rng.standard_normal((d, rank))
    return A @ A.T / rank + 0.05 * np.eye(d)


def test_full_distance_is_scipy_mahalanobis():
    rng = np.random.default_rng(11)
    K = bf16_rne(rng.standard_normal((15, 128)))
    C = _table(rng)
    Mq = _spd(rng)
    ref = cdist(K, C, "mahalanobis", VI=Mq) ** 2
    np.testing.assert_allclose(Qz.full_dists(K, C, Mq), ref, rtol=1e-11)


def test_full_form_golden_correlation_flips_candidate():
    # k = 0, mu_0 = e_0 + e_1, mu_1 = e_0 - e_1; Mq = I except Mq[0,1] = Mq[1,0] = 1/2.
    # Diagonal form (w = diag Mq = 1): both at 2, tie -> index 0.  Full form:
    # (e_0 + e_1)^T Mq (e_0 + e_1) = 2 + 2(1/2) = 3, (e_0 - e_1)^T Mq (e_0 - e_1) = 2 - 1 = 1 -> index 1.
    K = np.zeros((1, 128))
    C = np.zeros((2, 128))
    C[0, 0], C[0, 1] = 1.0, 1.0
    C[1, 0], C[1, 1] = 1.0, -1.0
    Mq = np.eye(128)
    Mq[0, 1] = Mq[1, 0] = 0.5
    np.testing.assert_array_equal(Qz.full_dists(K, C, Mq)[0], [3.0, 1.0])
    w = np.ones(128, np.float32)
    assert Qz.select_qsac(K, C, w, M=1)[0][0] == 0
    assert Qz.select_qsac(K, C, w, M=1, Mq=Mq)[0][0] == 1
    out = Qz.quantize_keys(K, C, w, None, M=1, flags=Qz.QSAC | Qz.QSAC_FULL, Mq=Mq)
    assert out["idx"][0] == 1


def test_full_form_with_diagonal_matrix_is_diagonal_qsac():
    w8 = datagen.make_workload("480p", heads=[0], n_chunks=2, chunk=400)
    K = w8.K[400:, 0].astype(np.float64)
    C = lloyd.lloyd(w8.K[:400, 0].astype(np.float64), 256, 2, seed=3, head=0)
    S, n = stats.update(np.zeros((128, 128)), 0, w8.Q[:400, 0])
    wt = stats.channel_weights(S, n)
    a, ia = Qz.select_qsac(K, C, wt, 8)
    b, ib = Qz.select_qsac(K, C, wt, 8, Mq=np.diag(wt.astype(np.float64)))
    np.testing.assert_allclose(ib["dq"], ia["dq"], rtol=1e-13)
    np.testing.assert_array_equal(np.sort(ib["cand"], axis=1), np.sort(ia["cand"], axis=1))
    np.testing.assert_array_equal(a, b)


def test_full_form_rotation_invariance():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((10, 128))
    C = rng.standard_normal((12, 128))
    Mq = _spd(rng)
    Qm, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    d0 = Qz.full_dists(K, C, Mq)
    d1 = Qz.full_dists(K @ Qm.T, C @ Qm.T, Qm @ Mq @ Qm.T)
    np.testing.assert_allclose(d1, d0, rtol=1e-9)


def test_full_form_all_candidates_is_score_argmin():
    # with M = n_c every centroid is a candidate: the choice is argmin (S, j)
    # whatever the distance
    rng = np.random.default_rng(2)
    K = bf16_rne(rng.standard_normal((30, 128)))
    C = _table(rng)
    wt = rng.uniform(0.2, 3.0, 128).astype(np.float32)
    a = Qz.select_qsac(K, C, wt, C.shape[0])[0]
    b = Qz.select_qsac(K, C, wt, C.shape[0], Mq=_spd(rng))[0]
    np.testing.assert_array_equal(a, b)


def test_second_moment_cold_start_and_mean():
    Q = np.arange(12.0).reshape(3, 4)
    S = Q.T @ Q
    np.testing.assert_array_equal(Qz.second_moment(S, 3), S / 3.0)
    np.testing.assert_array_equal(Qz.second_moment(np.zeros((4, 4)), 0), np.eye(4))
