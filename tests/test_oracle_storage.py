"""Pins of the oracle's storage refinements: the dense/sparse coefficient
layout, two-level group scales and the full-form keep test."""
import math
from fractions import Fraction

import numpy as np

import datagen
from oracle import quantize as Qz
from oracle import stats as OS
from oracle import storage as St
from oracle.formats import bf16_rne, fp16_bits


def test_layout_sizes_by_hand():
    # T = 100, r = 8, 90 kept.  Dense: 800 coefficient bytes + 200 scale bytes
    # (-> 208 on a 16-byte boundary) = 1008.  Sparse: 2 words -> 16 bitmap bytes,
    # 8 prefix bytes -> 16, 720 coefficient bytes, 180 scale bytes -> 192: 944.
    assert St.dense_bytes(100, 8) == 1008
    assert St.sparse_bytes(100, 90, 8) == 944
    assert St.choose_layout(100, 90, 8) == "sparse"
    # all kept: 1008 + 32 > 1008, dense; none kept: 32 bytes
    assert St.choose_layout(100, 100, 8) == "dense"
    assert St.sparse_bytes(100, 0, 8) == 32
    # a tie keeps the dense layout
    for T in range(1, 200):
        for count in range(T + 1):
            d, s = St.dense_bytes(T, 16), St.sparse_bytes(T, count, 16)
            assert St.choose_layout(T, count, 16) == ("sparse" if s < d else "dense")


def test_sparse_bitmap_by_hand():
    """T = 70, keys 0, 5, 63, 64 and 69 keep coefficients: word 0 has bits 0, 5
    and 63, word 1 bits 0 and 5; three kept keys precede word 1."""
    T, r = 70, 8
    rng = np.random.default_rng(1)
    Cq = rng.integers(-127, 128, (T, r)).astype(np.int8)
    cs = np.zeros(T, np.uint16)
    kept = [0, 5, 63, 64, 69]
    cs[kept] = fp16_bits(np.array([0.5, 0.25, 1.0, 2.0, 0.125]))
    p = St.pack_coefficients(Cq, cs)
    assert p["layout"] == "sparse" and p["count"] == 5
    assert int(p["bitmap"][0]) == 1 + 32 + (1 << 63)
    assert int(p["bitmap"][1]) == 33
    assert p["prefix"].tolist() == [0, 3]
    np.testing.assert_array_equal(p["c"], Cq[kept])
    np.testing.assert_array_equal(p["cs"], cs[kept])


def test_layout_round_trip():
    rng = np.random.default_rng(2)
    for T, r, frac in ((777, 8, 0.3), (64, 16, 0.0), (129, 32, 1.0), (1000, 8, 0.98), (1, 8, 1.0)):
        Cq = rng.integers(-127, 128, (T, r)).astype(np.int8)
        cs = fp16_bits(rng.uniform(1e-3, 1.0, T))
        drop = rng.random(T) > frac
        Cq[drop] = 0
        cs[drop] = 0
        p = St.pack_coefficients(Cq, cs)
        C2, cs2 = St.unpack_coefficients(p, T, r)
        np.testing.assert_array_equal(C2, Cq)
        np.testing.assert_array_equal(cs2, cs)
        assert p["bytes"] == min(St.dense_bytes(T, r), St.sparse_bytes(T, int((~drop).sum()), r)) or \
            p["bytes"] == St.dense_bytes(T, r)


def test_second_level_scale_exact():
    """The smallest power of two p >= 2^-24 with 255 p >= m, checked with
    exact rationals."""
    for m in [1e-9, 6e-8, 1e-3, 0.0039, 1.0 / 255, 0.5, 1.0, 2.0, 255.0, 1000.0, 65504.0]:
        p = St.second_level_scale(m)
        e = round(math.log2(p))
        assert p == 2.0 ** e and e >= -24
        assert Fraction(255) * Fraction(p) >= Fraction(m)
        if e > -24:
            assert Fraction(255) * Fraction(p) / 2 < Fraction(m)
    assert St.second_level_scale(0.0) == 0.0


def test_two_level_by_hand():
    # group 0: max 1.0 -> 2^-7 (255 / 128 = 1.99 >= 1 > 255 / 256); codes 64, 32, 128
    # group 1: max 2.0 -> 2^-6 (255 / 128 = 1.992 < 2 <= 255 / 64); codes 128, 0, 96
    s = np.array([[0.5, 2.0], [0.25, 0.0], [1.0, 1.5]])
    q, s2, steps = St.two_level_scales(s)
    assert s2.tolist() == [2.0 ** -7, 2.0 ** -6]
    assert q.tolist() == [[64, 128], [32, 0], [128, 96]]
    np.testing.assert_array_equal(steps, s)     # these steps are exact multiples


def test_two_level_invariants():
    """Codes at most 255, steps never below the fp16 step (so the coded range
    still covers the residuals) and exactly representable in fp16; the
    per-channel error stays within half the effective step; at the fp16 steps
    themselves the codec is the single-level one."""
    w = datagen.make_workload("480p", heads=[0], n_chunks=1, chunk=500)
    K = w.K[:, 0].astype(np.float64)
    from oracle import lloyd as OL
    C = OL.lloyd(K, 256, 2, seed=3, head=0)
    base = Qz.quantize_keys(K, C, None, None, M=8, flags=1)
    q, s2, steps = St.two_level_scales(base["scale"])
    assert q.max() <= 255
    assert np.all(steps >= base["scale"])
    assert np.all(steps.astype(np.float16).astype(np.float64) == steps)
    assert np.all(np.ceil(base["scale"] / s2) == q)
    r = Qz.residual(K, C[base["idx"]])
    qq, z, r_hat = St.encode_with_steps(r, steps)
    assert qq.max() <= 3 and z.max() <= 3
    stp = np.repeat(steps, 64, axis=1)
    assert np.all(np.abs(r - r_hat) <= stp / 2 * (1 + 2.0 ** -22))
    q1, z1, rh1 = St.encode_with_steps(r, base["scale"])
    np.testing.assert_array_equal(q1, base["q"])
    np.testing.assert_array_equal(z1, base["zero"])


def test_two_level_keys_pipeline():
    """The two-level keys keep the centroid choice; their PSAC error is
    X - (mu + r_hat) of the new codes, and with r = d and the unquantized
    coefficients the keys are restored exactly."""
    rng = np.random.default_rng(5)
    w = datagen.make_workload("480p", heads=[0], n_chunks=1, chunk=400)
    K = w.K[:, 0].astype(np.float64)
    from oracle import lloyd as OL
    C = OL.lloyd(K, 256, 2, seed=3, head=0)
    S, n = OS.update(np.zeros((128, 128)), 0, w.Q[:, 0])
    U = OS.principal_basis(S, n)["U_bf16"]
    base = Qz.quantize_keys(K, C, OS.channel_weights(S, n), U, M=8)
    two = St.requantize_two_level(K, C, base, U_bf16=U, w=OS.channel_weights(S, n), flags=3)
    np.testing.assert_array_equal(two["idx"], base["idx"])
    mu = C[base["idx"]]
    np.testing.assert_array_equal(two["E"], K - (mu + two["r_hat"]))
    full = np.linalg.qr(rng.standard_normal((128, 128)))[0]
    Craw = two["E"] @ full
    np.testing.assert_allclose(mu + two["r_hat"] + Craw @ full.T, K, atol=1e-12)


def test_keep_full_reduces_to_diagonal_and_to_the_query_history():
    """With M = diag(w) the full-form test is the diagonal one; with M = S / n
    its errors equal the mean of (q . e)^2 over the Query history itself."""
    rng = np.random.default_rng(7)
    T = 300
    E = rng.standard_normal((T, 128)) * 0.1
    U = bf16_rne(datagen.haar_orthogonal(rng, 128)[:, :8])
    Craw = E @ U
    cs = np.maximum(np.abs(Craw).max(axis=1) / 127, 1e-6)
    Cq = np.clip(np.rint(Craw / cs[:, None]), -127, 127).astype(np.int8)
    Cq[::3] = -Cq[::3]                      # a third of the tokens made worse by their coefficients
    wt = rng.uniform(0.1, 3.0, 128)
    k1, _, _ = St.psac_keep_full(E, Cq, cs, U, np.diag(wt))
    k2, _, _ = Qz.psac_keep(E, Cq, cs, U, wt)
    np.testing.assert_array_equal(k1, k2)
    assert 0 < k1.mean() < 1
    Q = rng.standard_normal((1000, 128)) @ np.diag(np.linspace(2, 0.1, 128))
    S, n = OS.update(np.zeros((128, 128)), 0, Q)
    keep, after, before = St.psac_keep_full(E, Cq, cs, U, S / n)
    D = (cs[:, None] * Cq) @ U.T
    np.testing.assert_allclose(before, np.mean((E @ Q.T) ** 2, axis=1), rtol=1e-10)
    np.testing.assert_allclose(after, np.mean(((E - D) @ Q.T) ** 2, axis=1), rtol=1e-10)
