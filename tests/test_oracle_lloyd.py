"""Pins of the oracle's seeded Lloyd iteration: published SplitMix64 outputs,
scikit-learn's Lloyd k-means, brute-force invariants."""
import json
import os

import numpy as np
import pytest

from oracle import lloyd
from oracle.formats import bf16_rne

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_outputs():
    g = json.load(open(os.path.join(GOLD, "splitmix64.json")))
    c0 = g["cases"][0]
    r = lloyd.SplitMix64(c0["seed"])
    assert [r.next() for _ in c0["outputs"]] == c0["outputs"]
    c1 = g["cases"][1]
    r = lloyd.SplitMix64(c1["seed"])
    assert [hex(r.next()) for _ in c1["outputs_hex"]] == c1["outputs_hex"]


def test_forgy_indices_distinct_and_permutation():
    idx = lloyd.forgy_indices(1000, 256, seed=7, head=3)
    assert len(set(idx.tolist())) == 256 and idx.min() >= 0 and idx.max() < 1000
    np.testing.assert_array_equal(idx, lloyd.forgy_indices(1000, 256, seed=7, head=3))
    assert not np.array_equal(idx, lloyd.forgy_indices(1000, 256, seed=7, head=4))
    # N == n_c: a full Fisher-Yates shuffle, i.e. a permutation
    assert sorted(lloyd.forgy_indices(256, 256, 0, 0).tolist()) == list(range(256))
    with pytest.raises(ValueError):
        lloyd.forgy_indices(255, 256, 0, 0)


def test_forgy_first_pick_by_hand():
    """Pick 0 = 0 + next() mod N with the generator seeded at seed + (head << 32)."""
    N = 4096
    r = lloyd.SplitMix64(5 + (2 << 32))
    first = r.next() % N
    assert lloyd.forgy_indices(N, 256, seed=5, head=2)[0] == first


def test_forgy_picks_by_hand():
    """Picks 0-3 of the seeded shuffle for N = 10, worked by hand from the
    published SplitMix64 outputs (tests/golden/forgy_tiny.json): a dropped
    '+ i', a modulus of N instead of N - i, or a missed swap each change them."""
    g = json.load(open(os.path.join(GOLD, "forgy_tiny.json")))
    sm = json.load(open(os.path.join(GOLD, "splitmix64.json")))["cases"][0]
    assert g["seed"] == sm["seed"]
    assert [s["output"] for s in g["steps"]] == sm["outputs"][:4]
    got = lloyd.forgy_indices(g["N"], g["n_c"], seed=g["seed"], head=g["head"])
    assert got.tolist() == g["picks"]


def test_forgy_skips_nonfinite_rows_by_hand():
    """A pick that lands on a row with a non-finite channel is dropped and the
    shuffle takes one more step (tests/golden/forgy_tiny.json, worked by hand)."""
    g = json.load(open(os.path.join(GOLD, "forgy_tiny.json")))
    fin = np.ones(g["N"], bool)
    fin[g["nonfinite_case"]["nonfinite_rows"]] = False
    got = lloyd.forgy_indices(g["N"], g["n_c"], seed=g["seed"], head=g["head"], finite=fin)
    assert got.tolist() == g["nonfinite_case"]["picks"]
    # fewer finite rows than centroids: the missing picks are marked
    fin[:] = False
    fin[[3, 5]] = True
    got = lloyd.forgy_indices(g["N"], g["n_c"], seed=g["seed"], head=g["head"], finite=fin)
    assert sorted(got[:2].tolist()) == [3, 5] and got[2:].tolist() == [-1, -1]


def test_lloyd_ignores_nonfinite_rows():
    """Rows with a NaN or infinite channel change nothing: the table built
    with them equals the one built on the finite rows alone (warm start), and
    a Forgy start takes only finite rows."""
    rng = np.random.default_rng(4)
    X = rng.standard_normal((300, 16))
    init = bf16_rne(X[:32] + 0.01)
    Xb = X.copy()
    bad = [3, 50, 51, 299]
    Xb[3, 0] = np.nan
    Xb[50, 5] = np.inf
    Xb[51, :] = -np.inf
    Xb[299, 15] = np.nan
    keep = np.setdiff1d(np.arange(300), bad)
    np.testing.assert_array_equal(lloyd.lloyd(Xb, 32, 4, init=init), lloyd.lloyd(X[keep], 32, 4, init=init))
    C0 = lloyd.lloyd(Xb, 32, 0, seed=2, head=1)
    assert np.all(np.isfinite(C0))
    picks = lloyd.forgy_indices(300, 32, 2, 1, finite=lloyd.finite_rows(Xb))
    assert not set(picks.tolist()) & set(bad)
    np.testing.assert_array_equal(C0, bf16_rne(Xb[picks]))


def test_lloyd_matches_sklearn():
    """Data whose cluster means are exact in bf16: every Lloyd step agrees with
    scikit-learn's Lloyd k-means from the same initial table."""
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(0)
    centers = rng.integers(-8, 8, (6, 16)).astype(np.float64) * 4.0
    offs = np.array([[1, 0], [-1, 0], [0, 1], [0, -1]], np.float64)   # sum to zero
    X = []
    for c in centers:
        for o in offs:
            x = c.copy()
            x[:2] += o
            X.append(x)
    X = np.array(X)
    init = X[[0, 4, 8, 12, 16, 20]] + 0.5
    ours = lloyd.lloyd(X, n_c=6, iters=5, init=bf16_rne(init))
    km = KMeans(n_clusters=6, init=bf16_rne(init), n_init=1, max_iter=5, tol=0.0,
                algorithm="lloyd").fit(X)
    # scikit-learn's own means carry float64 rounding (ulp level)
    np.testing.assert_allclose(np.sort(ours, axis=0), np.sort(km.cluster_centers_, axis=0), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(ours, centers)


def test_lloyd_nc_equals_n_gives_zero_residual():
    rng = np.random.default_rng(1)
    X = bf16_rne(rng.standard_normal((256, 128)))
    C = lloyd.lloyd(X, n_c=256, iters=3, seed=0, head=0)
    np.testing.assert_array_equal(np.sort(C, axis=0), np.sort(X, axis=0))
    a = lloyd.assign(X, C)
    np.testing.assert_array_equal(C[a], X)


def test_lloyd_objective_nonincreasing_and_empty_cluster():
    rng = np.random.default_rng(2)
    X = bf16_rne(rng.standard_normal((600, 128)))
    C, hist = lloyd.lloyd(X, n_c=32, iters=6, seed=3, head=1, return_history=True)
    objs = []
    for Ci, ai in hist:
        objs.append(np.sum((X - Ci[ai]) ** 2))
    objs.append(np.sum((X - C[lloyd.assign(X, C)]) ** 2))
    for a, b in zip(objs, objs[1:]):
        assert b <= a * (1 + 2 ** -7)      # non-increasing up to bf16 rounding of means
    # a centroid nobody is nearest to keeps its value
    init = np.concatenate([C[:31], np.full((1, 128), 1000.0)])
    C2 = lloyd.lloyd(X, n_c=32, iters=1, init=init)
    np.testing.assert_array_equal(C2[31], init[31])


def test_assign_tie_goes_to_lowest_index():
    C = np.array([[1.0] + [0.0] * 127, [-1.0] + [0.0] * 127])
    X = np.zeros((1, 128))
    assert lloyd.assign(X, C)[0] == 0
    assert lloyd.assign(X, C[::-1])[0] == 0


def test_lloyd_steps_match_sklearn_on_overlapping_clusters():
    """Each single Lloyd step equals scikit-learn's Lloyd step rounded to bf16
    (within one bf16 ulp, because scikit-learn's mean carries float64 rounding)."""
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(3)
    X = bf16_rne(rng.standard_normal((500, 128)) + rng.integers(0, 3, (500, 1)))
    C = bf16_rne(X[:12].copy())
    for _ in range(4):
        ours = lloyd.lloyd(X, n_c=12, iters=1, init=C)
        km = KMeans(n_clusters=12, init=C, n_init=1, max_iter=1, tol=0.0, algorithm="lloyd").fit(X)
        sk = km.cluster_centers_
        ulp = np.ldexp(1.0, np.frexp(np.abs(sk))[1] - 8)
        assert np.all(np.abs(ours - sk) <= ulp)
        assert np.mean(ours == bf16_rne(sk)) > 0.99
        C = ours
