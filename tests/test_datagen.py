"""The seeded synthetic generator: determinism, closed-form Query spectrum,
frame drift, bf16 hand-over."""
import numpy as np

import datagen


def test_deterministic_and_head_independent():
    a = datagen.make_workload("480p", heads=[0, 3], n_chunks=2, chunk=100)
    b = datagen.make_workload("480p", heads=[3], n_chunks=2, chunk=100)
    np.testing.assert_array_equal(a.K[:, 1], b.K[:, 0])
    np.testing.assert_array_equal(a.Q[:, 1], b.Q[:, 0])
    c = datagen.make_workload("480p", heads=[0, 3], n_chunks=2, chunk=100)
    np.testing.assert_array_equal(a.V, c.V)
    assert not np.array_equal(a.K[:, 0], a.K[:, 1])


def test_energy_closed_form():
    for f, rho in ((0.65, 0.87702), (0.60, 0.89178), (0.71, 0.85664)):
        r = datagen.rho_for_energy(f)
        assert abs(r - rho) < 5e-5
        assert abs((1 - r ** 8) / (1 - r ** 128) - f) < 1e-12
        lam = datagen.query_spectrum(f)
        assert abs(lam.sum() - 128) < 1e-9
        assert abs(lam[:8].sum() / lam.sum() - f) < 1e-12
        assert np.all(np.diff(lam) < 0)


def test_bf16_handover_and_shapes():
    w = datagen.make_workload("480p", heads=[1], n_chunks=3, chunk=64)
    assert w.K.shape == (192, 1, 128) and w.Q.shape == (192, 1, 128)
    bits = datagen.bf16_bits(w.K)
    assert bits.dtype == np.uint16
    t = datagen.make_workload("tiny", chunk=256)
    assert t.dtype == "f32" and t.Q.shape == (512, 1, 128)
    assert np.any(t.K.view(np.uint32) & 0xFFFF)


def test_frame_drift_and_cluster_noise():
    rng = datagen.rng_for(0, 9, 0, 0, 1)
    x = datagen.cluster_stream(rng, 4 * 2000, 2000, noise=0.0, drift=0.05)
    # with zero noise every token is one of 256 means; means move by N(0, 0.05^2) per frame
    f0 = np.unique(x[:2000], axis=0)
    f1 = np.unique(x[2000:4000], axis=0)
    assert f0.shape[0] <= 256 and f1.shape[0] <= 256
    sig = np.exp(datagen.rng_for(0, 9, 0, 0, 1).uniform(np.log(0.25), np.log(4.0), 128))
    assert 0.25 <= sig.min() and sig.max() <= 4.0


def test_device_layer_recipe():
    """The on-device draw of a layer (CPU device here): shapes, bf16, reproducible
    per (layer, seed), layers differ, and the Query spectrum's top-8 share is the
    requested one (within sampling error)."""
    import torch
    K, V, Q = datagen.device_layer("depth", 3, device="cpu", heads=4, n_tokens=3000, n_queries=4000)
    assert K.shape == (3000, 4, 128) and V.shape == K.shape and Q.shape == (4000, 4, 128)
    assert K.dtype == torch.bfloat16 and Q.dtype == torch.bfloat16
    K2, _, _ = datagen.device_layer("depth", 3, device="cpu", heads=4, n_tokens=3000, n_queries=4000)
    assert torch.equal(K, K2)
    K3, _, _ = datagen.device_layer("depth", 4, device="cpu", heads=4, n_tokens=3000, n_queries=4000)
    assert not torch.equal(K, K3)
    for h in range(4):
        q = Q[:, h].double().numpy()
        ev = np.linalg.eigvalsh(q.T @ q / len(q))[::-1]
        assert abs(ev[:8].sum() / ev.sum() - 0.65) < 0.03
        # 256 well-separated clusters: noise 0.1 around each token's mean
        x = K[:, h].float().numpy()
        assert 0.2 < np.median(x.std(axis=0)) < 4.0
