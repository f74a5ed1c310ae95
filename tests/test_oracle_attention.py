"""Pins of the oracle's attention: an independent blockwise online-softmax
implementation, scipy's softmax, and special cases."""
import numpy as np
import pytest
from scipy.special import softmax, logsumexp

import datagen
from oracle import attention as A
from oracle import lloyd, quantize as Qz, stats
from oracle.formats import bf16_rne


def _online_softmax(Q, K, V, scale, block=7):
    """Blockwise streaming softmax written independently of the oracle."""
    Tq, d = Q.shape
    m = np.full(Tq, -np.inf)
    l = np.zeros(Tq)
    acc = np.zeros((Tq, V.shape[1]))
    for s in range(0, K.shape[0], block):
        z = scale * (Q @ K[s:s + block].T)
        m_new = np.maximum(m, z.max(axis=1))
        corr = np.exp(m - m_new)
        p = np.exp(z - m_new[:, None])
        l = l * corr + p.sum(axis=1)
        acc = acc * corr[:, None] + p @ V[s:s + block]
        m = m_new
    return acc / l[:, None], m + np.log(l)


def test_attention_matches_online_softmax_and_scipy():
    rng = np.random.default_rng(0)
    Q = rng.standard_normal((9, 128)) * 2
    K = rng.standard_normal((50, 128))
    V = rng.standard_normal((50, 128))
    sc = 1 / np.sqrt(128)
    O, lse, top = A.softmax_attention(Q, K, V, sc)
    O2, lse2 = _online_softmax(Q, K, V, sc)
    assert np.max(np.abs(O - O2)) <= 1e-12 * np.max(np.abs(O))
    np.testing.assert_allclose(lse, lse2, rtol=1e-13)
    P = softmax(sc * Q @ K.T, axis=1)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(O, P @ V, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, logsumexp(sc * Q @ K.T, axis=1), rtol=1e-13)
    np.testing.assert_array_equal(top, np.argmax(Q @ K.T, axis=1))


def test_single_key_and_ties():
    rng = np.random.default_rng(1)
    Q = rng.standard_normal((3, 128))
    K = rng.standard_normal((1, 128))
    V = rng.standard_normal((1, 128))
    O, lse, top = A.softmax_attention(Q, K, V, 0.1)
    np.testing.assert_allclose(O, np.repeat(V, 3, axis=0), rtol=1e-15)
    np.testing.assert_allclose(lse, 0.1 * (Q @ K.T)[:, 0], rtol=1e-14)
    # duplicated keys: top-1 picks the lowest index
    K2 = np.concatenate([K, K, K])
    assert np.all(A.top1(Q, K2) == 0)
    assert A.shift_rate(np.array([0, 1, 2, 3]), np.array([0, 1, 5, 3])) == 0.25


def test_cache_attention_is_attention_on_dequantized_segments():
    w = datagen.make_workload("480p", heads=[0], n_chunks=2, chunk=300)
    K, V, Q = (w.K[:, 0].astype(np.float64), w.V[:, 0].astype(np.float64),
               w.Q[:, 0].astype(np.float64))
    segs = []
    S, n = np.zeros((128, 128)), 0
    prevk = prevv = None
    for t in range(2):
        sl = w.chunk_slice(t)
        Ck = lloyd.lloyd(K[sl], 256, 2 if t else 3, seed=11, init=prevk)
        Cv = lloyd.lloyd(V[sl], 256, 2 if t else 3, seed=12, init=prevv)
        U = stats.principal_basis(S, n)["U_bf16"] if n else None
        kq = Qz.quantize_keys(K[sl], Ck, stats.channel_weights(S, n), U, M=8)
        vq = Qz.quantize_values(V[sl], Cv)
        segs.append(dict(k_idx=kq["idx"], k_q=kq["q"], k_scale=kq["scale"], k_zero=kq["zero"],
                         k_Cq=kq["Cq"], k_cs=kq["c_scale"], k_centroids=Ck, U=U,
                         v_idx=vq["idx"], v_q=vq["q"], v_scale=vq["scale"], v_zero=vq["zero"],
                         v_centroids=Cv))
        S, n = stats.update(S, n, Q[sl])
        prevk, prevv = Ck, Cv
    sl = w.chunk_slice(1)
    O, lse, top = A.cache_attention(Q[sl], segs, 1 / np.sqrt(128))
    # brute force: element-wise dequantization with Python loops for a few keys
    Kh = []
    Vh = []
    for sg in segs:
        for t in range(len(sg["k_idx"])):
            kk = np.array(sg["k_centroids"][sg["k_idx"][t]], dtype=np.float64)
            vv = np.array(sg["v_centroids"][sg["v_idx"][t]], dtype=np.float64)
            for c in range(128):
                g = c // 64
                kk[c] += sg["k_scale"][t, g] * (int(sg["k_q"][t, c]) - int(sg["k_zero"][t, g]))
                vv[c] += sg["v_scale"][t, g] * (int(sg["v_q"][t, c]) - int(sg["v_zero"][t, g]))
            if sg["U"] is not None:
                for j in range(8):
                    kk += sg["k_cs"][t] * int(sg["k_Cq"][t, j]) * sg["U"][:, j]
            Kh.append(kk)
            Vh.append(vv)
    O2, lse2, top2 = A.softmax_attention(Q[sl], np.array(Kh), np.array(Vh), 1 / np.sqrt(128))
    assert np.max(np.abs(O - O2)) <= 1e-12 * np.max(np.abs(O))
    np.testing.assert_array_equal(top, top2)
    # the quantized cache stays close to the bf16 attention
    Oref, _, topref = A.softmax_attention(Q[sl], K, V, 1 / np.sqrt(128))
    assert np.linalg.norm(O - Oref) / np.linalg.norm(Oref) < 0.2


def test_bf16_active_chunk_segment():
    """A BF16 segment (the active chunk, QuantWM App. D.1) is read as its raw
    values.  Pins: (1) attention over [packed, BF16] is the log-sum-exp merge
    of the attentions over each part alone (softmax over a union of key sets);
    (2) a BF16 segment that holds a packed segment's reconstruction attends
    exactly like the packed segment."""
    w = datagen.make_workload("480p", heads=[0], n_chunks=2, chunk=300)
    K, V, Q = (w.K[:, 0].astype(np.float64), w.V[:, 0].astype(np.float64),
               w.Q[:, 0].astype(np.float64))
    sl0, sl1 = w.chunk_slice(0), w.chunk_slice(1)
    Ck = lloyd.lloyd(K[sl0], 256, 2, seed=11)
    Cv = lloyd.lloyd(V[sl0], 256, 2, seed=12)
    kq = Qz.quantize_keys(K[sl0], Ck, None, None, M=8)
    vq = Qz.quantize_values(V[sl0], Cv)
    packed = dict(k_idx=kq["idx"], k_q=kq["q"], k_scale=kq["scale"], k_zero=kq["zero"], k_Cq=kq["Cq"],
                  k_cs=kq["c_scale"], k_centroids=Ck, U=None, v_idx=vq["idx"], v_q=vq["q"],
                  v_scale=vq["scale"], v_zero=vq["zero"], v_centroids=Cv)
    active = dict(k_bf16=K[sl1], v_bf16=V[sl1])
    sc = 1 / np.sqrt(128)
    O, lse, top = A.cache_attention(Q[sl1], [packed, active], sc)
    Oa, la, ta = A.cache_attention(Q[sl1], [packed], sc)
    Ob, lb, tb = A.cache_attention(Q[sl1], [active], sc)
    m = np.maximum(la, lb)
    wa, wb = np.exp(la - m), np.exp(lb - m)
    merged = (wa[:, None] * Oa + wb[:, None] * Ob) / (wa + wb)[:, None]
    assert np.max(np.abs(O - merged)) <= 1e-12 * np.max(np.abs(O))
    np.testing.assert_allclose(lse, m + np.log(wa + wb), rtol=0, atol=1e-12)
    Kd, Vd = A.segment_kv(packed)
    O2, lse2, top2 = A.cache_attention(Q[sl1], [dict(k_bf16=Kd, v_bf16=Vd), active], sc)
    assert np.array_equal(O, O2) and np.array_equal(top, top2)


def test_decode_segment_is_the_rounded_reconstruction():
    """Decode (QuantWM App. D.1 / Fig. 9): bf16 values within half a bf16 ulp of
    the exact reconstruction; a key whose residual and PSAC terms vanish decodes
    to its centroid exactly."""
    from oracle import formats as F
    w = datagen.make_workload("480p", heads=[0], n_chunks=1, chunk=300)
    K, V, Q = (w.K[:, 0].astype(np.float64), w.V[:, 0].astype(np.float64), w.Q[:, 0].astype(np.float64))
    Ck = lloyd.lloyd(K, 256, 2, seed=11)
    Cv = lloyd.lloyd(V, 256, 2, seed=12)
    S, n = stats.update(np.zeros((128, 128)), 0, Q)
    U = stats.principal_basis(S, n)["U_bf16"]
    kq = Qz.quantize_keys(K, Ck, stats.channel_weights(S, n), U, M=8)
    vq = Qz.quantize_values(V, Cv)
    seg = dict(k_idx=kq["idx"], k_q=kq["q"], k_scale=kq["scale"], k_zero=kq["zero"], k_Cq=kq["Cq"],
               k_cs=kq["c_scale"], k_centroids=Ck, U=U, v_idx=vq["idx"], v_q=vq["q"], v_scale=vq["scale"],
               v_zero=vq["zero"], v_centroids=Cv)
    Kx, Vx = A.segment_kv(seg)
    Kd, Vd = A.decode_segment(seg)
    for X, Xd in ((Kx, Kd), (Vx, Vd)):
        assert np.array_equal(F.bf16_rne(Xd), Xd)                  # bf16 values
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(Xd), 1e-30))) - 7)
        assert np.all(np.abs(Xd - X) <= ulp / 2 + 1e-300)
    seg0 = dict(seg, k_scale=np.zeros_like(seg["k_scale"]), k_cs=np.zeros_like(seg["k_cs"]))
    K0, _ = A.decode_segment(seg0)
    assert np.array_equal(K0, np.asarray(Ck, np.float64)[np.asarray(kq["idx"], np.int64)])
