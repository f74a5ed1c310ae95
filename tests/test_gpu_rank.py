"""The PSAC rank ablation (QuantWM App. C.2, Table 9: r = 8, 16, 32) on the
GPU against the oracle: the principal basis of rank r, the keys' coefficients,
the BF16 decoder and the fused attention over chunks of mixed ranks."""
import sys

import numpy as np
import pytest

import datagen
from oracle import attention as OA
from oracle import lloyd as OL
from oracle import quantize as Qz
from oracle import stats as OS

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def qwm():
    import torch
    assert torch.cuda.is_available()
    import bit_kv_cache_head_amd as q
    return q


@pytest.mark.parametrize("r", [16, 32])
def test_basis_of_rank(qwm, r):
    """Top-r eigenpairs of M_h: U within one bf16 ulp per entry, eigenvalues and
    the energy share to 1e-6, against the oracle's cyclic Jacobi."""
    import torch
    from gpu_helpers import dev_tokens, host
    _log(f"basis r={r}")
    w = datagen.make_workload("480p", heads=[0, 1, 2], n_chunks=1, chunk=1560)
    st = qwm.QueryStats(3, r=r)
    qwm.update_query_stats(dev_tokens(w.Q, "bf16"), st, compute_basis=True)
    torch.cuda.synchronize()
    for h in range(3):
        S, n = OS.update(np.zeros((128, 128)), 0, w.Q[:, h])
        b = OS.principal_basis(S, n, r=r)
        Ug = host(st.U[h])
        assert Ug.shape == (128, r)
        ulp = np.ldexp(1.0, np.frexp(np.abs(b["U_bf16"]))[1] - 8)
        assert np.all(np.abs(Ug - b["U_bf16"]) <= ulp), np.max(np.abs(Ug - b["U_bf16"]) / ulp)
        np.testing.assert_allclose(st.lam[h].cpu().numpy(), b["lam"], rtol=1e-6)
        assert abs(float(st.energy[h]) - b["energy"]) < 1e-6
        _log(f"  head {h}: sweeps {int(st.iters[h])}, energy {float(st.energy[h]):.4f}")
        assert int(st.iters[h]) > 0


def test_basis_of_rank_deficient(qwm):
    """Five Queries, rank 16: the five nonzero eigenpairs match the oracle; the
    rest of the basis is finite, orthonormal and has zero eigenvalues."""
    import torch
    from gpu_helpers import dev_tokens, host
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=5)
    st = qwm.QueryStats(2, r=16)
    qwm.update_query_stats(dev_tokens(w.Q[:5], "bf16"), st, compute_basis=True)
    torch.cuda.synchronize()
    for h in range(2):
        S, n = OS.update(np.zeros((128, 128)), 0, w.Q[:5, h])
        b = OS.principal_basis(S, n, r=16)
        Ug = host(st.U[h])
        assert np.all(np.isfinite(Ug))
        ulp = np.ldexp(1.0, np.frexp(np.abs(b["U_bf16"][:, :5]))[1] - 8)
        assert np.all(np.abs(Ug[:, :5] - b["U_bf16"][:, :5]) <= ulp)
        np.testing.assert_allclose(Ug.T @ Ug, np.eye(16), atol=2e-2)
        lam = st.lam[h].cpu().numpy()
        np.testing.assert_allclose(lam[:5], b["lam"][:5], rtol=1e-6)
        assert np.all(np.abs(lam[5:]) <= 1e-6 * lam[0])


def _inputs(r, T=777, heads=(0, 1)):
    w = datagen.make_workload("480p", heads=list(heads), n_chunks=2, chunk=T)
    K = w.K[T:2 * T]
    tables, ws, Us = [], [], []
    for h in range(len(heads)):
        tables.append(OL.lloyd(w.K[:T, h].astype(np.float64), 256, 3, seed=5, head=h))
        S, n = OS.update(np.zeros((128, 128)), 0, w.Q[:T, h])
        ws.append(OS.channel_weights(S, n))
        Us.append(OS.principal_basis(S, n, r=r)["U_bf16"])
    return w, K, np.stack(tables), np.stack(ws), np.stack(Us)


@pytest.mark.parametrize("r,flags", [(16, 3), (32, 3), (16, 7), (32, 2), (16, 0)])
def test_keys_of_rank(qwm, r, flags):
    """Keys with a rank-r basis: indices and codes bit-exact, C within one LSB,
    c_scale within one fp16 ulp; the keep test's decisions equal except where
    the criterion is at rounding level."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, dev_basis, packed_host, idx_mismatches_allowed, compare_codec
    _log(f"keys r={r} flags={flags}")
    T = 777
    w, K, Ct, wt, Ut = _inputs(r, T)
    diag = qwm.new_diag()
    out = qwm.quantize_keys(dev_tokens(K, "bf16"), dev_table(Ct), torch.from_numpy(wt).cuda(), dev_basis(Ut), M=8,
                            flags=flags, diag=diag)
    torch.cuda.synchronize()
    assert out.r == r and tuple(out.c.shape) == (2, T, r)
    g = packed_host(out)
    for h in range(2):
        o = Qz.quantize_keys(K[:, h].astype(np.float64), Ct[h], wt[h], Ut[h], M=8, flags=flags)
        kind = "qsac" if flags & 1 else "nearest"
        nmis, nbad = idx_mismatches_allowed(kind, o, g["idx"][h], K[:, h], Ct[h], w=wt[h], M=8)
        assert nbad == 0
        same = o["idx"] == g["idx"][h]
        compare_codec(o, {k: v[h] for k, v in g.items()}, T, same)
        if flags & 4:
            g_keep = (g["c_scale_bits"][h] != 0) | np.any(g["c"][h] != 0, axis=1)
            dis = same & (g_keep != o["keep"]["keep"])
            # both sides decide in fp64 from the same coefficients: only criteria at
            # rounding level may differ
            crit, base = o["keep"]["crit"], o["keep"]["base"]
            assert np.all(np.abs(crit[dis]) <= 1e-12 * (base[dis] + 1e-300)), np.nonzero(dis)[0][:5]
            same = same & ~dis
        dc = np.abs(g["c"][h].astype(np.int64) - o["Cq"].astype(np.int64))[same]
        assert dc.max(initial=0) <= 1
        cs_g = g["c_scale_bits"][h][same].astype(np.int64)
        cs_o = o["c_scale_bits"][same].astype(np.int64)
        assert np.abs(cs_g - cs_o).max(initial=0) <= 1
        _log(f"  head {h}: {nmis} near-ties, C off by one LSB: {int((dc == 1).sum())}, "
             f"c_scale off by one ulp: {int((cs_g != cs_o).sum())}")


def _segments_of_ranks(w, sizes, ranks, H):
    """Oracle-quantized consecutive chunks, chunk i with PSAC rank ranks[i]
    (None: a cold-start chunk without basis)."""
    segs = []
    S = [np.zeros((128, 128)) for _ in range(H)]
    n = [0] * H
    pos = 0
    for T, r in zip(sizes, ranks):
        sl = slice(pos, pos + T)
        per = []
        for h in range(H):
            Kc, Vc = w.K[sl, h].astype(np.float64), w.V[sl, h].astype(np.float64)
            src = slice(pos, pos + T) if T >= 256 else slice(-256, None)   # a short chunk: a table from 256 later tokens
            Ck = OL.lloyd(w.K[src, h].astype(np.float64), 256, 2, seed=31, head=h)
            Cv = OL.lloyd(w.V[src, h].astype(np.float64), 256, 2, seed=32, head=h)
            U = OS.principal_basis(S[h], n[h], r=r)["U_bf16"] if (n[h] and r) else None
            kq = Qz.quantize_keys(Kc, Ck, OS.channel_weights(S[h], n[h]), U, M=8)
            if U is None and r:
                kq["Cq"] = np.zeros((T, r), np.int8)    # stored width of a chunk coded without basis
            vq = Qz.quantize_values(Vc, Cv)
            per.append(dict(k=dict(codes=kq["codes"], idx=kq["idx"], scale_bits=kq["scale_bits"], zeros=kq["zeros"],
                                   Cq=kq["Cq"], c_scale_bits=kq["c_scale_bits"]),
                            v=dict(codes=vq["codes"], idx=vq["idx"], scale_bits=vq["scale_bits"], zeros=vq["zeros"]),
                            Ck=Ck, Cv=Cv, U=U,
                            oracle=dict(k_idx=kq["idx"], k_q=kq["q"], k_scale=kq["scale"], k_zero=kq["zero"],
                                        k_Cq=kq["Cq"], k_cs=kq["c_scale"], k_centroids=Ck, U=U,
                                        v_idx=vq["idx"], v_q=vq["q"], v_scale=vq["scale"], v_zero=vq["zero"],
                                        v_centroids=Cv)))
            S[h], n[h] = OS.update(S[h], n[h], w.Q[sl, h])
        segs.append(per)
        pos += T
    return segs


def _upload(qwm, segs, H):
    from gpu_helpers import upload_packed, dev_table, dev_basis
    keep = []
    for per in segs:
        T = len(per[0]["k"]["idx"])
        kp = upload_packed(qwm.PackedChunk, H, T, True, [p["k"] for p in per])
        vp = upload_packed(qwm.PackedChunk, H, T, False, [p["v"] for p in per])
        kc = dev_table(np.stack([p["Ck"] for p in per]))
        vc = dev_table(np.stack([p["Cv"] for p in per]))
        U = None if per[0]["U"] is None else dev_basis(np.stack([p["U"] for p in per]))
        keep.append((kp, vp, kc, vc, U))
    return keep


@pytest.mark.parametrize("ranks", [(8, 16, 16, 8), (16, 32, 8, 32), (32, 32, 32, 32)])
def test_attention_and_decode_of_mixed_ranks(qwm, ranks):
    """Chunks of ranks 8, 16 and 32 in one attention call (the first chunk a
    cold start), against the oracle's attention over the same packed chunks;
    the decoder bit-exact per chunk."""
    import torch
    from gpu_helpers import dev_tokens, check_top1_near_tie
    sizes = [300, 257, 64, 130]
    _log(f"attention over ranks {ranks}")
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=sum(sizes) + 200)
    segs = _segments_of_ranks(w, sizes, ranks, 2)
    keep = _upload(qwm, segs, 2)
    Qv = w.Q[-200:]
    out, lse, top1 = qwm.attention(dev_tokens(Qv, "bf16"), qwm.segment_array(keep), want_lse=True, want_top1=True)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for h in range(2):
        oseg = [s[h]["oracle"] for s in segs]
        O, L, top = OA.cache_attention(Qv[:, h].astype(np.float64), oseg, 1 / np.sqrt(128))
        err = np.linalg.norm(out[:, h] - O) / np.linalg.norm(O)
        _log(f"  head {h}: rel L2 {err:.2e}")
        assert err <= 2e-3
        np.testing.assert_allclose(lse.cpu().numpy()[h], L, rtol=1e-4, atol=1e-4)
        check_top1_near_tie(top1.cpu().numpy()[h], top, Qv[:, h], oseg)
    for si, ((kp, vp, kc, vc, U), T) in enumerate(zip(keep, sizes)):
        Kd, Vd = qwm.decode_segment(kp, vp, kc, vc, U)
        torch.cuda.synchronize()
        for h in range(2):
            Ko, Vo = OA.decode_segment(segs[si][h]["oracle"])
            assert np.array_equal(Kd[:, h].float().cpu().numpy(), Ko), (si, h)
            assert np.array_equal(Vd[:, h].float().cpu().numpy(), Vo), (si, h)
