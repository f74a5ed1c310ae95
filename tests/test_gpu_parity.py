"""GPU parity of every hot-path stage against the CPU oracle, on the same seeded
inputs, through the C ABI.  Bars: bit-exact centroid indices, INT2 codes,
scales and zero-points (mismatches allowed only at counted near-ties of
relative gap < 1e-6); PSAC INT8 coefficients within +-1 LSB and their scale
within one fp16 ulp; w within 1e-6 relative; U within one bf16 ulp; attention
relative L2 <= 2e-3 against the oracle run on the same packed cache."""
import sys

import numpy as np
import pytest

import datagen
from oracle import attention as OA
from oracle import formats as F
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
    import bit_kv_cache_head_amd as q     # raises when the HIP library is missing
    return q


# ---------------------------------------------------------------------------
# Query statistics and principal basis
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,dtype", [("480p", "bf16"), ("tiny", "f32")])
def test_query_stats_and_basis(qwm, name, dtype):
    import torch
    from gpu_helpers import dev_tokens, host
    _log(f"stats {name}")
    w = datagen.make_workload(name, heads=[0, 1, 2] if name == "480p" else None, n_chunks=2, chunk=300,
                              n_queries=None if name == "480p" else 333)
    H = w.H
    st = qwm.QueryStats(H)
    # cold start: no Queries yet -> w = 1, no basis
    qwm.update_query_stats(dev_tokens(w.Q[:0], dtype), st, compute_basis=True)
    torch.cuda.synchronize()
    assert torch.all(st.w == 1) and torch.all(st.n == 0) and torch.all(st.U.float() == 0)
    Qs = [w.Q[:150], w.Q[150:]] if name == "480p" else [w.Q]
    S = [np.zeros((128, 128)) for _ in range(H)]
    n = [0] * H
    for Qc in Qs:
        qwm.update_query_stats(dev_tokens(Qc, dtype), st, compute_basis=True)
        for h in range(H):
            S[h], n[h] = OS.update(S[h], n[h], Qc[:, h])
    torch.cuda.synchronize()
    for h in range(H):
        # Each 16-token MFMA partial is a sum of exact products rounded in fp32 before
        # it is added in fp64: |dS_ij| <= gamma_16 sum_t |q_ti q_tj| <= gamma_16 sqrt(S_ii S_jj)
        # (Cauchy-Schwarz), gamma_16 = 16u / (1 - 16u) < 1e-6 with u = 2^-24; fp32 Queries
        # take the fp64 path (error ~1e-16).
        gamma = 1e-6 if dtype == "bf16" else 1e-13
        dS = np.abs(st.S[h].cpu().numpy() - S[h])
        bound = gamma * np.sqrt(np.outer(np.diag(S[h]), np.diag(S[h])))
        assert np.all(dS <= bound), float(np.max(dS / bound))
        assert int(st.n[h]) == n[h]
        np.testing.assert_allclose(st.w[h].cpu().numpy(), OS.channel_weights(S[h], n[h]), rtol=1e-6)
        b = OS.principal_basis(S[h], n[h])
        assert int(st.iters[h]) > 0, "eigen-iteration did not converge"
        Ug = host(st.U[h])
        ulp = np.ldexp(1.0, np.frexp(np.abs(b["U_bf16"]))[1] - 8)
        assert np.all(np.abs(Ug - b["U_bf16"]) <= ulp), np.max(np.abs(Ug - b["U_bf16"]) / ulp)
        np.testing.assert_allclose(st.lam[h].cpu().numpy(), b["lam"], rtol=1e-6)
        assert abs(float(st.energy[h]) - b["energy"]) < 1e-6


def test_basis_rank_deficient(qwm):
    """Fewer Queries than basis columns: M_h has rank 5, so only the top five
    eigenpairs are unique.  They must match the oracle; the rest of the basis
    must stay finite and orthonormal (to bf16 precision), with zero Ritz
    values."""
    import torch
    from gpu_helpers import dev_tokens, host
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=5)
    Qc = w.Q[:5]
    st = qwm.QueryStats(2)
    qwm.update_query_stats(dev_tokens(Qc, "bf16"), st, compute_basis=True)
    torch.cuda.synchronize()
    for h in range(2):
        S, n = OS.update(np.zeros((128, 128)), 0, Qc[:, h])
        b = OS.principal_basis(S, n)
        Ug = host(st.U[h])
        assert np.all(np.isfinite(Ug))
        ulp = np.ldexp(1.0, np.frexp(np.abs(b["U_bf16"][:, :5]))[1] - 8)
        assert np.all(np.abs(Ug[:, :5] - b["U_bf16"][:, :5]) <= ulp)
        np.testing.assert_allclose(Ug.T @ Ug, np.eye(8), atol=2e-2)
        lam = st.lam[h].cpu().numpy()
        np.testing.assert_allclose(lam[:5], b["lam"][:5], rtol=1e-6)
        assert np.all(np.abs(lam[5:]) <= 1e-6 * lam[0])


# ---------------------------------------------------------------------------
# Lloyd centroid tables
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,dtype,T", [("480p", "bf16", 777), ("tiny", "f32", 600)])
def test_lloyd_tables(qwm, name, dtype, T):
    import torch
    from gpu_helpers import dev_tokens, dev_table, host
    _log(f"lloyd {name} T={T}")
    w = datagen.make_workload(name, heads=[0, 1] if name == "480p" else None, n_chunks=1, chunk=T)
    X = w.K
    H = w.H
    seed = 1234
    diag = qwm.new_diag()
    Cg = qwm.build_centroids(dev_tokens(X, dtype), iters=4, seed=seed, diag=diag)
    torch.cuda.synchronize()
    for h in range(H):
        Co = OL.lloyd(X[:, h].astype(np.float64), 256, 4, seed=seed, head=h)
        np.testing.assert_array_equal(host(Cg[h]), Co)
    # warm start from a given table, two more iterations
    init = np.stack([OL.lloyd(X[:, h].astype(np.float64), 256, 1, seed=7, head=h) for h in range(H)])
    Cw = qwm.build_centroids(dev_tokens(X, dtype), iters=2, init=dev_table(init), diag=diag)
    torch.cuda.synchronize()
    for h in range(H):
        Co = OL.lloyd(X[:, h].astype(np.float64), 256, 2, init=init[h])
        np.testing.assert_array_equal(host(Cw[h]), Co)
    _log(f"  diag {diag.tolist()}")
    assert int(diag[0]) == 0


@pytest.mark.parametrize("name,dtype,T", [("480p", "bf16", 777), ("tiny", "f32", 600)])
def test_lloyd_tables_fine_values(qwm, name, dtype, T):
    """A head holding a channel value far finer than the channel's largest
    (here 2^-100 against O(1)) cannot keep exact 64-bit fixed-point member
    sums: that head takes the fp64 sums, the other head the integer ones, and
    both tables match the oracle bit for bit over 6 iterations, seeded."""
    import torch
    from gpu_helpers import dev_tokens, host
    _log(f"lloyd with a fine value {name} T={T}")
    w = datagen.make_workload(name, heads=[0, 1] if name == "480p" else None, n_chunks=1, chunk=T)
    X = w.K.copy()
    H = w.H
    X[T // 3, 0, 17] = 2.0 ** -100     # exact in bf16 and fp32
    X[T // 2, 0, 40] = -3.0 * 2.0 ** -90
    seed = 4242
    Cg = qwm.build_centroids(dev_tokens(X, dtype), iters=6, seed=seed)
    torch.cuda.synchronize()
    for h in range(H):
        Co = OL.lloyd(X[:, h].astype(np.float64), 256, 6, seed=seed, head=h)
        np.testing.assert_array_equal(host(Cg[h]), Co)


@pytest.mark.parametrize("name,dtype,T", [("480p", "bf16", 777), ("tiny", "f32", 600)])
def test_lloyd_tables_nonfinite_rows(qwm, name, dtype, T):
    """Rows with a NaN or infinite channel take no part in the table: Forgy
    picks that land on them are dropped (the shuffle goes on), and they are no
    cluster's members.  Against the oracle, seeded and warm-started."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, host
    _log(f"lloyd with non-finite rows {name} T={T}")
    w = datagen.make_workload(name, heads=[0, 1] if name == "480p" else None, n_chunks=1, chunk=T)
    X = w.K.copy()
    H = w.H
    seed = 99
    for h in range(H):
        picks = OL.forgy_indices(T, 256, seed, h)
        bad = [int(picks[3]), int(picks[200]), 0, T - 1, T // 2 + h]   # two of them Forgy picks
        X[bad[0], h, 5] = np.nan
        X[bad[1], h, :] = np.inf
        X[bad[2], h, 127] = -np.inf
        X[bad[3], h, 64] = np.nan
        X[bad[4], h, 0] = np.inf
    nbad = sum(int((~OL.finite_rows(X[:, h])).sum()) for h in range(H))
    diag = qwm.new_diag()
    Cg = qwm.build_centroids(dev_tokens(X, dtype), iters=3, seed=seed, diag=diag)
    torch.cuda.synchronize()
    for h in range(H):
        Co = OL.lloyd(X[:, h].astype(np.float64), 256, 3, seed=seed, head=h)
        assert np.all(np.isfinite(Co))
        np.testing.assert_array_equal(host(Cg[h]), Co)
    assert int(diag[0]) == nbad          # once per call: later iterations skip excluded rows
    init = np.stack([OL.lloyd(X[:, h].astype(np.float64), 256, 1, seed=7, head=h) for h in range(H)])
    Cw = qwm.build_centroids(dev_tokens(X, dtype), iters=2, init=dev_table(init))
    torch.cuda.synchronize()
    for h in range(H):
        np.testing.assert_array_equal(host(Cw[h]), OL.lloyd(X[:, h].astype(np.float64), 256, 2, init=init[h]))


# ---------------------------------------------------------------------------
# Key and value quantization
# ---------------------------------------------------------------------------
def _key_inputs(name, T, heads, seed=5):
    w = datagen.make_workload(name, heads=heads, n_chunks=2, chunk=T,
                              n_queries=None if name != "tiny" else 400)
    K = w.K[T:2 * T] if name != "tiny" else w.K[:T]
    H = w.H
    tables, ws, Us = [], [], []
    for h in range(H):
        prev = w.K[:T, h].astype(np.float64)
        tables.append(OL.lloyd(prev, 256, 3, seed=seed, head=h))
        S, n = OS.update(np.zeros((128, 128)), 0, w.Q[: min(T, w.Q.shape[0]), h])
        ws.append(OS.channel_weights(S, n))
        Us.append(OS.principal_basis(S, n)["U_bf16"])
    return w, K, np.stack(tables), np.stack(ws), np.stack(Us)


@pytest.mark.parametrize("flags,M", [(3, 8), (1, 8), (2, 8), (0, 8), (3, 1), (3, 4), (3, 16), (3, 256), (7, 8), (6, 8),
                                     (7, 16), (7, 256)])
def test_quantize_keys(qwm, flags, M):
    import torch
    from gpu_helpers import dev_tokens, dev_table, dev_basis, packed_host, idx_mismatches_allowed, compare_codec
    _log(f"keys flags={flags} M={M}")
    T = 777
    w, K, Ct, wt, Ut = _key_inputs("480p", T, [0, 1])
    H = w.H
    diag = qwm.new_diag()
    wdev = torch.from_numpy(wt).cuda()
    out = qwm.quantize_keys(dev_tokens(K, "bf16"), dev_table(Ct), wdev, dev_basis(Ut), M=M, flags=flags,
                            diag=diag)
    torch.cuda.synchronize()
    g = packed_host(out)
    total_mis = 0
    for h in range(H):
        o = Qz.quantize_keys(K[:, h].astype(np.float64), Ct[h], wt[h], Ut[h], M=M, flags=flags)
        kind = "qsac" if flags & 1 else "nearest"
        nmis, nbad = idx_mismatches_allowed(kind, o, g["idx"][h], K[:, h], Ct[h], w=wt[h], M=M)
        assert nbad == 0, f"head {h}: {nbad} centroid choices differ beyond near-ties"
        total_mis += nmis
        same = o["idx"] == g["idx"][h]
        compare_codec(o, {k: v[h] for k, v in g.items()}, T, same)
        if flags & 4:
            # keep test: decisions agree except near ties.  The kernel decides in
            # fp32 on coefficients within 1 LSB of the oracle's, so a tie is a
            # criterion below the effect of one LSB in every coefficient plus
            # fp32 rounding: 2 c_s sum_c w_c sum_r |U_cr| (|D_c| + |E_c| + c_s |U_cr|)
            # + 2^-16 sum_c w_c (D_c^2 + E_c^2)
            full = Qz.quantize_keys(K[:, h].astype(np.float64), Ct[h], wt[h], Ut[h], M=M, flags=flags & ~4)
            ki = o["keep"]
            g_keep = (g["c_scale_bits"][h] != 0) | np.any(g["c"][h] != 0, axis=1)
            mu = np.asarray(Ct[h], np.float64)[np.asarray(o["idx"], np.int64)]
            E = K[:, h].astype(np.float64) - (mu + o["r_hat"])
            Ua = np.abs(np.asarray(Ut[h], np.float64))
            cs = full["c_scale"]
            D = (cs[:, None] * full["Cq"].astype(np.float64)) @ np.asarray(Ut[h], np.float64).T
            wk = np.asarray(wt[h], np.float32).astype(np.float64) if flags & 1 else np.ones(128)
            tol = (2 * cs * np.sum(wk * Ua.sum(axis=1)[None, :] * (np.abs(D) + np.abs(E) + cs[:, None]), axis=1)
                   + 2.0 ** -16 * np.sum(wk * (D * D + E * E), axis=1))
            dis = same & (g_keep != ki["keep"])
            assert np.all(np.abs(ki["crit"][dis]) <= tol[dis]), np.nonzero(dis)[0][:5]
            same = same & (g_keep == ki["keep"])
            _log(f"  head {h}: kept {ki['keep'].mean():.3f}, decision near-ties {int(dis.sum())}")
        if flags & 2:
            dc = np.abs(g["c"][h].astype(np.int64) - o["Cq"].astype(np.int64))
            assert dc[same].max() <= 1
            gs = F.bits_to_fp16(g["c_scale_bits"][h])
            os_ = o["c_scale"]
            ulp = np.ldexp(1.0, np.frexp(np.maximum(os_, 6.1e-5))[1] - 11)
            assert np.all(np.abs(gs - os_)[same] <= ulp[same])
            _log(f"  head {h}: C exact {np.mean(dc[same] == 0):.5f}, c_scale exact {np.mean(gs[same] == os_[same]):.5f}")
        else:
            assert np.all(g["c"][h] == 0) and np.all(g["c_scale_bits"][h] == 0)
    _log(f"  idx near-tie mismatches {total_mis}, diag {diag.tolist()}")


@pytest.mark.parametrize("flags,M", [(3, 8), (7, 4), (1, 1), (3, 256)])
def test_quantize_keys_full_matrix(qwm, flags, M):
    """QSAC candidates by the full Query second-moment matrix (App. C.4
    ablation) against the oracle's direct quadratic form."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, dev_basis, packed_host, idx_mismatches_allowed, compare_codec
    _log(f"keys full-matrix flags={flags} M={M}")
    T = 400
    w, K, Ct, wt, Ut = _key_inputs("480p", T, [0, 1])
    H = w.H
    Ss, ns = [], []
    for h in range(H):
        S, n = OS.update(np.zeros((128, 128)), 0, w.Q[: min(T, w.Q.shape[0]), h])
        Ss.append(S)
        ns.append(n)
    diag = qwm.new_diag()
    out = qwm.quantize_keys_fullq(dev_tokens(K, "bf16"), dev_table(Ct), torch.from_numpy(np.stack(Ss)).cuda(),
                                  torch.tensor(ns, dtype=torch.int64).cuda(), torch.from_numpy(wt).cuda(),
                                  dev_basis(Ut), M=M, flags=flags, diag=diag)
    torch.cuda.synchronize()
    g = packed_host(out)
    total_mis = 0
    for h in range(H):
        Mq = Qz.second_moment(Ss[h], ns[h])
        o = Qz.quantize_keys(K[:, h].astype(np.float64), Ct[h], wt[h], Ut[h], M=M, flags=flags | Qz.QSAC_FULL, Mq=Mq)
        nmis, nbad = idx_mismatches_allowed("qsac", o, g["idx"][h], K[:, h], Ct[h], w=wt[h], M=M)
        assert nbad == 0, f"head {h}: {nbad} centroid choices differ beyond near-ties"
        total_mis += nmis
        same = o["idx"] == g["idx"][h]
        compare_codec(o, {k: v[h] for k, v in g.items()}, T, same)
        g_keep = (g["c_scale_bits"][h] != 0) | np.any(g["c"][h] != 0, axis=1)
        if flags & 4:
            # both sides decide the keep test in fp64 on coefficients within 1 LSB
            full = Qz.quantize_keys(K[:, h].astype(np.float64), Ct[h], wt[h], Ut[h], M=M,
                                    flags=(flags & ~4) | Qz.QSAC_FULL, Mq=Mq)
            ki = o["keep"]
            mu = np.asarray(Ct[h], np.float64)[np.asarray(o["idx"], np.int64)]
            E = K[:, h].astype(np.float64) - (mu + o["r_hat"])
            Ua = np.abs(np.asarray(Ut[h], np.float64))
            cs = full["c_scale"]
            D = (cs[:, None] * full["Cq"].astype(np.float64)) @ np.asarray(Ut[h], np.float64).T
            wk = np.asarray(wt[h], np.float32).astype(np.float64)
            tol = 2 * cs * np.sum(wk * Ua.sum(axis=1)[None, :] * (np.abs(D) + np.abs(E) + cs[:, None]), axis=1)
            dis = same & (g_keep != ki["keep"])
            assert np.all(np.abs(ki["crit"][dis]) <= tol[dis]), np.nonzero(dis)[0][:5]
            same = same & (g_keep == ki["keep"])
        if flags & 2:
            dc = np.abs(g["c"][h].astype(np.int64) - o["Cq"].astype(np.int64))
            assert dc[same].max() <= 1
        else:
            assert np.all(g["c"][h] == 0) and np.all(g["c_scale_bits"][h] == 0)
        _log(f"  head {h}: idx differs from the diagonal form on "
             f"{int(np.sum(o['idx'] != Qz.quantize_keys(K[:, h].astype(np.float64), Ct[h], wt[h], None, M=M, flags=1)['idx']))} tokens")
    _log(f"  idx near-tie mismatches {total_mis}, diag {diag.tolist()}")


def test_quantize_keys_full_matrix_cold_start(qwm):
    """n = 0: M_h = I and w = 1, i.e. the Euclidean QSAC choice."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, packed_host, idx_mismatches_allowed, compare_codec
    T = 300
    w, K, Ct, wt, Ut = _key_inputs("480p", T, [0, 1])
    H = w.H
    out = qwm.quantize_keys_fullq(dev_tokens(K, "bf16"), dev_table(Ct),
                                  torch.zeros(H, 128, 128, dtype=torch.float64).cuda(),
                                  torch.zeros(H, dtype=torch.int64).cuda(), None, None, M=8, flags=1)
    torch.cuda.synchronize()
    g = packed_host(out)
    for h in range(H):
        o = Qz.quantize_keys(K[:, h].astype(np.float64), Ct[h], None, None, M=8, flags=1)
        nmis, nbad = idx_mismatches_allowed("qsac", o, g["idx"][h], K[:, h], Ct[h], None, 8)
        assert nbad == 0
        compare_codec(o, {k: v[h] for k, v in g.items()}, T, o["idx"] == g["idx"][h])


@pytest.mark.parametrize("T,dtype", [(1, "bf16"), (129, "f32"), (257, "bf16")])
def test_quantize_keys_full_matrix_shapes(qwm, T, dtype):
    """Full-matrix QSAC at a single token, a ragged fp32 chunk and a ragged bf16
    chunk (the kernel's grid covers four tokens per block)."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, dev_basis, packed_host, idx_mismatches_allowed, compare_codec
    w, K, Ct, wt, Ut = _key_inputs("480p", 300, [0, 1])   # tables from 300 tokens (Forgy needs >= 256)
    K = np.ascontiguousarray(K[:T])
    H = w.H
    Ss, ns = [], []
    for h in range(H):
        S, n = OS.update(np.zeros((128, 128)), 0, w.Q[:300, h])
        Ss.append(S)
        ns.append(n)
    out = qwm.quantize_keys_fullq(dev_tokens(K, dtype), dev_table(Ct), torch.from_numpy(np.stack(Ss)).cuda(),
                                  torch.tensor(ns, dtype=torch.int64).cuda(), torch.from_numpy(wt).cuda(),
                                  dev_basis(Ut), M=8, flags=3)
    torch.cuda.synchronize()
    g = packed_host(out)
    for h in range(H):
        o = Qz.quantize_keys(K[:, h].astype(np.float64), Ct[h], wt[h], Ut[h], M=8, flags=3 | Qz.QSAC_FULL,
                             Mq=Qz.second_moment(Ss[h], ns[h]))
        nmis, nbad = idx_mismatches_allowed("qsac", o, g["idx"][h], K[:, h], Ct[h], w=wt[h], M=8)
        assert nbad == 0
        same = o["idx"] == g["idx"][h]
        compare_codec(o, {k: v[h] for k, v in g.items()}, T, same)
        dc = np.abs(g["c"][h].astype(np.int64) - o["Cq"].astype(np.int64))
        assert dc[same].max() <= 1


@pytest.mark.parametrize("M", [8, 16])
def test_quantize_keys_keep_rejections(qwm, M):
    """The keep test where it rejects often: strongly non-uniform weights and a
    random basis (not the weights' eigenvectors), so the compensation raises the
    weighted error of about a fifth of the keys.  At M = 16 many tokens take the
    exact fp64 path, which must apply the test too."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, dev_basis, packed_host, idx_mismatches_allowed, compare_codec
    T = 777
    w, K, Ct, _, _ = _key_inputs("480p", T, [0, 1])
    rng = np.random.default_rng(7)
    wq = np.exp(rng.uniform(-3, 3, (2, 128))).astype(np.float32)
    Ur = np.stack([F.bf16_rne(np.linalg.qr(rng.standard_normal((128, 8)))[0]) for _ in range(2)])
    diag = qwm.new_diag()
    out = qwm.quantize_keys(dev_tokens(K, "bf16"), dev_table(Ct), torch.from_numpy(wq).cuda(), dev_basis(Ur),
                            M=M, flags=7, diag=diag)
    torch.cuda.synchronize()
    g = packed_host(out)
    for h in range(2):
        o = Qz.quantize_keys(K[:, h].astype(np.float64), Ct[h], wq[h], Ur[h], M=M, flags=7)
        nmis, nbad = idx_mismatches_allowed("qsac", o, g["idx"][h], K[:, h], Ct[h], w=wq[h], M=M)
        assert nbad == 0
        same = o["idx"] == g["idx"][h]
        compare_codec(o, {k: v[h] for k, v in g.items()}, T, same)
        full = Qz.quantize_keys(K[:, h].astype(np.float64), Ct[h], wq[h], Ur[h], M=M, flags=3)
        ki = o["keep"]
        assert (~ki["keep"]).sum() > 50
        g_keep = (g["c_scale_bits"][h] != 0) | np.any(g["c"][h] != 0, axis=1)
        mu = np.asarray(Ct[h], np.float64)[np.asarray(o["idx"], np.int64)]
        E = K[:, h].astype(np.float64) - (mu + o["r_hat"])
        Ua = np.abs(np.asarray(Ur[h], np.float64))
        cs = full["c_scale"]
        D = (cs[:, None] * full["Cq"].astype(np.float64)) @ np.asarray(Ur[h], np.float64).T
        wk = wq[h].astype(np.float64)
        tol = (2 * cs * np.sum(wk * Ua.sum(axis=1)[None, :] * (np.abs(D) + np.abs(E) + cs[:, None]), axis=1)
               + 2.0 ** -16 * np.sum(wk * (D * D + E * E), axis=1))
        dis = same & (g_keep != ki["keep"])
        assert np.all(np.abs(ki["crit"][dis]) <= tol[dis]), np.nonzero(dis)[0][:5]
        agree = same & (g_keep == ki["keep"])
        dc = np.abs(g["c"][h].astype(np.int64) - o["Cq"].astype(np.int64))
        assert dc[agree].max() <= 1
        _log(f"  M={M} head {h}: rejected {int((~ki['keep']).sum())}, decision near-ties {int(dis.sum())}, "
             f"diag {diag.tolist()}")


@pytest.mark.parametrize("M", [8, 256])
def test_quantize_keys_cold_start_and_fp32(qwm, M):
    """Chunk 0: w = 1 and no basis (PSAC inactive); fp32 tokens.  M = 256: every
    centroid a candidate (the exhaustive variant of the selection kernel)."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, packed_host, idx_mismatches_allowed, compare_codec
    _log(f"fp32 keys M={M}")
    T = 600
    w, K, Ct, wt, Ut = _key_inputs("tiny", T, None)
    out = qwm.quantize_keys(dev_tokens(K, "f32"), dev_table(Ct), None, None, M=M, flags=3)
    torch.cuda.synchronize()
    g = packed_host(out)
    o = Qz.quantize_keys(K[:, 0].astype(np.float64), Ct[0], None, None, M=M, flags=3)
    nmis, nbad = idx_mismatches_allowed("qsac", o, g["idx"][0], K[:, 0], Ct[0], None, M)
    assert nbad == 0
    compare_codec(o, {k: v[0] for k, v in g.items()}, T, o["idx"] == g["idx"][0])
    assert np.all(g["c"] == 0)
    # fp32 with weights and PSAC
    wdev = torch.from_numpy(wt).cuda()
    from gpu_helpers import dev_basis
    out = qwm.quantize_keys(dev_tokens(K, "f32"), dev_table(Ct), wdev, dev_basis(Ut), M=M, flags=3)
    torch.cuda.synchronize()
    g = packed_host(out)
    o = Qz.quantize_keys(K[:, 0].astype(np.float64), Ct[0], wt[0], Ut[0], M=M, flags=3)
    nmis, nbad = idx_mismatches_allowed("qsac", o, g["idx"][0], K[:, 0], Ct[0], wt[0], M)
    assert nbad == 0
    same = o["idx"] == g["idx"][0]
    compare_codec(o, {k: v[0] for k, v in g.items()}, T, same)
    assert np.abs(g["c"][0].astype(int) - o["Cq"].astype(int))[same].max() <= 1


@pytest.mark.parametrize("T", [777, 1, 64, 129])
def test_quantize_values(qwm, T):
    import torch
    from gpu_helpers import dev_tokens, dev_table, packed_host, idx_mismatches_allowed, compare_codec
    _log(f"values T={T}")
    w = datagen.make_workload("480p", heads=[3, 4], n_chunks=2, chunk=max(T, 300))
    V = w.V[-T:]
    Ct = np.stack([OL.lloyd(w.V[:300, h].astype(np.float64), 256, 2, seed=9, head=h) for h in range(2)])
    out = qwm.quantize_values(dev_tokens(V, "bf16"), dev_table(Ct))
    torch.cuda.synchronize()
    g = packed_host(out)
    for h in range(2):
        o = Qz.quantize_values(V[:, h].astype(np.float64), Ct[h])
        nmis, nbad = idx_mismatches_allowed("nearest", o, g["idx"][h], V[:, h], Ct[h])
        assert nbad == 0
        compare_codec(o, {k: v[h] for k, v in g.items()}, T, o["idx"] == g["idx"][h])


def test_nonfinite_and_degenerate_tokens(qwm):
    import torch
    from gpu_helpers import dev_tokens, dev_table, packed_host
    w = datagen.make_workload("480p", heads=[0], n_chunks=1, chunk=300)
    K = w.K.copy()
    Ct = OL.lloyd(K[:, 0].astype(np.float64), 256, 2, seed=3, head=0)[None]
    K[5, 0, 7] = np.nan
    K[9, 0, 100] = np.inf
    K[11, 0] = Ct[0, 17]            # exactly a centroid: zero residual, zero scales
    diag = qwm.new_diag()
    out = qwm.quantize_keys(dev_tokens(K, "bf16"), dev_table(Ct), None, None, M=8, flags=1, diag=diag)
    torch.cuda.synchronize()
    g = packed_host(out)
    for t in (5, 9):
        assert g["idx"][0, t] == 0 and np.all(g["codes"][0, t] == 0) and np.all(g["scale_bits"][0, t] == 0)
    assert int(diag[0]) == 2
    assert g["idx"][0, 11] == 17 and np.all(g["scale_bits"][0, 11] == 0) and np.all(g["codes"][0, 11] == 0)
    z = F.unpack_zeros(g["zeros"][0, :150], 300)
    assert np.all(z[11] == 0) and np.all(z[5] == 0)
    o = Qz.quantize_keys(np.delete(K[:, 0], [5, 9], axis=0).astype(np.float64), Ct[0], None, None, M=8, flags=1)
    keep = np.delete(np.arange(300), [5, 9])
    np.testing.assert_array_equal(g["idx"][0, keep], o["idx"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scale_saturation(qwm, dtype):
    """Residual ranges past 3 x 65504 and PSAC coefficients past 127 x 65504:
    the fp16 scales saturate at 65504 and are counted (the degenerate-input
    reading); codes, scales, zero-points and c_scale bit for bit against the
    oracle, C within 1 LSB, the counter equal to the oracle's saturations."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, dev_basis, packed_host, idx_mismatches_allowed, compare_codec
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=400)
    K = w.K.copy()
    Ct = np.stack([OL.lloyd(K[:, h].astype(np.float64), 256, 2, seed=5, head=h) for h in range(2)])
    rng = np.random.default_rng(21)
    Ub = np.stack([F.bf16_rne(datagen.haar_orthogonal(rng, 128)[:, :8]) for _ in range(2)])
    wt = rng.uniform(0.2, 3.0, (2, 128)).astype(np.float32)
    # group 0 of token 3: range 4e5 (scale 4e5 / 3 > 65504); token 7: group 1 at +-1e7
    # (both scales saturate, and the uncoded error drives |C| past 127 x 65504);
    # token 11: -3e5 in one channel; token 12: one channel at 2e5, just past the limit
    for h in range(2):
        K[3, h, 10] = 4.0e5
        K[7, h, 64:] = np.where(np.arange(64) % 2 == 0, 1.0e7, -1.0e7)
        K[11, h, 100] = -3.0e5
        K[12, h, 5] = 2.0e5
    if dtype == "bf16":
        K = F.bf16_rne(K.astype(np.float64)).astype(np.float32)
    diag = qwm.new_diag()
    kp = qwm.quantize_keys(dev_tokens(K, dtype), dev_table(Ct), torch.from_numpy(wt).cuda(), dev_basis(Ub), M=8,
                           flags=3, diag=diag)
    torch.cuda.synchronize()
    g = packed_host(kp)
    want_sat = 0
    for h in range(2):
        o = Qz.quantize_keys(K[:, h].astype(np.float64), Ct[h], wt[h], Ub[h], M=8, flags=3)
        nmis, nbad = idx_mismatches_allowed("qsac", o, g["idx"][h], K[:, h], Ct[h], w=wt[h], M=8)
        assert nbad == 0
        same = o["idx"] == g["idx"][h]
        assert same[[3, 7, 11, 12]].all()
        compare_codec(o, {k: v[h] for k, v in g.items()}, 400, same)
        assert np.array_equal(g["c_scale_bits"][h][same], o["c_scale_bits"][same])
        assert np.abs(g["c"][h].astype(np.int64) - o["Cq"].astype(np.int64))[same].max() <= 1
        sat_c = int(np.sum(np.max(np.abs(o["C_raw"]), axis=1) > 127.0 * 65504.0))
        assert o["saturated"] >= 4 and sat_c >= 1
        for t in (3, 7, 11, 12):
            assert 0x7BFF in g["scale_bits"][h][t]
        assert g["c_scale_bits"][h][7] == 0x7BFF
        want_sat += o["saturated"] + sat_c
    _log(f"  saturations: {int(diag[2])} (oracle {want_sat})")
    assert int(diag[2]) == want_sat


# ---------------------------------------------------------------------------
# Attention over the compressed cache
# ---------------------------------------------------------------------------
def _oracle_segments(w, chunk_sizes, heads):
    """Quantize consecutive chunks with the oracle (its own tables, stats and
    basis), returning per-segment per-head dicts and packed arrays."""
    H = len(heads)
    segs = []
    S = [np.zeros((128, 128)) for _ in range(H)]
    n = [0] * H
    prevk = [None] * H
    prevv = [None] * H
    pos = 0
    for ci, T in enumerate(chunk_sizes):
        sl = slice(pos, pos + T)
        per = []
        for h in range(H):
            Kc = w.K[sl, h].astype(np.float64)
            Vc = w.V[sl, h].astype(np.float64)
            iters = 2 if prevk[h] is not None else 3
            if T >= 256 or prevk[h] is not None:
                Ck = OL.lloyd(Kc, 256, iters, seed=21, head=h, init=prevk[h])
                Cv = OL.lloyd(Vc, 256, iters, seed=22, head=h, init=prevv[h])
            else:   # a first chunk shorter than the table: seed it from 256 later tokens
                Ck = OL.lloyd(w.K[-256:, h].astype(np.float64), 256, 1, seed=21, head=h)
                Cv = OL.lloyd(w.V[-256:, h].astype(np.float64), 256, 1, seed=22, head=h)
            U = OS.principal_basis(S[h], n[h])["U_bf16"] if n[h] else None
            kq = Qz.quantize_keys(Kc, Ck, OS.channel_weights(S[h], n[h]), U, M=8)
            vq = Qz.quantize_values(Vc, Cv)
            per.append(dict(k=kq, v=vq, Ck=Ck, Cv=Cv, U=U,
                            oracle=dict(k_idx=kq["idx"], k_q=kq["q"], k_scale=kq["scale"], k_zero=kq["zero"],
                                        k_Cq=kq["Cq"], k_cs=kq["c_scale"], k_centroids=Ck, U=U,
                                        v_idx=vq["idx"], v_q=vq["q"], v_scale=vq["scale"], v_zero=vq["zero"],
                                        v_centroids=Cv)))
            S[h], n[h] = OS.update(S[h], n[h], w.Q[sl, h])
            prevk[h], prevv[h] = Ck, Cv
        segs.append(per)
        pos += T
    return segs


def _upload_segments(qwm, segs, H):
    import torch
    from gpu_helpers import upload_packed, dev_table, dev_basis
    keep = []
    lst = []
    for per in segs:
        T = len(per[0]["k"]["idx"])
        kp = upload_packed(qwm.PackedChunk, H, T, True, [p["k"] for p in per])
        vp = upload_packed(qwm.PackedChunk, H, T, False, [p["v"] for p in per])
        kc = dev_table(np.stack([p["Ck"] for p in per]))
        vc = dev_table(np.stack([p["Cv"] for p in per]))
        U = None if per[0]["U"] is None else dev_basis(np.stack([p["U"] for p in per]))
        keep.append((kp, vp, kc, vc, U))
        lst.append((kp, vp, kc, vc, U))
    dseg = qwm.segment_array(lst)
    total = dseg.total
    return dseg, total, keep


@pytest.mark.parametrize("want_top1,sizes", [(True, [300, 257, 64, 1, 130]), (False, [300, 257, 64, 1, 130]),
                                              (True, [64, 1, 130])])
def test_attention_on_oracle_cache(qwm, want_top1, sizes):
    import torch
    from gpu_helpers import dev_tokens
    _log(f"attention oracle cache {sizes}")
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=sum(sizes) + 256)
    segs = _oracle_segments(w, sizes, [0, 1])
    dseg, total, keep = _upload_segments(qwm, segs, 2)
    Qv = w.Q[-200:]
    out, lse, top1 = qwm.attention(dev_tokens(Qv, "bf16"), dseg, want_lse=True,
                                   want_top1=want_top1)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for h in range(2):
        O, L, top = OA.cache_attention(Qv[:, h].astype(np.float64), [s[h]["oracle"] for s in segs],
                                       1 / np.sqrt(128))
        err = np.linalg.norm(out[:, h] - O) / np.linalg.norm(O)
        _log(f"  head {h}: rel L2 {err:.2e}")
        assert err <= 2e-3
        np.testing.assert_allclose(lse.cpu().numpy()[h], L, rtol=1e-4, atol=1e-4)
        if want_top1:
            _check_top1(top1.cpu().numpy()[h], top, Qv[:, h], segs, h)


@pytest.mark.parametrize("tq", [1, 33, 257, 513])
def test_attention_query_counts(qwm, tq):
    """One Query, a ragged wave, and query blocks of 256 whose last block holds
    a single Query (its other waves idle), against the oracle."""
    import torch
    from gpu_helpers import dev_tokens
    sizes = [300, 130]
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=sum(sizes) + 600)
    segs = _oracle_segments(w, sizes, [0, 1])
    dseg, total, keep = _upload_segments(qwm, segs, 2)
    Qv = w.Q[-tq:]
    out, lse, top1 = qwm.attention(dev_tokens(Qv, "bf16"), dseg, want_lse=True, want_top1=True)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for h in range(2):
        O, L, top = OA.cache_attention(Qv[:, h].astype(np.float64), [s[h]["oracle"] for s in segs], 1 / np.sqrt(128))
        err = np.linalg.norm(out[:, h] - O) / np.linalg.norm(O)
        assert err <= 2e-3, (tq, h, err)
        np.testing.assert_allclose(lse.cpu().numpy()[h], L, rtol=1e-4, atol=1e-4)
        _check_top1(top1.cpu().numpy()[h], top, Qv[:, h], segs, h)


def _slice_quantized(o: dict, sl: slice, keys: bool) -> dict:
    """Token range sl of one head's oracle quantization, repacked as a chunk of its own."""
    r = {"idx": o["idx"][sl], "q": o["q"][sl], "scale": o["scale"][sl], "zero": o["zero"][sl],
         "scale_bits": o["scale_bits"][sl], "codes": F.pack_codes(o["q"][sl]), "zeros": F.pack_zeros(o["zero"][sl])}
    if keys:
        r.update(Cq=o["Cq"][sl], c_scale=o["c_scale"][sl], c_scale_bits=o["c_scale_bits"][sl])
    return r


def test_attention_over_many_small_segments(qwm):
    """150 segments of 1..40 keys (more than the 64 descriptors a wave scans at
    once when it locates its share, one-key segments, a ragged tile in almost
    every segment), all with PSAC, against the oracle over the same segments."""
    import torch
    from gpu_helpers import dev_tokens
    rng = np.random.default_rng(12)
    sizes = [int(x) for x in rng.integers(1, 41, 150)]
    sizes[3] = sizes[70] = 1
    T = sum(sizes)
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=T + 600)
    per_head = []
    for h in range(2):
        Ck = OL.lloyd(w.K[-512:, h].astype(np.float64), 256, 2, seed=31, head=h)
        Cv = OL.lloyd(w.V[-512:, h].astype(np.float64), 256, 2, seed=32, head=h)
        S, n = OS.update(np.zeros((128, 128)), 0, w.Q[-300:, h])
        U = OS.principal_basis(S, n)["U_bf16"]
        kq = Qz.quantize_keys(w.K[:T, h].astype(np.float64), Ck, OS.channel_weights(S, n), U, M=8)
        vq = Qz.quantize_values(w.V[:T, h].astype(np.float64), Cv)
        per_head.append((Ck, Cv, U, kq, vq))
    segs, pos = [], 0
    for Tn in sizes:
        sl = slice(pos, pos + Tn)
        per = []
        for h in range(2):
            Ck, Cv, U, kq, vq = per_head[h]
            k, v = _slice_quantized(kq, sl, True), _slice_quantized(vq, sl, False)
            per.append(dict(k=k, v=v, Ck=Ck, Cv=Cv, U=U,
                            oracle=dict(k_idx=k["idx"], k_q=k["q"], k_scale=k["scale"], k_zero=k["zero"],
                                        k_Cq=k["Cq"], k_cs=k["c_scale"], k_centroids=Ck, U=U,
                                        v_idx=v["idx"], v_q=v["q"], v_scale=v["scale"], v_zero=v["zero"],
                                        v_centroids=Cv)))
        segs.append(per)
        pos += Tn
    dseg, total, keep = _upload_segments(qwm, segs, 2)
    assert total == T
    Qv = w.Q[-130:]
    out, lse, _ = qwm.attention(dev_tokens(Qv, "bf16"), dseg, want_lse=True)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for h in range(2):
        O, L, _ = OA.cache_attention(Qv[:, h].astype(np.float64), [s[h]["oracle"] for s in segs], 1 / np.sqrt(128))
        err = np.linalg.norm(out[:, h] - O) / np.linalg.norm(O)
        _log(f"  150 segments, head {h}: rel L2 {err:.2e}")
        assert err <= 2e-3
        np.testing.assert_allclose(lse.cpu().numpy()[h], L, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("split", [1, 2, 4])
def test_attention_merge_of_two_parts(qwm, split):
    """Attention over the first `split` segments and over the rest, joined by
    qwm_attention_merge, against the oracle over all of them; out written over
    the first part's buffer (allowed aliasing)."""
    import torch
    from gpu_helpers import dev_tokens
    sizes = [300, 257, 64, 1, 130]
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=sum(sizes) + 256)
    segs = _oracle_segments(w, sizes, [0, 1])
    da, ta, ka = _upload_segments(qwm, segs[:split], 2)
    db, tb, kb = _upload_segments(qwm, segs[split:], 2)
    Qv = w.Q[-200:]
    Qd = dev_tokens(Qv, "bf16")
    oa, la, _ = qwm.attention(Qd, da, want_lse=True)
    ob, lb, _ = qwm.attention(Qd, db, want_lse=True)
    out, lse = qwm.attention_merge(oa, la, ob, lb, out=oa, want_lse=True)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for h in range(2):
        O, L, _ = OA.cache_attention(Qv[:, h].astype(np.float64), [s[h]["oracle"] for s in segs], 1 / np.sqrt(128))
        err = np.linalg.norm(out[:, h] - O) / np.linalg.norm(O)
        _log(f"  split {split} head {h}: rel L2 {err:.2e}")
        assert err <= 2e-3
        np.testing.assert_allclose(lse.cpu().numpy()[h], L, rtol=1e-4, atol=1e-4)
    # a part without keys (lse = -inf) leaves the other unchanged
    empty_l = torch.full_like(lb, -float("inf"))
    o2, l2 = qwm.attention_merge(ob, lb, torch.zeros_like(ob), empty_l, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, ob) and torch.equal(l2, lb)


@pytest.mark.parametrize("sizes,active", [([300, 257], 173), ([64], 1), ([], 130), ([], 1), ([130, 1], 64)])
def test_attention_with_bf16_active_chunk(qwm, sizes, active):
    """Packed chunks plus the BF16 active chunk (QuantWM App. D.1): the active
    chunk's K/V are strided [T, H, 128] views of the token arrays, its length
    ragged against the 64-key tile; with no packed chunk at all as well."""
    import torch
    from gpu_helpers import dev_tokens
    _log(f"attention with a BF16 active chunk: packed {sizes}, active {active}")
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=sum(sizes) + active + 256)
    segs = _oracle_segments(w, sizes, [0, 1]) if sizes else []
    dseg, total, keep = _upload_segments(qwm, segs, 2) if sizes else (None, 0, [])
    pos = sum(sizes)
    assert total == pos
    Kall = dev_tokens(w.K, "bf16")
    Vall = dev_tokens(w.V, "bf16")
    Kact, Vact = Kall[pos:pos + active], Vall[pos:pos + active]    # views: stride_t = H * 128
    Qv = w.Q[-200:]
    out, lse, top1 = qwm.attention(dev_tokens(Qv, "bf16"), dseg, want_lse=True, want_top1=True,
                                   active=(Kact, Vact))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for h in range(2):
        osegs = [s[h]["oracle"] for s in segs] + [dict(k_bf16=w.K[pos:pos + active, h].astype(np.float64),
                                                       v_bf16=w.V[pos:pos + active, h].astype(np.float64))]
        O, L, top = OA.cache_attention(Qv[:, h].astype(np.float64), osegs, 1 / np.sqrt(128))
        err = np.linalg.norm(out[:, h] - O) / np.linalg.norm(O)
        Kcat = np.concatenate([OA.segment_kv(sg)[0] for sg in osegs])
        # LSE is 1-Lipschitz in the max-norm of the logits.  The kernel's logits
        # use fp16 K0_hat (one RNE rounding, <= 2^-11 relative per element) and
        # the fp16 PSAC product; its sum uses fp16 probabilities rounded toward
        # zero (< 2^-10 relative each).  Bound per Query: scale * 2^-10 *
        # max_j sum_c |q_c k_jc| (the K0_hat term, doubled for the PSAC and fp32
        # terms) + 2^-9.
        qa = np.abs(Qv[:, h].astype(np.float64))
        tol = (1 / np.sqrt(128)) * 2.0 ** -10 * np.max(qa @ np.abs(Kcat).T, axis=1) + 2.0 ** -9
        lerr = np.abs(lse.cpu().numpy()[h] - L)
        _log(f"  head {h}: rel L2 {err:.2e}, max |lse error| {lerr.max():.2e} (bound >= {tol.min():.2e})")
        assert err <= 2e-3
        assert np.all(lerr <= tol)
        Lg = Qv[:, h].astype(np.float64) @ Kcat.T
        gt = top1.cpu().numpy()[h]
        for i in np.nonzero(gt != top)[0]:
            a, b = Lg[i, top[i]], Lg[i, gt[i]]
            assert abs(a - b) <= 1e-3 * abs(a), (i, a, b)


def test_decode_segment_and_dense_attention(qwm):
    """The decoder of QuantWM App. D.1 / Fig. 9 (BF16 reconstruction of packed
    chunks, PSAC included): bit-exact against the oracle's rounded exact
    values; then attention over the decoded rows as one dense chunk matches
    the oracle's attention over the same bf16 values."""
    import torch
    from gpu_helpers import dev_tokens
    sizes = [300, 130, 64]
    _log(f"decode {sizes}")
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=sum(sizes) + 256)
    segs = _oracle_segments(w, sizes, [0, 1])
    _, _, keep = _upload_segments(qwm, segs, 2)
    total = sum(sizes)
    Kd = torch.empty(total, 2, 128, dtype=torch.bfloat16, device="cuda")
    Vd = torch.empty_like(Kd)
    pos = 0
    for (kp, vp, kc, vc, U), T in zip(keep, sizes):
        qwm.decode_segment(kp, vp, kc, vc, U, Kd[pos:pos + T], Vd[pos:pos + T])
        pos += T
    torch.cuda.synchronize()
    Kg, Vg = Kd.float().cpu().numpy(), Vd.float().cpu().numpy()
    pos = 0
    for si, T in enumerate(sizes):
        for h in range(2):
            Ko, Vo = OA.decode_segment(segs[si][h]["oracle"])
            assert np.array_equal(Kg[pos:pos + T, h], Ko), (si, h)
            assert np.array_equal(Vg[pos:pos + T, h], Vo), (si, h)
        pos += T
    Qv = w.Q[-200:]
    out, lse, _ = qwm.attention(dev_tokens(Qv, "bf16"), None, want_lse=True, active=(Kd, Vd))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for h in range(2):
        O, L, _ = OA.softmax_attention(Qv[:, h].astype(np.float64), Kg[:, h].astype(np.float64),
                                       Vg[:, h].astype(np.float64), 1 / np.sqrt(128))
        err = np.linalg.norm(out[:, h] - O) / np.linalg.norm(O)
        _log(f"  dense over decoded rows, head {h}: rel L2 {err:.2e}")
        assert err <= 2e-3


@pytest.mark.parametrize("stages", [1, 2, 3])
def test_prq_quantize(qwm, stages):
    """QVG's progressive residual quantization (summary Sec. 2B): every stage's
    table and assignment and the last stage's codes, bit-exact against the
    oracle (fp32 stage residuals on both sides)."""
    import torch
    from gpu_helpers import dev_tokens, packed_host, compare_codec
    from oracle import prq
    _log(f"prq {stages} stages")
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=600)
    X = dev_tokens(w.K, "bf16")
    first, C_last, last = qwm.prq_quantize(X, stages, iters=3, seed=9)
    torch.cuda.synchronize()
    for h in range(2):
        ofirst, oC, olast, _ = prq.prq_quantize(w.K[:, h].astype(np.float64), stages, 3, seed=9, head=h)
        for (C, idx), (Co, ao) in zip(first, ofirst):
            assert np.array_equal(C[h].float().cpu().numpy(), Co)
            assert np.array_equal(idx[h].cpu().numpy(), ao)
        assert np.array_equal(C_last[h].float().cpu().numpy(), oC)
        g = packed_host(last)
        assert np.array_equal(g["idx"][h], olast["idx"])
        compare_codec(olast, {k: v[h] for k, v in g.items()}, 600, np.ones(600, bool))


def _check_top1(gt, ot, Qh, segs, h):
    """Top-1 agrees except where the oracle's top-2 logit gap is < 1e-3 relative."""
    from gpu_helpers import check_top1_near_tie
    check_top1_near_tie(gt, ot, Qh, [s[h]["oracle"] for s in segs])


def test_attention_full_shape_random_cache(qwm):
    """480p step shape: 25 segments x 1,560 keys, 1,560 queries, 12 heads, the
    bench's launch configuration; seeded random packed cache; sampled queries."""
    import torch
    from gpu_helpers import dev_tokens, upload_packed, dev_table, dev_basis, check_top1_near_tie
    _log("attention full shape")
    rng = np.random.default_rng(77)
    H, T, nseg, Tq = 12, 1560, 25, 1560
    lst, oracle_segs = [], []
    for s in range(nseg):
        kh, vh, ors = [], [], []
        Ck = F.bf16_rne(rng.standard_normal((H, 256, 128)) * 2)
        Cv = F.bf16_rne(rng.standard_normal((H, 256, 128)) * 2)
        U = None
        if s > 0:
            U = np.stack([F.bf16_rne(datagen.haar_orthogonal(rng, 128)[:, :8]) for _ in range(H)])
        for h in range(H):
            def one(keys):
                q = rng.integers(0, 4, (T, 128)).astype(np.uint8)
                z = rng.integers(0, 4, (T, 2)).astype(np.uint8)
                sc = (rng.uniform(0.01, 0.2, (T, 2))).astype(np.float16).astype(np.float64)
                d = dict(q=q, zero=z, scale=sc, idx=rng.integers(0, 256, T).astype(np.uint8),
                         codes=F.pack_codes(q), zeros=F.pack_zeros(z), scale_bits=F.fp16_bits(sc))
                if keys:
                    d["Cq"] = rng.integers(-127, 128, (T, 8)).astype(np.int8)
                    d["c_scale"] = rng.uniform(1e-4, 1e-3, T).astype(np.float16).astype(np.float64)
                    d["c_scale_bits"] = F.fp16_bits(d["c_scale"])
                return d
            kq, vq = one(True), one(False)
            kh.append(kq)
            vh.append(vq)
            ors.append(dict(k_idx=kq["idx"], k_q=kq["q"], k_scale=kq["scale"], k_zero=kq["zero"], k_Cq=kq["Cq"],
                            k_cs=kq["c_scale"], k_centroids=Ck[h], U=None if U is None else U[h],
                            v_idx=vq["idx"], v_q=vq["q"], v_scale=vq["scale"], v_zero=vq["zero"],
                            v_centroids=Cv[h]))
        kp = upload_packed(qwm.PackedChunk, H, T, True, kh)
        vp = upload_packed(qwm.PackedChunk, H, T, False, vh)
        lst.append((kp, vp, dev_table(Ck), dev_table(Cv), None if U is None else dev_basis(U)))
        oracle_segs.append(ors)
    dseg = qwm.segment_array(lst)
    total = dseg.total
    Qv = datagen.make_workload("480p", heads=list(range(H)), n_chunks=1, chunk=Tq).Q
    out, lse, top1 = qwm.attention(dev_tokens(Qv, "bf16"), dseg, want_lse=True, want_top1=True)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    sample = np.array([0, 1, 127, 128, 777, 1535, 1536, 1559])
    for h in (0, 5, 11):
        O, L, top = OA.cache_attention(Qv[sample, h].astype(np.float64), [s[h] for s in oracle_segs],
                                       1 / np.sqrt(128))
        err = np.linalg.norm(out[sample, h] - O) / np.linalg.norm(O)
        _log(f"  head {h}: rel L2 {err:.2e}")
        assert err <= 2e-3
        np.testing.assert_allclose(lse.cpu().numpy()[h, sample], L, rtol=1e-4, atol=1e-4)
        check_top1_near_tie(top1.cpu().numpy()[h, sample], top, Qv[sample, h], [s[h] for s in oracle_segs])


# ---------------------------------------------------------------------------
# Streaming pipeline, end to end, and determinism
# ---------------------------------------------------------------------------
def test_streaming_pipeline_end_to_end(qwm):
    """Three 300-token chunks, 2 heads: GPU pipeline (stats -> basis -> Lloyd ->
    keys -> values -> attention) against the oracle pipeline from the same inputs."""
    import torch
    from gpu_helpers import dev_tokens, packed_host, host
    _log("pipeline")
    H, T, nch = 2, 300, 3
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=nch, chunk=T)
    st = qwm.QueryStats(H)
    ref = _oracle_segments(w, [T] * nch, [0, 1])
    gsegs = []
    prev = (None, None)
    for c in range(nch):
        sl = w.chunk_slice(c)
        K, V = dev_tokens(w.K[sl], "bf16"), dev_tokens(w.V[sl], "bf16")
        if c == 0:
            Ck = qwm.build_centroids(K, 3, seed=21)
            Cv = qwm.build_centroids(V, 3, seed=22)
            kp = qwm.quantize_keys(K, Ck, None, None, M=8, flags=3)
            U = None
        else:
            Ck = qwm.build_centroids(K, 2, init=prev[0])
            Cv = qwm.build_centroids(V, 2, init=prev[1])
            U = st.U.clone()
            kp = qwm.quantize_keys(K, Ck, st.w.clone(), U, M=8, flags=3)
        vp = qwm.quantize_values(V, Cv)
        qwm.update_query_stats(dev_tokens(w.Q[sl], "bf16"), st, compute_basis=True)
        torch.cuda.synchronize()
        for h in range(H):
            np.testing.assert_array_equal(host(Ck[h]), ref[c][h]["Ck"])
            np.testing.assert_array_equal(host(Cv[h]), ref[c][h]["Cv"])
            gk = packed_host(kp)
            assert np.mean(gk["idx"][h] == ref[c][h]["k"]["idx"]) == 1.0
        gsegs.append((kp, vp, Ck, Cv, U))
        prev = (Ck, Cv)
    dseg = qwm.segment_array(gsegs)
    total = dseg.total
    Qv = w.Q[w.chunk_slice(nch - 1)]
    out, _, _ = qwm.attention(dev_tokens(Qv, "bf16"), dseg)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for h in range(H):
        O, _, _ = OA.cache_attention(Qv[:, h].astype(np.float64), [s[h]["oracle"] for s in ref], 1 / np.sqrt(128))
        assert np.linalg.norm(out[:, h] - O) / np.linalg.norm(O) <= 2e-3


def test_determinism(qwm):
    import torch
    from gpu_helpers import dev_tokens, packed_host
    w = datagen.make_workload("480p", heads=[0, 1, 2], n_chunks=1, chunk=1000)
    K = dev_tokens(w.K, "bf16")
    C1 = qwm.build_centroids(K, 3, seed=5)
    C2 = qwm.build_centroids(K, 3, seed=5)
    st = qwm.QueryStats(3)
    qwm.update_query_stats(dev_tokens(w.Q, "bf16"), st)
    a = packed_host(qwm.quantize_keys(K, C1, st.w, st.U, M=8, flags=3))
    b = packed_host(qwm.quantize_keys(K, C2, st.w, st.U, M=8, flags=3))
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
