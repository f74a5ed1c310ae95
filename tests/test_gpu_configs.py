"""GPU parity at the five workloads' real shapes, in the launch configurations
the library uses for them (all heads, full chunk lengths, full caches).

The oracle is slow, so it checks sampled heads (and, for the 28,000-token
depth chunk, sampled tokens) of every GPU call; every input it uses is its own
or seeded (tables from its Forgy seeding or its Lloyd, statistics from its
update).  Attention at full shape runs on seeded random packed caches, checked
on sampled Queries.  The tiny workload runs end to end.
"""
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


def _forgy_tables(X, seed):
    """Oracle Forgy seeding for every head of X [T, H, d]: [H, 256, 128]."""
    return np.stack([F.bf16_rne(X[OL.forgy_indices(X.shape[0], 256, seed, h), h].astype(np.float64))
                     for h in range(X.shape[1])])


def _check_keys(kind, o, g, h, K, C, w, M, flags, rows=None):
    """GPU packed keys of head h against the oracle's dict o (on `rows`)."""
    from gpu_helpers import idx_mismatches_allowed, compare_codec
    gi = g["idx"][h] if rows is None else g["idx"][h][rows]
    nmis, nbad = idx_mismatches_allowed(kind, o, gi, K, C, w=w, M=M)
    assert nbad == 0, f"{nbad} centroid choices differ beyond near-ties"
    same = o["idx"] == gi
    sub = {k: (v[h] if rows is None else v[h][rows]) for k, v in g.items() if k != "zeros"}
    if rows is None:
        sub["zeros"] = g["zeros"][h]
        compare_codec(o, sub, len(o["idx"]), same)
    else:
        gq = F.unpack_codes(sub["codes"], 128)
        np.testing.assert_array_equal(gq[same], o["q"][same])
        np.testing.assert_array_equal(sub["scale_bits"][same], o["scale_bits"][same])
        gz = F.unpack_zeros(g["zeros"][h][: (g["idx"].shape[1] + 1) // 2], g["idx"].shape[1])[rows]
        np.testing.assert_array_equal(gz[same], o["zero"][same])
    if "c" in sub:
        if flags & 2:
            assert np.abs(sub["c"].astype(np.int64) - o["Cq"].astype(np.int64))[same].max() <= 1
        else:
            assert np.all(sub["c"] == 0)
    return nmis


# (name, f_energy): chunk lengths and head counts come from the workload itself
FULL = [("480p", None), ("720p", 0.60), ("720p", 0.71), ("depth", None), ("rollout", None)]


@pytest.mark.parametrize("name,f", FULL)
def test_full_size_stages(qwm, name, f):
    """Statistics + basis, Forgy seeding, a Lloyd iteration, keys (every
    ablation on the rollout workload) and values on one full chunk of the
    workload, all heads on the GPU; the oracle checks sampled heads."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, dev_basis, host, packed_host
    _log(f"full-size stages {name} f={f}")
    w = datagen.make_workload(name, n_chunks=1, f_energy=f)
    H, T = w.H, w.chunk
    heads = [0, H - 1]
    K, V, Q = w.K[:T], w.V[:T], w.Q
    dK, dV = dev_tokens(K, "bf16"), dev_tokens(V, "bf16")

    # statistics and basis over the chunk's Queries
    st = qwm.QueryStats(H)
    qwm.update_query_stats(dev_tokens(Q, "bf16"), st, compute_basis=True)
    torch.cuda.synchronize()
    ob = {}
    for h in heads:
        S, n = OS.update(np.zeros((128, 128)), 0, Q[:, h])
        b = OS.principal_basis(S, n)
        ob[h] = (OS.channel_weights(S, n), b["U_bf16"])
        Ug = host(st.U[h])
        ulp = np.ldexp(1.0, np.frexp(np.abs(b["U_bf16"]))[1] - 8)
        assert np.all(np.abs(Ug - b["U_bf16"]) <= ulp)
        np.testing.assert_allclose(st.w[h].cpu().numpy(), ob[h][0], rtol=1e-6)
        np.testing.assert_allclose(st.lam[h].cpu().numpy(), b["lam"], rtol=1e-6)
    _log("  stats ok")

    # Forgy seeding (all heads) and one Lloyd iteration from it (sampled heads)
    C0 = _forgy_tables(K, 31)
    g0 = qwm.build_centroids(dK, 0, seed=31)
    g1 = qwm.build_centroids(dK, 1, init=dev_table(C0))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(g0), C0)
    g1h = host(g1)
    for h in heads:
        np.testing.assert_array_equal(g1h[h], OL.lloyd(K[:, h].astype(np.float64), 256, 1, init=C0[h]))
    _log("  centroids ok")

    # keys and values with the oracle's tables and statistics (head 0's w and U
    # on every head, head H-1's own where sampled)
    wt = np.stack([ob[heads[0]][0]] * H)
    Ub = np.stack([ob[heads[0]][1]] * H)
    wt[heads[1]], Ub[heads[1]] = ob[heads[1]][0], ob[heads[1]][1]
    rows = None if T <= 4096 else np.sort(np.random.default_rng(3).choice(T, 4096, replace=False))
    flag_set = [0, 1, 2, 3] if name == "rollout" else [3]
    for flags in flag_set:
        kp = qwm.quantize_keys(dK, dev_table(C0), torch.from_numpy(wt.astype(np.float32)).cuda(), dev_basis(Ub),
                               M=8, flags=flags)
        torch.cuda.synchronize()
        g = packed_host(kp)
        mis = 0
        for h in heads:
            Kh = K[:, h] if rows is None else K[rows, h]
            o = Qz.quantize_keys(Kh.astype(np.float64), C0[h], wt[h], Ub[h], M=8, flags=flags)
            kind = "qsac" if flags & 1 else "nearest"
            mis += _check_keys(kind, o, g, h, Kh, C0[h], wt[h] if flags & 1 else None, 8, flags, rows)
        _log(f"  keys flags={flags} ok ({mis} counted near-ties)")
    CV = _forgy_tables(V, 32)
    vp = qwm.quantize_values(dV, dev_table(CV))
    torch.cuda.synchronize()
    g = packed_host(vp)
    for h in heads:
        Vh = V[:, h] if rows is None else V[rows, h]
        o = Qz.quantize_values(Vh.astype(np.float64), CV[h])
        _check_keys("nearest", o, g, h, Vh, CV[h], None, 1, 0, rows)
    _log("  values ok")


def _random_cache(qwm, H, sizes, seed):
    """Seeded random packed cache: per segment and head, random codes, indices,
    zero-points, fp16 scales, INT8 coefficients and centroid tables, a basis
    for every segment but the first.  Heads differ (head h shifts the base
    draw), so a head mix-up cannot pass.  Returns the device segment array and
    a function giving the oracle's segment dicts for one head."""
    import torch
    from gpu_helpers import upload_packed, dev_table, dev_basis
    rng = np.random.default_rng(seed)
    keep, lst, base = [], [], []
    for s, T in enumerate(sizes):
        b = dict(q=rng.integers(0, 4, (T, 128)).astype(np.uint8), z=rng.integers(0, 4, (T, 2)).astype(np.uint8),
                 sc=rng.uniform(0.01, 0.2, (T, 2)).astype(np.float16).astype(np.float64),
                 idx=rng.integers(0, 256, T).astype(np.uint8), vidx=rng.integers(0, 256, T).astype(np.uint8),
                 Cq=rng.integers(-127, 128, (T, 8)).astype(np.int8),
                 cs=rng.uniform(1e-4, 1e-3, T).astype(np.float16).astype(np.float64),
                 Ck=F.bf16_rne(rng.standard_normal((256, 128)) * 2), Cv=F.bf16_rne(rng.standard_normal((256, 128)) * 2),
                 U=None if s == 0 else F.bf16_rne(datagen.haar_orthogonal(rng, 128)[:, :8]))
        base.append(b)

    def head(s, h):
        b = base[s]
        q = (b["q"] + h) % 4
        z = (b["z"] + (h % 3)) % 4
        idx = ((b["idx"].astype(np.int64) + 7 * h) % 256).astype(np.uint8)
        vidx = ((b["vidx"].astype(np.int64) + 11 * h) % 256).astype(np.uint8)
        Ck = np.roll(b["Ck"], h, axis=0)
        Cv = np.roll(b["Cv"], -h, axis=0)
        U = None if b["U"] is None else np.roll(b["U"], h, axis=0)
        return dict(k_idx=idx, k_q=q, k_scale=b["sc"], k_zero=z, k_Cq=b["Cq"], k_cs=b["cs"], k_centroids=Ck, U=U,
                    v_idx=vidx, v_q=(q + 1) % 4, v_scale=b["sc"][:, ::-1].copy(), v_zero=z[:, ::-1].copy(),
                    v_centroids=Cv)

    for s, T in enumerate(sizes):
        hs = [head(s, h) for h in range(H)]
        kd = [dict(codes=F.pack_codes(x["k_q"]), idx=x["k_idx"], scale_bits=F.fp16_bits(x["k_scale"]),
                   zeros=F.pack_zeros(x["k_zero"]), Cq=x["k_Cq"], c_scale_bits=F.fp16_bits(x["k_cs"])) for x in hs]
        vd = [dict(codes=F.pack_codes(x["v_q"]), idx=x["v_idx"], scale_bits=F.fp16_bits(x["v_scale"]),
                   zeros=F.pack_zeros(x["v_zero"])) for x in hs]
        kp = upload_packed(qwm.PackedChunk, H, T, True, kd)
        vp = upload_packed(qwm.PackedChunk, H, T, False, vd)
        kc = dev_table(np.stack([x["k_centroids"] for x in hs]))
        vc = dev_table(np.stack([x["v_centroids"] for x in hs]))
        U = None if hs[0]["U"] is None else dev_basis(np.stack([x["U"] for x in hs]))
        keep.append((kp, vp, kc, vc, U))
        lst.append((kp, vp, kc, vc, U))
        torch.cuda.synchronize()
    dseg = qwm.segment_array(lst)
    total = dseg.total
    return dseg, total, keep, (lambda h: [head(s, h) for s in range(len(sizes))])


# (name, segment sizes, queries, heads): the attention calls of the workloads
ATTN = [("720p", [3600] * 25, 3600, 40), ("depth", [28000], 1560, 40), ("rollout", [1560] * 40, 1560, 24),
        ("tiny", [4096], 512, 1)]


@pytest.mark.parametrize("name,sizes,tq,H", ATTN)
def test_attention_full_shapes(qwm, name, sizes, tq, H):
    import torch
    from gpu_helpers import dev_tokens, check_top1_near_tie
    _log(f"attention full shape {name}: H={H}, {len(sizes)} segments, {sum(sizes)} keys, {tq} queries")
    dseg, total, keep, oseg = _random_cache(qwm, H, sizes, seed={"720p": 71, "depth": 72, "rollout": 73, "tiny": 74}[name])
    dtype = "f32" if name == "tiny" else "bf16"
    Qv = datagen.make_workload(name, heads=list(range(H)), n_chunks=1, chunk=tq, n_queries=tq).Q
    out, lse, top1 = qwm.attention(dev_tokens(Qv, dtype), dseg, want_lse=True, want_top1=True)
    torch.cuda.synchronize()
    out, lse, top1 = out.cpu().numpy(), lse.cpu().numpy(), top1.cpu().numpy()
    sample = np.unique(np.array([0, 1, 31, 32, 255, 256, tq // 2, tq - 2, tq - 1]))
    for h in sorted({0, H // 2, H - 1}):
        Qh = Qv[sample, h].astype(np.float64)
        if dtype == "bf16":
            Qh = F.bf16_rne(Qh)
        O, L, top = OA.cache_attention(Qh, oseg(h), 1 / np.sqrt(128))
        err = np.linalg.norm(out[sample, h] - O) / np.linalg.norm(O)
        _log(f"  head {h}: rel L2 {err:.2e}")
        assert err <= 2e-3
        np.testing.assert_allclose(lse[h, sample], L, rtol=1e-4, atol=1e-4)
        nt = check_top1_near_tie(top1[h, sample], top, Qh, oseg(h))
        _log(f"  head {h}: top-1 ok ({nt} counted near-ties)")


def test_tiny_config_end_to_end(qwm):
    """The tiny workload in full: 4,096 fp32 keys and values, 512 Queries, one
    head; stats -> basis -> 10 seeded Lloyd iterations (K and V) -> QSAC+PSAC
    keys (M = 8) -> values -> attention, against the oracle pipeline."""
    import torch
    from gpu_helpers import dev_tokens, host, packed_host
    _log("tiny end to end")
    w = datagen.make_workload("tiny")
    K, V, Q = w.K, w.V, w.Q
    st = qwm.QueryStats(1)
    qwm.update_query_stats(dev_tokens(Q, "f32"), st, compute_basis=True)
    Ck = qwm.build_centroids(dev_tokens(K, "f32"), 10, seed=101)
    Cv = qwm.build_centroids(dev_tokens(V, "f32"), 10, seed=102)
    kp = qwm.quantize_keys(dev_tokens(K, "f32"), Ck, st.w, st.U, M=8, flags=3)
    vp = qwm.quantize_values(dev_tokens(V, "f32"), Cv)
    segs = qwm.segment_array([(kp, vp, Ck, Cv, st.U)])
    total = segs.total
    out, lse, top1 = qwm.attention(dev_tokens(Q, "f32"), segs, want_lse=True, want_top1=True)
    torch.cuda.synchronize()
    # oracle pipeline
    S, n = OS.update(np.zeros((128, 128)), 0, Q[:, 0])
    wts = OS.channel_weights(S, n)
    b = OS.principal_basis(S, n)
    oCk = OL.lloyd(K[:, 0].astype(np.float64), 256, 10, seed=101, head=0)
    oCv = OL.lloyd(V[:, 0].astype(np.float64), 256, 10, seed=102, head=0)
    np.testing.assert_array_equal(host(Ck[0]), oCk)
    np.testing.assert_array_equal(host(Cv[0]), oCv)
    Ug = host(st.U[0])
    ulp = np.ldexp(1.0, np.frexp(np.abs(b["U_bf16"]))[1] - 8)
    assert np.all(np.abs(Ug - b["U_bf16"]) <= ulp)
    _log("  stats, basis and tables ok")
    # keys are checked against the oracle run with the GPU-independent inputs
    # (its own tables, w and basis); the GPU's basis can differ by an ulp
    okq = Qz.quantize_keys(K[:, 0].astype(np.float64), oCk, wts, b["U_bf16"], M=8)
    ovq = Qz.quantize_values(V[:, 0].astype(np.float64), oCv)
    g = packed_host(kp)
    mis = _check_keys("qsac", okq, g, 0, K[:, 0], oCk, wts, 8, 3)
    _check_keys("nearest", ovq, packed_host(vp), 0, V[:, 0], oCv, None, 1, 0)
    _log(f"  keys and values ok ({mis} counted near-ties)")
    seg = dict(k_idx=okq["idx"], k_q=okq["q"], k_scale=okq["scale"], k_zero=okq["zero"], k_Cq=okq["Cq"],
               k_cs=okq["c_scale"], k_centroids=oCk, U=b["U_bf16"], v_idx=ovq["idx"], v_q=ovq["q"],
               v_scale=ovq["scale"], v_zero=ovq["zero"], v_centroids=oCv)
    O, L, top = OA.cache_attention(Q[:, 0].astype(np.float64), [seg], 1 / np.sqrt(128))
    o = out.cpu().numpy()[:, 0]
    err = np.linalg.norm(o - O) / np.linalg.norm(O)
    _log(f"  attention rel L2 {err:.2e}")
    assert err <= 2e-3
    # LSE: the GPU rounds fp32 Queries and the dequantized keys to fp16 (relative
    # 2^-11 each), so a logit moves by at most 2^-10 sum_c |q_c k_c| / sqrt(d)
    # plus fp32 accumulation; the LSE moves by at most the largest such change
    Kd, _ = OA.segment_kv(seg)
    bound = 2.0 ** -10 * (np.abs(Q[:, 0].astype(np.float64)) @ np.abs(Kd).T).max(axis=1) / np.sqrt(128) + 1e-4
    assert np.all(np.abs(lse.cpu().numpy()[0] - L) <= bound)


def test_reference_top1_and_shift_rate(qwm):
    """Top-1 over the unquantized bf16 keys (the shift-rate reference) on the
    rollout workload's final cache (62,400 keys, 24 heads), against the oracle
    on sampled Queries (equal, or a logit near-tie)."""
    import torch
    from gpu_helpers import dev_tokens
    _log("reference top-1, rollout shape")
    w = datagen.make_workload("rollout")
    K = w.K
    Qv = w.Q[w.chunk_slice(w.n_chunks - 1)]
    top = qwm.reference_top1(dev_tokens(Qv, "bf16"), dev_tokens(K, "bf16"))
    torch.cuda.synchronize()
    top = top.cpu().numpy()
    rng = np.random.default_rng(9)
    for h in (0, 11, 23):
        sample = rng.choice(Qv.shape[0], 64, replace=False)
        Kh = K[:, h].astype(np.float64)
        Qs = Qv[sample, h].astype(np.float64)
        logits = Qs @ Kh.T
        ref = np.argmax(logits, axis=1)
        g = top[h, sample]
        r = np.arange(len(sample))
        gap = logits[r, ref] - logits[r, g]
        # fp32 accumulation of 128 exact products: error well below 1e-5 of sum |q_c k_c|
        mag = np.abs(Qs) @ np.abs(Kh).T
        assert np.all(gap <= 1e-5 * mag[r, ref]), gap.max()
        assert np.mean(g == ref) >= 0.95
    # shift rate between a cache attention top-1 and the reference: identical inputs give 0
    assert OA.shift_rate(top[0], top[0]) == 0.0


def _oracle_lloyd_unit(args):
    X, iters, seed, head = args
    from oracle import lloyd as L
    return L.lloyd(X, 256, iters, seed=seed, head=head)


def test_depth_layer_lloyd_ten_iterations(qwm):
    """The depth workload's table build as the bench runs it: 10 seeded Lloyd
    iterations over a full 28,000-token layer, all 40 heads in one call (the
    layer drawn on the device); heads 0 and 39 against the oracle's Lloyd, bit
    for bit, the oracle's two heads in parallel processes."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import torch
    from gpu_helpers import host
    _log("depth layer: 10 seeded Lloyd iterations, 28,000 tokens x 40 heads")
    K, _, _ = datagen.device_layer("depth", 0)
    C = qwm.build_centroids(K, 10, seed=1)
    torch.cuda.synchronize()
    heads = [0, 39]
    units = [(K[:, h].double().cpu().numpy(), 10, 1, h) for h in heads]
    with cf.ProcessPoolExecutor(max_workers=2, mp_context=mp.get_context("spawn")) as ex:
        tables = list(ex.map(_oracle_lloyd_unit, units))
    Cg = host(C)
    for h, Co in zip(heads, tables):
        np.testing.assert_array_equal(Cg[h], Co)
        _log(f"  head {h}: table bit-exact")


def test_attention_over_quantized_depth_layer(qwm):
    """Attention over a quantized depth layer as the bench builds it: all 40
    heads of a full 28,000-token layer quantized on the GPU (QSAC + PSAC keys,
    M = 8, and values) with the oracle's Forgy tables and statistics, then
    attended by the layer's 1,560 Queries.  For heads 0 and 39 the oracle
    quantizes the same tokens with the same tables and attends to its own
    cache; sampled Queries agree to the attention tolerance.  Centroid choices
    may differ only at counted near-ties, and so may a top-1 key."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, dev_basis, packed_host
    _log("attention over a quantized depth layer: 28,000 keys x 40 heads, 1,560 Queries")
    w = datagen.make_workload("depth", n_chunks=1)
    H, T = w.H, w.chunk
    K, V, Q = w.K[:T], w.V[:T], w.Q
    heads = [0, H - 1]
    ob = {}
    for h in heads:
        S, n = OS.update(np.zeros((128, 128)), 0, Q[:, h])
        b = OS.principal_basis(S, n)
        ob[h] = (OS.channel_weights(S, n), b["U_bf16"])
    wt = np.stack([ob[heads[0]][0]] * H)
    Ub = np.stack([ob[heads[0]][1]] * H)
    wt[heads[1]], Ub[heads[1]] = ob[heads[1]][0], ob[heads[1]][1]
    CK, CV = _forgy_tables(K, 41), _forgy_tables(V, 42)
    dCK, dCV, dU = dev_table(CK), dev_table(CV), dev_basis(Ub)
    kp = qwm.quantize_keys(dev_tokens(K, "bf16"), dCK, torch.from_numpy(wt.astype(np.float32)).cuda(), dU,
                           M=8, flags=3)
    vp = qwm.quantize_values(dev_tokens(V, "bf16"), dCV)
    seg = qwm.segment_array([(kp, vp, dCK, dCV, dU)])
    out, lse, top1 = qwm.attention(dev_tokens(Q, "bf16"), seg, want_lse=True, want_top1=True)
    torch.cuda.synchronize()
    out, lse, top1 = out.cpu().numpy(), lse.cpu().numpy(), top1.cpu().numpy()
    gk, gv = packed_host(kp), packed_host(vp)
    tq = Q.shape[0]
    sample = np.unique(np.array([0, 1, 31, 32, 255, 256, tq // 2, tq - 2, tq - 1]))
    for h in heads:
        ok = Qz.quantize_keys(K[:, h].astype(np.float64), CK[h], wt[h], Ub[h], M=8, flags=3)
        ov = Qz.quantize_values(V[:, h].astype(np.float64), CV[h])
        nk = _check_keys("qsac", ok, gk, h, K[:, h], CK[h], wt[h], 8, 3)
        nv = _check_keys("nearest", ov, gv, h, V[:, h], CV[h], None, 1, 0)
        differ = (ok["idx"] != gk["idx"][h]) | (ov["idx"] != gv["idx"][h])
        oseg = [dict(k_idx=ok["idx"], k_q=ok["q"], k_scale=ok["scale"], k_zero=ok["zero"], k_Cq=ok["Cq"],
                     k_cs=ok["c_scale"], k_centroids=CK[h], U=Ub[h], v_idx=ov["idx"], v_q=ov["q"],
                     v_scale=ov["scale"], v_zero=ov["zero"], v_centroids=CV[h])]
        Qh = F.bf16_rne(Q[sample, h].astype(np.float64))
        O, L, top = OA.cache_attention(Qh, oseg, 1 / np.sqrt(128))
        err = np.linalg.norm(out[sample, h] - O) / np.linalg.norm(O)
        _log(f"  head {h}: {nk} + {nv} near-tie centroid choices, rel L2 {err:.2e}")
        assert err <= 2e-3
        np.testing.assert_allclose(lse[h, sample], L, rtol=1e-4, atol=1e-4)
        gt = top1[h, sample]
        keep = ~(differ[gt] | differ[top])      # a top-1 key whose own coding differs is a counted near-tie
        from gpu_helpers import check_top1_near_tie
        nt = check_top1_near_tie(gt[keep], top[keep], Qh[keep], oseg)
        _log(f"  head {h}: top-1 ok ({nt} near-tie logits, {int((~keep).sum())} on near-tie keys)")
