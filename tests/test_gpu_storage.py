"""The stored-format refinements on the GPU against the oracle: two-level
group scales (rainbus digest, method step (3)), the keep test with the full
Query second moment (method step (4)), and the per-head dense / sparse
coefficient layout (QuantWM v2 App. D.1); attention and the decoder over
chunks stored in these forms."""
import sys

import numpy as np
import pytest

import datagen
from oracle import attention as OA
from oracle import formats as F
from oracle import lloyd as OL
from oracle import quantize as Qz
from oracle import stats as OS
from oracle import storage as St

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


def _inputs(T=777, heads=(0, 1), r=8):
    w = datagen.make_workload("480p", heads=list(heads), n_chunks=2, chunk=T)
    K, V = w.K[T:2 * T], w.V[T:2 * T]
    Ck, Cv, ws, Us, Ss = [], [], [], [], []
    for h in range(len(heads)):
        Ck.append(OL.lloyd(w.K[:T, h].astype(np.float64), 256, 3, seed=5, head=h))
        Cv.append(OL.lloyd(w.V[:T, h].astype(np.float64), 256, 3, seed=6, head=h))
        S, n = OS.update(np.zeros((128, 128)), 0, w.Q[:T, h])
        ws.append(OS.channel_weights(S, n))
        Us.append(OS.principal_basis(S, n, r=r)["U_bf16"])
        Ss.append((S, n))
    return w, K, V, np.stack(Ck), np.stack(Cv), np.stack(ws), np.stack(Us), Ss


@pytest.mark.parametrize("flags,r", [(3, 8), (7, 8), (3, 16)])
def test_two_level_scales(qwm, flags, r):
    """Keys and values converted to two-level scales: second-level scales, step
    codes, codes and zero-points bit-exact against the oracle's conversion of
    its own chunk; C within one LSB."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, dev_basis, packed_host
    _log(f"two-level scales flags={flags} r={r}")
    T = 777
    w, K, V, Ck, Cv, wt, Ut, _ = _inputs(T, r=r)
    dK, dV = dev_tokens(K, "bf16"), dev_tokens(V, "bf16")
    tk, tv, wd, Ud = dev_table(Ck), dev_table(Cv), torch.from_numpy(wt).cuda(), dev_basis(Ut)
    kp = qwm.quantize_keys(dK, tk, wd, Ud, M=8, flags=flags)
    vp = qwm.quantize_values(dV, tv)
    qwm.two_level_scales(dK, tk, kp, wd, Ud, flags=flags)
    qwm.two_level_scales(dV, tv, vp)
    torch.cuda.synchronize()
    gk, gv = packed_host(kp), packed_host(vp)
    for h in range(2):
        ok = Qz.quantize_keys(K[:, h].astype(np.float64), Ck[h], wt[h], Ut[h], M=8, flags=flags)
        ov = Qz.quantize_values(V[:, h].astype(np.float64), Cv[h])
        assert np.array_equal(ok["idx"], gk["idx"][h]) and np.array_equal(ov["idx"], gv["idx"][h])
        tk2 = St.requantize_two_level(K[:, h].astype(np.float64), Ck[h], ok, U_bf16=Ut[h], w=wt[h], flags=flags)
        tv2 = St.requantize_two_level(V[:, h].astype(np.float64), Cv[h], ov)
        for o, g, p in ((tk2, gk, kp), (tv2, gv, vp)):
            np.testing.assert_array_equal(p.scale2[h].cpu().numpy().view(np.uint16), o["scale2_bits"])
            np.testing.assert_array_equal(p.scale_q[h].cpu().numpy(), o["scale_q"])
            np.testing.assert_array_equal(F.unpack_codes(g["codes"][h], 128), o["q"])
            np.testing.assert_array_equal(F.unpack_zeros(g["zeros"][h][: (T + 1) // 2], T), o["zero"])
        dc = np.abs(gk["c"][h].astype(np.int64) - tk2["Cq"].astype(np.int64))
        same = np.ones(T, bool)
        if flags & 4:   # the keep decisions agree except at rounding level (both in fp64)
            g_keep = gk["c_scale_bits"][h] != 0
            o_keep = tk2["c_scale_bits"] != 0
            same = g_keep == o_keep
            assert same.mean() > 0.999
        assert dc[same].max() <= 1
        _log(f"  head {h}: s2 K {tk2['scale2'].tolist()} V {tv2['scale2'].tolist()}, C off by one: "
             f"{int((dc[same] == 1).sum())}")


def test_keep_full_pass(qwm):
    """The keep test with e^T (S / n) e on keys quantized without the diagonal
    test: the same keys keep their coefficients as in the oracle, except where
    the two errors agree to rounding level; kept coefficients unchanged."""
    import torch
    from gpu_helpers import dev_tokens, dev_table, dev_basis, packed_host
    T = 777
    w, K, V, Ck, Cv, wt, Ut, Ss = _inputs(T)
    st = qwm.QueryStats(2)
    st.S.copy_(torch.from_numpy(np.stack([S for S, _ in Ss])))
    st.n.copy_(torch.tensor([n for _, n in Ss]))
    kp = qwm.quantize_keys(dev_tokens(K, "bf16"), dev_table(Ck), torch.from_numpy(wt).cuda(), dev_basis(Ut), M=8,
                           flags=3)
    before = packed_host(kp)
    qwm.psac_keep_full(dev_tokens(K, "bf16"), dev_table(Ck), st, dev_basis(Ut), kp)
    torch.cuda.synchronize()
    g = packed_host(kp)
    for h in range(2):
        o = Qz.quantize_keys(K[:, h].astype(np.float64), Ck[h], wt[h], Ut[h], M=8, flags=3)
        mu = Ck[h][o["idx"].astype(np.int64)]
        E = K[:, h].astype(np.float64) - (mu + o["r_hat"])
        S, n = Ss[h]
        keep, after, bef = St.psac_keep_full(E, o["Cq"], o["c_scale"], Ut[h], S / n)
        gk = g["c_scale_bits"][h] != 0
        dis = gk != keep
        assert np.all(np.abs(after[dis] - bef[dis]) <= 1e-9 * bef[dis]), np.nonzero(dis)[0][:5]
        np.testing.assert_array_equal(g["c"][h][gk], before["c"][h][gk])
        np.testing.assert_array_equal(g["c"][h][~gk], 0)
        _log(f"  head {h}: kept {gk.mean():.4f} (oracle {keep.mean():.4f}), rounding-level disagreements {int(dis.sum())}")


def _oracle_coeffs(T, r, kept_frac, seed):
    rng = np.random.default_rng(seed)
    Cq = rng.integers(-127, 128, (T, r)).astype(np.int8)
    cs = F.fp16_bits(rng.uniform(1e-3, 1.0, T))
    drop = rng.random(T) > kept_frac
    Cq[drop] = 0
    cs[drop] = 0
    return Cq, cs


@pytest.mark.parametrize("r", [8, 16, 32])
def test_compact_layouts(qwm, r):
    """The per-head layout choice and bytes against the oracle's packing, on
    oracle coefficients uploaded to the device: heads with 30 %, 97 %, 100 % and
    0 % of the keys kept (T = 1,000: sparse, sparse, dense, sparse)."""
    import torch
    from bit_kv_cache_head_amd import QWM_LAYOUT_DENSE
    T, fracs = 1000, [0.3, 0.97, 1.0, 0.0]
    H = len(fracs)
    heads = [_oracle_coeffs(T, r, f, 10 + i) for i, f in enumerate(fracs)]
    kp = qwm.PackedChunk(T, H, True, r=r)
    kp.c.copy_(torch.from_numpy(np.stack([c for c, _ in heads])))
    kp.c_scale.copy_(torch.from_numpy(np.stack([s for _, s in heads]).view(np.int16)))
    used = torch.zeros(1, dtype=torch.int64, device="cuda")
    qwm.compact_coefficients(kp, used=used)
    torch.cuda.synchronize()
    arena = kp.carena.cpu().numpy()
    for h, (lay, count, off) in enumerate(kp.layouts()):
        p = St.pack_coefficients(*heads[h])
        assert lay == (1 if p["layout"] == "sparse" else QWM_LAYOUT_DENSE) and count == p["count"], (h, lay, count)
        reg = arena[off: off + p["bytes"]]
        al = lambda n: (n + 15) // 16 * 16
        if p["layout"] == "dense":
            np.testing.assert_array_equal(reg[: T * r].view(np.int8).reshape(T, r), p["c"])
            np.testing.assert_array_equal(reg[al(T * r): al(T * r) + 2 * T].view(np.uint16), p["cs"])
        else:
            nw = (T + 63) // 64
            np.testing.assert_array_equal(reg[: 8 * nw].view(np.uint64), p["bitmap"])
            o = al(8 * nw)
            np.testing.assert_array_equal(reg[o: o + 4 * nw].view(np.uint32), p["prefix"])
            o += al(4 * nw)
            np.testing.assert_array_equal(reg[o: o + count * r].view(np.int8).reshape(count, r), p["c"])
            o += al(count * r)
            np.testing.assert_array_equal(reg[o: o + 2 * count].view(np.uint16), p["cs"])
        _log(f"  head {h}: {p['layout']}, {count} kept, {p['bytes']} bytes")
    assert int(used.item()) == sum(St.pack_coefficients(*x)["bytes"] for x in heads)


def _two_level_segment(qwm, w, sl, H, r, two, keep_frac_drop, rng):
    """One chunk quantized by the oracle (own tables and basis), optionally
    with two-level scales and with some coefficients dropped; device arrays
    uploaded, and the oracle's segment dicts."""
    import torch
    from gpu_helpers import upload_packed, dev_table, dev_basis
    per, kd, vd = [], [], []
    for h in range(H):
        Kc, Vc = w.K[sl, h].astype(np.float64), w.V[sl, h].astype(np.float64)
        Ck = OL.lloyd(w.K[-600:, h].astype(np.float64), 256, 2, seed=41, head=h)
        Cv = OL.lloyd(w.V[-600:, h].astype(np.float64), 256, 2, seed=42, head=h)
        S, n = OS.update(np.zeros((128, 128)), 0, w.Q[:300, h])
        U = OS.principal_basis(S, n, r=r)["U_bf16"]
        kq = Qz.quantize_keys(Kc, Ck, OS.channel_weights(S, n), U, M=8)
        vq = Qz.quantize_values(Vc, Cv)
        if two:
            kq = St.requantize_two_level(Kc, Ck, kq, U_bf16=U, w=OS.channel_weights(S, n), flags=3)
            vq = St.requantize_two_level(Vc, Cv, vq)
            ks, vs = kq["steps"], vq["steps"]
        else:
            ks, vs = kq["scale"], vq["scale"]
        Cq, cs = kq["Cq"].copy(), kq["c_scale"].copy()
        drop = rng.random(len(cs)) < keep_frac_drop
        Cq[drop] = 0
        cs[drop] = 0
        kd.append(dict(codes=kq["codes"], idx=kq["idx"], scale_bits=F.fp16_bits(ks), zeros=kq["zeros"], Cq=Cq,
                       c_scale_bits=F.fp16_bits(cs), sq=kq.get("scale_q"), s2=kq.get("scale2_bits")))
        vd.append(dict(codes=vq["codes"], idx=vq["idx"], scale_bits=F.fp16_bits(vs), zeros=vq["zeros"],
                       sq=vq.get("scale_q"), s2=vq.get("scale2_bits")))
        per.append(dict(Ck=Ck, Cv=Cv, U=U, oracle=dict(k_idx=kq["idx"], k_q=kq["q"], k_scale=ks, k_zero=kq["zero"],
                                                       k_Cq=Cq, k_cs=cs, k_centroids=Ck, U=U, v_idx=vq["idx"],
                                                       v_q=vq["q"], v_scale=vs, v_zero=vq["zero"], v_centroids=Cv)))
    T = sl.stop - sl.start
    kp = upload_packed(qwm.PackedChunk, H, T, True, kd)
    vp = upload_packed(qwm.PackedChunk, H, T, False, vd)
    if two:
        for p, d in ((kp, kd), (vp, vd)):
            p.scale_q = torch.from_numpy(np.stack([x["sq"] for x in d])).cuda()
            p.scale2 = torch.from_numpy(np.stack([x["s2"] for x in d]).view(np.int16)).cuda()
    kc = dev_table(np.stack([p["Ck"] for p in per]))
    vc = dev_table(np.stack([p["Cv"] for p in per]))
    U = dev_basis(np.stack([p["U"] for p in per]))
    return (kp, vp, kc, vc, U), [p["oracle"] for p in per]


def test_attention_and_decode_over_stored_forms(qwm):
    """Attention over four chunks: plain; two-level; compacted coefficients
    with a third dropped (sparse heads); two-level and compacted, rank 16.
    Against the oracle's attention over the same chunks; the decoder bit-exact."""
    import torch
    from gpu_helpers import dev_tokens, check_top1_near_tie
    H = 2
    rng = np.random.default_rng(3)
    w = datagen.make_workload("480p", heads=[0, 1], n_chunks=1, chunk=1400)
    plan = [(slice(0, 300), 8, False, 0.0, False), (slice(300, 557), 8, True, 0.0, False),
            (slice(557, 900), 8, False, 0.33, True), (slice(900, 1000), 16, True, 0.5, True)]
    keep, oseg = [], [[] for _ in range(H)]
    for sl, r, two, drop, compact in plan:
        seg, od = _two_level_segment(qwm, w, sl, H, r, two, drop, rng)
        if compact:
            qwm.compact_coefficients(seg[0])
        keep.append(seg)
        for h in range(H):
            oseg[h].append(od[h])
    torch.cuda.synchronize()
    layouts = [kp.layouts() for (kp, _, _, _, _) in keep if kp.cdir is not None]
    _log(f"  compacted layouts: {layouts}")
    assert any(l[0] == 1 for ls in layouts for l in ls)
    Qv = w.Q[-200:]
    out, lse, top1 = qwm.attention(dev_tokens(Qv, "bf16"), qwm.segment_array(keep), want_lse=True, want_top1=True)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for h in range(H):
        O, L, top = OA.cache_attention(Qv[:, h].astype(np.float64), oseg[h], 1 / np.sqrt(128))
        err = np.linalg.norm(out[:, h] - O) / np.linalg.norm(O)
        _log(f"  head {h}: rel L2 {err:.2e}")
        assert err <= 2e-3
        np.testing.assert_allclose(lse.cpu().numpy()[h], L, rtol=1e-4, atol=1e-4)
        check_top1_near_tie(top1.cpu().numpy()[h], top, Qv[:, h], oseg[h])
    for si, (kp, vp, kc, vc, U) in enumerate(keep):
        Kd, Vd = qwm.decode_segment(kp, vp, kc, vc, U)
        torch.cuda.synchronize()
        for h in range(H):
            Ko, Vo = OA.decode_segment(oseg[h][si])
            assert np.array_equal(Kd[:, h].float().cpu().numpy(), Ko), (si, h)
            assert np.array_equal(Vd[:, h].float().cpu().numpy(), Vo), (si, h)
