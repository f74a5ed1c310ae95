"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
reading packed chunks back, running the oracle on the same inputs, and the
parity rules (bit-exact indices and codes except counted near-ties)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import formats as F
from oracle import quantize as Qz


def dev_tokens(x: np.ndarray, dtype: str) -> torch.Tensor:
    """[T, H, d] float32 array (bf16-valued for 'bf16') -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def dev_table(C: np.ndarray) -> torch.Tensor:
    """[H, 256, 128] bf16-valued -> device bf16."""
    return torch.from_numpy(np.ascontiguousarray(C, dtype=np.float32)).to(torch.bfloat16).cuda()


def dev_basis(U: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(U, dtype=np.float32)).to(torch.bfloat16).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def packed_host(p) -> dict:
    """Per-head numpy views of a PackedChunk."""
    d = {
        "codes": p.codes.cpu().numpy(), "idx": p.idx.cpu().numpy(),
        "scale_bits": p.scale.cpu().numpy().view(np.uint16), "zeros": p.zeros.cpu().numpy(),
    }
    if p.keys:
        d["c"] = p.c.cpu().numpy()
        d["c_scale_bits"] = p.c_scale.cpu().numpy().view(np.uint16)
    return d


def upload_packed(PackedChunk, H: int, T: int, keys: bool, heads_out: list) -> object:
    """Device PackedChunk holding the oracle's packed arrays (one dict per head);
    the PSAC rank is the width of the oracle's coefficients."""
    r = heads_out[0]["Cq"].shape[1] if keys else 8
    pc = PackedChunk(T, H, keys, r=r)
    zs = pc.zeros.shape[1]
    codes = np.stack([o["codes"] for o in heads_out])
    idx = np.stack([o["idx"] for o in heads_out])
    scale = np.stack([o["scale_bits"] for o in heads_out]).view(np.int16)
    zeros = np.zeros((H, zs), np.uint8)
    for h, o in enumerate(heads_out):
        zeros[h, :len(o["zeros"])] = o["zeros"]
    pc.codes.copy_(torch.from_numpy(codes))
    pc.idx.copy_(torch.from_numpy(idx))
    pc.scale.copy_(torch.from_numpy(np.ascontiguousarray(scale)))
    pc.zeros.copy_(torch.from_numpy(zeros))
    if keys:
        pc.c.copy_(torch.from_numpy(np.stack([o["Cq"] for o in heads_out])))
        pc.c_scale.copy_(torch.from_numpy(np.stack([o["c_scale_bits"] for o in heads_out]).view(np.int16)))
    return pc


def idx_mismatches_allowed(kind: str, orc: dict, gpu_idx: np.ndarray, K: np.ndarray, C: np.ndarray,
                           w=None, M: int = 8, rel: float = 1e-6):
    """Tokens whose GPU centroid differs from the oracle's.  Returns (n_mismatch,
    n_not_allowed).  A mismatch is allowed only when the oracle's relative gap
    between the two choices is below `rel` (on S for QSAC, on the distance
    otherwise, or at the top-M boundary)."""
    o = orc["idx"].astype(np.int64)
    g = gpu_idx.astype(np.int64)
    bad = np.nonzero(o != g)[0]
    not_ok = 0
    for t in bad:
        if kind == "qsac":
            ww = np.ones(K.shape[1], np.float32) if w is None else w
            dq = orc["info"]["dq"][t]
            order = np.argsort(dq, kind="stable")
            Wg = np.asarray(ww, np.float64).reshape(-1, 64).sum(axis=1)
            def S_of(j):
                r = np.float32(1) * K[t].astype(np.float32) - C[j].astype(np.float32)
                _, _, R = Qz.group_ranges(r[None])
                return float(Qz.qsac_score(R, Wg)[0])
            so, sg = S_of(o[t]), S_of(g[t])
            ok = abs(sg - so) <= rel * max(so, 1e-300)
            if not ok and g[t] not in order[:M]:
                # GPU picked outside the oracle's top-M: allowed only if the boundary is a near-tie
                dm = dq[order[M - 1]]
                ok = abs(dq[g[t]] - dm) <= rel * max(dm, 1e-300)
        else:
            d = orc["info"]["dq"][t]
            ok = abs(d[g[t]] - d[o[t]]) <= rel * max(d[o[t]], 1e-300)
        not_ok += int(not ok)
    return len(bad), not_ok


def compare_codec(orc: dict, gpu: dict, T: int, mask: np.ndarray):
    """Codes, scales and zero-points must be bit-exact on tokens with equal idx."""
    gq = F.unpack_codes(gpu["codes"], 128)
    np.testing.assert_array_equal(gq[mask], orc["q"][mask])
    np.testing.assert_array_equal(gpu["scale_bits"][mask], orc["scale_bits"][mask])
    gz = F.unpack_zeros(gpu["zeros"][: (T + 1) // 2], T)
    np.testing.assert_array_equal(gz[mask], orc["zero"][mask])


def check_top1_near_tie(gt, ot, Qh, oracle_segs):
    """Top-1 must agree except where the oracle's top-2 logit gap is below
    1e-3 relative: every mismatch must be such a near-tie.  gt, ot: GPU and
    oracle top-1 of the Queries Qh [n, d]; oracle_segs: the oracle's segment
    dicts of the head.  Returns the number of (allowed) mismatches."""
    from oracle import attention as OA
    Kall = np.concatenate([OA.segment_kv(s)[0] for s in oracle_segs])
    L = np.asarray(Qh, np.float64) @ Kall.T
    bad = np.nonzero(np.asarray(gt) != np.asarray(ot))[0]
    for i in bad:
        a, b = L[i, ot[i]], L[i, gt[i]]
        assert abs(a - b) <= 1e-3 * abs(a), (int(i), a, b)
    return len(bad)
