"""Benchmark of the QuantWM 2-bit KV-cache hot path on one MI355X.

One step = one streaming chunk of the 480p-shaped single-layer workload
(H = 12 heads, d = 128; 24 cached latent frames of 30x52 = 1,560 tokens plus
the new frame): update the Query statistics with the previous chunk's Queries
and re-derive the principal basis, refresh the K and V centroid tables with 3
warm-started Lloyd iterations, quantize the new Keys (QSAC + PSAC) and Values,
then attend with the new chunk's 1,560 Queries over all 39,000 cached keys in
25 compressed segments.  Inputs are seeded synthetic caches resident in HBM.

Prints one JSON line.  `value` = new-chunk tokens per second through the whole
step; the attention kernel's roofline and the CPU oracle baseline ride along.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2516.6
H, CHUNK, NCHUNK, D = 12, 1560, 25, 128
ATTN_FLOP_PER_QKH = 2 * (128 + 8) + 2 * 128           # 528: logits (with PSAC) + PV
KEY_BYTES_PER_TOKEN_HEAD = 256 + 47.5                  # read bf16 key, write packed key
KEY_TABLE_BYTES_PER_HEAD = 256 * 128 * 2 + 128 * 4 + 128 * 8 * 2   # centroids + w + U
PACKED_BYTES_PER_KEY_HEAD = 85.0                       # K 47.5 + V 37.5 bytes read by attention
SEG_TABLE_BYTES_PER_HEAD = 2 * 256 * 128 * 2 + 128 * 8 * 2


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-queries", type=int, default=48)
    return ap.parse_args()


class Step:
    """Device state of the workload and the streaming step."""

    def __init__(self, qwm, torch, w):
        self.qwm, self.torch = qwm, torch
        dev = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()
        self.K, self.V, self.Q = dev(w.K), dev(w.V), dev(w.Q)
        self.st = qwm.QueryStats(H)
        self.segs = []
        self.tables = []
        prev = None
        for c in range(NCHUNK - 1):                     # prefill the cache causally
            sl = w.chunk_slice(c)
            seg, prev = self._chunk(c, sl, prev, keep=True)
            self.segs.append(seg)
            self.tables.append(prev)
        self.prev = prev
        sl = w.chunk_slice(NCHUNK - 1)
        self.sl_new = sl
        self.sl_prevq = w.chunk_slice(NCHUNK - 2)
        # buffers of the new chunk
        self.Ck = torch.empty(H, 256, D, dtype=torch.bfloat16, device="cuda")
        self.Cv = torch.empty_like(self.Ck)
        self.kp = qwm.PackedChunk(CHUNK, H, True)
        self.vp = qwm.PackedChunk(CHUNK, H, False)
        self.segs.append((self.kp, self.vp, self.Ck, self.Cv, self.st.U))
        self.dsegs, self.total = qwm.segments_tensor(self.segs)
        self.diag = qwm.new_diag()
        # the Query statistics and basis only feed the key quantization: they run on
        # a side stream, overlapped with the Lloyd refresh
        self.side = torch.cuda.Stream()
        self.stats_done = torch.cuda.Event()

    def _chunk(self, c, sl, prev, keep):
        qwm = self.qwm
        K, V = self.K[sl], self.V[sl]
        if prev is None:
            Ck = qwm.build_centroids(K, 10, seed=1)
            Cv = qwm.build_centroids(V, 10, seed=2)
            kp = qwm.quantize_keys(K, Ck, None, None, M=8, flags=3)
            U = None
        else:
            Ck = qwm.build_centroids(K, 3, init=prev[0])
            Cv = qwm.build_centroids(V, 3, init=prev[1])
            U = self.st.U.clone()
            kp = qwm.quantize_keys(K, Ck, self.st.w, U, M=8, flags=3)
        vp = qwm.quantize_values(V, Cv)
        if c < NCHUNK - 2:        # the step itself adds the previous chunk's Queries
            qwm.update_query_stats(self.Q[sl], self.st, compute_basis=True)
        return (kp, vp, Ck, Cv, U), (Ck, Cv)

    def run(self, events=None):
        qwm = self.qwm
        rec = (lambda i: events[i].record()) if events is not None else (lambda i: None)
        K, V = self.K[self.sl_new], self.V[self.sl_new]
        torch = self.torch
        main = torch.cuda.current_stream()
        rec(0)
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            qwm.update_query_stats(self.Q[self.sl_prevq], self.st, compute_basis=True)
            self.stats_done.record(self.side)
        rec(1)
        qwm.build_centroids(K, 3, init=self.prev[0], out=self.Ck, diag=self.diag)
        qwm.build_centroids(V, 3, init=self.prev[1], out=self.Cv, diag=self.diag)
        rec(2)
        main.wait_event(self.stats_done)
        qwm.quantize_keys(K, self.Ck, self.st.w, self.st.U, M=8, flags=3, out=self.kp, diag=self.diag)
        rec(3)
        qwm.quantize_values(V, self.Cv, out=self.vp, diag=self.diag)
        rec(4)
        out, _, _ = qwm.attention(self.Q[self.sl_new], self.dsegs, NCHUNK, self.total)
        rec(5)
        return out


def cpu_baseline(w, nq):
    """The oracle (untuned) on one head of the step; extrapolated to the whole
    step (12 heads, 1,560 queries).  Attention is timed on `nq` sampled queries
    over all 25 segments, whose packed contents are seeded random arrays."""
    import numpy as np
    from oracle import attention as OA, formats as F, lloyd as OL, quantize as Qz, stats as OS
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    h = 0
    sl = w.chunk_slice(NCHUNK - 1)
    slp = w.chunk_slice(NCHUNK - 2)
    K = w.K[sl, h].astype(np.float64)
    Vv = w.V[sl, h].astype(np.float64)
    S0, n0 = OS.update(np.zeros((D, D)), 0, w.Q[:slp.start, h])
    prevk = OL.lloyd(w.K[slp, h].astype(np.float64), 256, 1, seed=1, head=h)
    prevv = OL.lloyd(w.V[slp, h].astype(np.float64), 256, 1, seed=2, head=h)
    t0 = time.perf_counter()
    S, n = OS.update(S0, n0, w.Q[slp, h])
    basis = OS.principal_basis(S, n)
    wts = OS.channel_weights(S, n)
    Ck = OL.lloyd(K, 256, 3, init=prevk)
    Cv = OL.lloyd(Vv, 256, 3, init=prevv)
    kq = Qz.quantize_keys(K, Ck, wts, basis["U_bf16"], M=8)
    vq = Qz.quantize_values(Vv, Cv)
    t_quant = time.perf_counter() - t0
    rng = np.random.default_rng(5)
    segs = []
    for s in range(NCHUNK):
        q = rng.integers(0, 4, (CHUNK, 128)).astype(np.uint8)
        z = rng.integers(0, 4, (CHUNK, 2)).astype(np.uint8)
        sc = rng.uniform(0.01, 0.2, (CHUNK, 2)).astype(np.float16).astype(np.float64)
        segs.append(dict(k_idx=rng.integers(0, 256, CHUNK), k_q=q, k_scale=sc, k_zero=z,
                         k_Cq=rng.integers(-127, 128, (CHUNK, 8)), k_cs=np.full(CHUNK, 1e-3),
                         k_centroids=Ck, U=basis["U_bf16"], v_idx=rng.integers(0, 256, CHUNK), v_q=q,
                         v_scale=sc, v_zero=z, v_centroids=Cv))
    Qs = w.Q[sl, h][:nq].astype(np.float64)
    t1 = time.perf_counter()
    OA.cache_attention(Qs, segs, 1 / np.sqrt(D))
    t_attn = time.perf_counter() - t1
    step_s = H * (t_quant + t_attn * CHUNK / nq)
    return {"value": CHUNK / step_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"head 0 of the step: stats+Jacobi basis, 3+3 Lloyd iterations, QSAC+PSAC keys and "
                      f"values of the 1,560-token chunk ({t_quant:.2f} s), attention of {nq} queries over "
                      f"39,000 keys ({t_attn:.2f} s); extrapolated x12 heads and x{CHUNK // nq} queries",
            "seconds_sampled": round(t_quant + t_attn, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU path is not "
              f"part of this build", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import bit_kv_cache_head_amd as qwm
    import datagen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log("generating the 480p workload")
    w = datagen.make_workload("480p")
    log("prefilling 24 chunks")
    step = Step(qwm, torch, w)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    step.diag.zero_()
    step.run()
    torch.cuda.synchronize()
    diag_step = step.diag.tolist()
    log("timing")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step.run(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_end) / args.steps
    names = ["launch_stats", "lloyd_kv", "keys_incl_stats_wait", "values", "attention"]
    stage = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
    attn_ms = stage["attention"]
    flops = ATTN_FLOP_PER_QKH * CHUNK * step.total * H
    achieved = flops / (attn_ms * 1e-3) / 1e12
    attn_bytes = PACKED_BYTES_PER_KEY_HEAD * step.total * H + SEG_TABLE_BYTES_PER_HEAD * H * NCHUNK \
        + CHUNK * H * (256 + 512)
    key_bytes = KEY_BYTES_PER_TOKEN_HEAD * CHUNK * H + KEY_TABLE_BYTES_PER_HEAD * H

    # bulk key throughput: the 24 cached chunks' keys in one call (QSAC + PSAC)
    Kall = step.K[: (NCHUNK - 1) * CHUNK]
    kb = qwm.PackedChunk(Kall.shape[0], H, True)
    for _ in range(2):
        qwm.quantize_keys(Kall, step.prev[0], step.st.w, step.st.U, M=8, flags=3, out=kb)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    nb = 5
    for _ in range(nb):
        qwm.quantize_keys(Kall, step.prev[0], step.st.w, step.st.U, M=8, flags=3, out=kb)
    e1.record()
    torch.cuda.synchronize()
    bulk_ms = e0.elapsed_time(e1) / nb
    bulk_bytes = KEY_BYTES_PER_TOKEN_HEAD * Kall.shape[0] * H + KEY_TABLE_BYTES_PER_HEAD * H

    res = {
        "metric": "Key tokens/s quantized (QSAC+PSAC) + compressed-cache attention MFMA %/HBM GB/s",
        "value": round(CHUNK / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "480p-shaped single layer, streaming step: H=12, d=128, 24 cached chunks "
                               "+ 1 new chunk of 1,560 tokens (39,000 keys in 25 segments), 1,560 queries; "
                               "M=8, r=8, 256 centroids, 3 warm Lloyd iterations",
                   "heads": H, "chunk_tokens": CHUNK, "cached_keys": int(step.total), "queries": CHUNK},
        "roofline": {"kernel": "attention (fused dequant + PSAC + online softmax; includes the split merge)",
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "flop_per_launch": flops, "avg_launch_ms": round(attn_ms, 4),
                     "compressed_GBps": round(attn_bytes / (attn_ms * 1e-3) / 1e9, 1)},
        "stages_ms": {k: round(v, 4) for k, v in stage.items()},
        "keys_step": {"token_heads": CHUNK * H, "ms_incl_stats_wait": round(stage["keys_incl_stats_wait"], 4)},
        "keys_bulk": {"tokens": int(Kall.shape[0]), "token_heads": int(Kall.shape[0]) * H,
                      "ms": round(bulk_ms, 4),
                      "tokens_per_s": round(Kall.shape[0] / (bulk_ms * 1e-3), 1),
                      "GBps": round(bulk_bytes / (bulk_ms * 1e-3) / 1e9, 1),
                      "hbm_frac": round(bulk_bytes / (bulk_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "wall_s_timed": round(wall, 3),
        "exact_fallbacks_per_step": int(diag_step[1]), "nonfinite_rows_per_step": int(diag_step[0]),
        "eig_iterations": step.st.iters.tolist(),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle sample")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_queries)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
