"""Benchmark of the QuantWM 2-bit KV-cache hot path on one MI355X.

Default workload (depth): the full-depth memory case.  40 layers x 40 heads x
d = 128, 28,000 cached tokens per layer (about 21.4 GiB of bf16 K + V), all
resident in HBM, drawn on the device from the seeded recipe.  One step is the
whole hot path over every layer: update the Query statistics from the layer's
1,560 Queries and derive the principal basis, build the K and V centroid tables
(10 seeded Lloyd iterations each), quantize the Keys (QSAC + PSAC, M = 8) and
the Values, then attend with the 1,560 Queries over the layer's 2-bit cache.

`value` is the metric's first half: Key tokens quantized per second by
qwm_quantize_keys (QSAC + PSAC), token positions across all heads, from HIP
events around every key call of the timed steps.  `roofline` is the
compressed-cache attention's MFMA fraction (the metric's second half), from
HIP events around every attention call.  Per-stage rooflines, resident bytes
and compression ratio, device counters, the rollout ablations (token-shift
rates) and the CPU oracle baseline with a parity sample ride along.

Other workloads (--workload), parity-test shapes reported for context:
  480p    streaming step of the 480p-shaped layer (H = 12, 25 x 1,560-token chunks)
  720p    the same with H = 40 and 3,600-token chunks
  tiny    one pass: 4,096 fp32 keys/values, 512 Queries, 10 seeded Lloyd iterations
  rollout causal rollout of 40 chunks (H = 24) for each ablation (nearest
          centroid, QSAC, PSAC, QSAC + PSAC); per-ablation throughput and the
          top-1 shift rate against attention over the bf16 keys

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2516.6
D = 128
ATTN_FLOP_PER_QKH = 2 * (128 + 8) + 2 * 128           # 528: logits (with PSAC) + PV
KEY_BYTES_PER_TOKEN_HEAD = 256 + 47.5                  # read bf16 key, write packed key
KEY_TABLE_BYTES_PER_HEAD = 256 * 128 * 2 + 128 * 4 + 128 * 8 * 2   # centroids + w + U
PACKED_BYTES_PER_KEY_HEAD = 85.0                       # K 47.5 + V 37.5 bytes read by attention
SEG_TABLE_BYTES_PER_HEAD = 2 * 256 * 128 * 2 + 128 * 8 * 2        # K, V centroids + U = 133,120
BITS_PER_TOKEN_HEAD = 680                              # K 380 + V 300 bits resident
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_480p_step_traffic.md")
DEPTH_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_depth_traffic.md")
VALUE_BYTES_PER_TOKEN_HEAD = 256 + 37.5                # read bf16 value, write packed value
LLOYD_FLOP_PER_TOKEN_HEAD = 2 * 256 * 128              # one assignment GEMM per iteration
ATTN_SOURCE = os.path.join(ROOT, "bit_kv_cache_head_amd", "csrc", "attention.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="depth", choices=["depth", "480p", "720p", "tiny", "rollout"])
    ap.add_argument("--layers", type=int, default=40, help="depth: layers of the cache (40 = full depth)")
    ap.add_argument("--no-rollout", action="store_true", help="depth: skip the rollout ablations extra")
    ap.add_argument("--no-extras", action="store_true",
                    help="depth: skip the rank sweep, stored-format and rollout extras")
    ap.add_argument("--f-energy", type=float, default=None, help="top-8 Query energy (720p: 0.60 or 0.71)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-ab", action="store_true",
                    help="skip the extras after the step (decode + dense attention comparison, M sweep, multi-stage "
                         "codec); profiled runs use it, so the attention kernel's dispatches are the fused calls alone")
    ap.add_argument("--cpu-sample-queries", type=int, default=480)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run device copies of a known size (reference for HBM byte counters)")
    return ap.parse_args()


COPY_BYTES = 256 * 2 ** 20


def copy_calibration(torch):
    """Three device-to-device copies of 256 MiB: a kernel whose HBM traffic is
    known (reads and writes COPY_BYTES each), profiled beside the hot path to
    scale the FETCH_SIZE / WRITE_SIZE counters."""
    x = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    del x, y


def attention_traffic(path=TRAFFIC_FILE):
    """HBM bytes per attention launch from the committed counter summary, when
    it was taken on the attention source as it is now; else None."""
    try:
        text = open(path).read()
    except OSError:
        return None
    sha = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()[:16]
    fields = {}
    for line in text.splitlines():
        for key in ("source_sha", "hbm_bytes_per_launch"):
            if line.startswith(key + ":"):
                fields[key] = line.split(":", 1)[1].strip()
    if fields.get("source_sha") != sha or "hbm_bytes_per_launch" not in fields:
        return None
    return float(fields["hbm_bytes_per_launch"])


class Stream:
    """Streaming step: a causally prefilled cache of n-1 chunks plus the step
    that adds chunk n-1 (480p and 720p workloads)."""

    def __init__(self, qwm, torch, w):
        self.qwm, self.torch = qwm, torch
        self.H, self.chunk, self.nch = w.H, w.chunk, w.n_chunks
        dev = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()
        self.K, self.V, self.Q = dev(w.K), dev(w.V), dev(w.Q)
        self.st = qwm.QueryStats(self.H)
        self.segs = []
        prev = None
        for c in range(self.nch - 1):                    # prefill the cache causally
            seg, prev = self._chunk(c, w.chunk_slice(c), prev)
            self.segs.append(seg)
        self.prev = prev
        self.sl_new = w.chunk_slice(self.nch - 1)
        self.sl_prevq = w.chunk_slice(self.nch - 2)
        H, T = self.H, self.chunk
        self.Ck = torch.empty(H, 256, D, dtype=torch.bfloat16, device="cuda")
        self.Cv = torch.empty_like(self.Ck)
        self.kp = qwm.PackedChunk(T, H, True)
        self.vp = qwm.PackedChunk(T, H, False)
        # Two sets of statistics outputs (w, U, eigenvalues) over one running sum
        # (S, n): a step's keys read one set while the update for the next step
        # writes the other, so the update need not wait for the keys.  The new
        # chunk's segment names the basis its keys were coded with: one segment
        # table per set.
        self.stb = qwm.QueryStats(self.H)
        self.stb.S, self.stb.n = self.st.S, self.st.n
        self.stb.w.copy_(self.st.w)
        self.stb.U.copy_(self.st.U)
        self.stats = [self.st, self.stb]
        self.dsegs_pp = []
        for sx in self.stats:
            d = qwm.segment_array(self.segs + [(self.kp, self.vp, self.Ck, self.Cv, sx.U)])
            self.total = d.total
            self.dsegs_pp.append(d)
        self.parity = 0
        self.cur_seg = (self.kp, self.vp, self.Ck, self.Cv, self.st.U)   # the new chunk as last coded
        self.diag = qwm.new_diag()
        self.vdiag = qwm.new_diag()      # the V side counts on its own stream
        # the Query statistics and basis only feed the key quantization, and the V side
        # (table refresh, values) is independent of the K side: each runs on its own
        # stream.  The statistics a step's keys need come from the previous chunk's
        # Queries, so each step launches the next step's update (into the other
        # output set) at its start; it runs beside the step's Lloyd iterations and
        # keys (small, launch-bound kernels), not beside its attention
        self.side = torch.cuda.Stream()
        self.vside = torch.cuda.Stream()
        self.stats_done = [torch.cuda.Event(), torch.cuda.Event()]   # one per statistics set
        self.fork = torch.cuda.Event()
        self.v_done = torch.cuda.Event()
        self.primed = False
        self.queries = T
        self.new_tokens = T
        self.stage_names = ["lloyd_k", "side_launch_and_stats_wait", "keys", "values_wait", "attention"]

    def _chunk(self, c, sl, prev):
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
        if c < self.nch - 2:        # the step itself adds the previous chunk's Queries
            qwm.update_query_stats(self.Q[sl], self.st, compute_basis=True)
        return (kp, vp, Ck, Cv, U), (Ck, Cv)

    def run(self, events=None):
        qwm, torch = self.qwm, self.torch
        rec = (lambda i: events[i].record()) if events is not None else (lambda i: None)
        K, V = self.K[self.sl_new], self.V[self.sl_new]
        main = torch.cuda.current_stream()
        p = self.parity
        cur, nxt = self.stats[p], self.stats[p ^ 1]
        if not self.primed:          # the first step's statistics (afterwards: the previous step's launch)
            self.side.wait_stream(main)
            self._launch_stats(cur, p)
            self.primed = True
        rec(0)
        # the side streams start from here: after everything earlier on this stream,
        # the previous step's attention (which read set p ^ 1's basis) included
        self.fork.record(main)
        # the critical path is issued first: the K table refresh
        qwm.build_centroids(K, 3, init=self.prev[0], out=self.Ck, diag=self.diag)
        rec(1)
        self.side.wait_event(self.fork)
        self._launch_stats(nxt, p ^ 1)   # the next step's statistics (one update + basis per step)
        self.vside.wait_event(self.fork)
        with torch.cuda.stream(self.vside):
            qwm.build_centroids(V, 3, init=self.prev[1], out=self.Cv, diag=self.vdiag)
            qwm.quantize_values(V, self.Cv, out=self.vp, diag=self.vdiag)
            self.v_done.record(self.vside)
        main.wait_event(self.stats_done[p])
        rec(2)
        qwm.quantize_keys(K, self.Ck, cur.w, cur.U, M=8, flags=3, out=self.kp, diag=self.diag)
        self.cur_seg = (self.kp, self.vp, self.Ck, self.Cv, cur.U)
        rec(3)
        main.wait_event(self.v_done)
        rec(4)
        out, _, _ = qwm.attention(self.Q[self.sl_new], self.dsegs_pp[self.parity])
        rec(5)
        self.parity ^= 1
        return out

    def all_segs(self):
        """Every segment of the cache: the prefilled chunks and the new one."""
        return self.segs + [self.cur_seg]

    def join(self):
        """Make the current stream wait for the statistics the last step launched."""
        self.torch.cuda.current_stream().wait_event(self.stats_done[self.parity])

    def _launch_stats(self, st, i):
        with self.torch.cuda.stream(self.side):
            self.qwm.update_query_stats(self.Q[self.sl_prevq], st, compute_basis=True)
            self.stats_done[i].record(self.side)


class OnePass:
    """One pass over a single chunk (tiny): statistics
    and basis from the Queries, 10 seeded Lloyd iterations for K and V, keys,
    values, attention of the Queries over the chunk."""

    def __init__(self, qwm, torch, w):
        self.qwm, self.torch = qwm, torch
        self.H, self.chunk = w.H, w.chunk
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        dev = lambda a: torch.from_numpy(a).to(dt).cuda()
        self.K, self.V, self.Q = dev(w.K), dev(w.V), dev(w.Q)
        H, T = self.H, w.T
        self.st = qwm.QueryStats(H)
        self.Ck = torch.empty(H, 256, D, dtype=torch.bfloat16, device="cuda")
        self.Cv = torch.empty_like(self.Ck)
        self.kp = qwm.PackedChunk(T, H, True)
        self.vp = qwm.PackedChunk(T, H, False)
        self.dsegs = qwm.segment_array([(self.kp, self.vp, self.Ck, self.Cv, self.st.U)])
        self.total = self.dsegs.total
        self.diag = qwm.new_diag()
        self.nch = 1
        self.queries = int(w.Q.shape[0])
        self.new_tokens = T
        self.stage_names = ["stats_and_basis", "lloyd_kv_10", "keys", "values", "attention"]

    def run(self, events=None):
        qwm = self.qwm
        rec = (lambda i: events[i].record()) if events is not None else (lambda i: None)
        rec(0)
        self.st.reset()
        qwm.update_query_stats(self.Q, self.st, compute_basis=True)
        rec(1)
        qwm.build_centroids(self.K, 10, seed=1, out=self.Ck, diag=self.diag)
        qwm.build_centroids(self.V, 10, seed=2, out=self.Cv, diag=self.diag)
        rec(2)
        qwm.quantize_keys(self.K, self.Ck, self.st.w, self.st.U, M=8, flags=3, out=self.kp, diag=self.diag)
        rec(3)
        qwm.quantize_values(self.V, self.Cv, out=self.vp, diag=self.diag)
        rec(4)
        out, _, _ = qwm.attention(self.Q, self.dsegs)
        rec(5)
        return out


class FullDepth:
    """The full-depth memory case: every layer's cache resident in HBM; one
    step runs the whole hot path over all layers.

    Per layer, three streams: the statistics and basis on one side stream
    (they feed only the keys), the V table and the values on another (they
    feed only the attention), the K table, the keys and the attention on the
    main stream.  The two tables' Lloyd iterations share the GPU; the key call
    starts once the V side is done, so it has the GPU to itself, as does the
    attention after it.  HIP events on the main stream bracket every key call
    and every attention call."""

    LLOYD_ITERS = 10

    def __init__(self, qwm, torch, datagen, layers, f_energy=None):
        self.qwm, self.torch = qwm, torch
        self.L = layers
        self.layers = []
        for l in range(layers):
            K, V, Q = datagen.device_layer("depth", l, f_energy=f_energy)
            self.layers.append((K, V, Q))
        K0, _, Q0 = self.layers[0]
        self.T, self.H = K0.shape[0], K0.shape[1]
        self.queries = Q0.shape[0]
        H, T = self.H, self.T
        self.st, self.Ck, self.Cv, self.kp, self.vp, self.segs = [], [], [], [], [], []
        for l in range(layers):
            st = qwm.QueryStats(H)
            Ck = torch.empty(H, 256, D, dtype=torch.bfloat16, device="cuda")
            Cv = torch.empty_like(Ck)
            kp = qwm.PackedChunk(T, H, True)
            vp = qwm.PackedChunk(T, H, False)
            self.st.append(st); self.Ck.append(Ck); self.Cv.append(Cv); self.kp.append(kp); self.vp.append(vp)
            self.segs.append(qwm.segment_array([(kp, vp, Ck, Cv, st.U)]))
        self.diag = qwm.new_diag()
        self.vdiag = qwm.new_diag()
        self.side = torch.cuda.Stream()
        self.vside = torch.cuda.Stream()
        self.fork = [torch.cuda.Event() for _ in range(layers)]
        self.stats_done = [torch.cuda.Event() for _ in range(layers)]
        self.v_done = [torch.cuda.Event() for _ in range(layers)]
        self.total = T
        self.nch = 1
        self.new_tokens = T * layers
        self.out = None

    def run(self, events=None):
        """events: None, or a list that receives one (keys start, keys end,
        attention start, attention end) tuple of timing events per layer."""
        qwm, torch = self.qwm, self.torch
        main = torch.cuda.current_stream()
        for l in range(self.L):
            K, V, Q = self.layers[l]
            st = self.st[l]
            self.fork[l].record(main)
            self.side.wait_event(self.fork[l])
            with torch.cuda.stream(self.side):
                st.reset()
                qwm.update_query_stats(Q, st, compute_basis=True)
                self.stats_done[l].record(self.side)
            self.vside.wait_event(self.fork[l])
            with torch.cuda.stream(self.vside):
                qwm.build_centroids(V, self.LLOYD_ITERS, seed=2, out=self.Cv[l], diag=self.vdiag)
                qwm.quantize_values(V, self.Cv[l], out=self.vp[l], diag=self.vdiag)
                self.v_done[l].record(self.vside)
            qwm.build_centroids(K, self.LLOYD_ITERS, seed=1, out=self.Ck[l], diag=self.diag)
            main.wait_event(self.stats_done[l])
            main.wait_event(self.v_done[l])
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if events is not None else None
            if ev: ev[0].record(main)
            qwm.quantize_keys(K, self.Ck[l], st.w, st.U, M=8, flags=3, out=self.kp[l], diag=self.diag)
            if ev: ev[1].record(main)
            if ev: ev[2].record(main)
            self.out, _, _ = qwm.attention(Q, self.segs[l])
            if ev: ev[3].record(main)
            if ev: events.append(ev)
        return self.out

    def resident_bytes(self):
        """Bytes the compressed cache holds: packed chunks plus per-(layer, head)
        tables (K and V centroids, the basis)."""
        packed = sum(kp.nbytes() + vp.nbytes() for kp, vp in zip(self.kp, self.vp))
        tables = self.L * self.H * SEG_TABLE_BYTES_PER_HEAD
        return packed, tables


def depth_timed(step, torch, steps, warmup):
    """Warm-up, then `steps` timed steps bracketed by synchronisation; per-call
    key and attention times from the events of every layer of every step."""
    import numpy as np
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    for d in (step.diag, step.vdiag):
        d.zero_()
    step.run()
    torch.cuda.synchronize()
    diag_step = (step.diag + step.vdiag).tolist()
    evs = []
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(steps):
        step.run(evs)
    torch.cuda.current_stream().wait_stream(step.side)
    torch.cuda.current_stream().wait_stream(step.vside)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_end) / steps
    keys_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    attn_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    return ms, keys_ms, attn_ms, wall, diag_step


def stage_rooflines(torch, qwm, step, keys_ms, attn_ms):
    """Kernel-level rates of the depth layer's stages, each against the roofline
    that bounds it (algorithmic work per unit as the design notes state it),
    timed one call at a time after the step (layer 0's inputs)."""
    H, T, Tq = step.H, step.T, step.queries
    K, V, Q = step.layers[0]
    st, Ck, Cv, kp, vp = step.st[0], step.Ck[0], step.Cv[0], step.kp[0], step.vp[0]

    def timed(fn, n=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    st2 = qwm.QueryStats(H)
    iters = FullDepth.LLOYD_ITERS
    lbuild = timed(lambda: qwm.build_centroids(K, iters, seed=1, out=torch.empty_like(Ck)))
    vals = timed(lambda: qwm.quantize_values(V, Cv, out=vp))
    stats = timed(lambda: (st2.reset(), qwm.update_query_stats(Q, st2, compute_basis=True)))
    kms = float(keys_ms.mean())
    ams = float(attn_ms.mean())
    th = T * H
    kbytes = KEY_BYTES_PER_TOKEN_HEAD * th + KEY_TABLE_BYTES_PER_HEAD * H
    vbytes = VALUE_BYTES_PER_TOKEN_HEAD * th + 256 * 128 * 2 * H
    aflop = ATTN_FLOP_PER_QKH * Tq * T * H
    abytes = PACKED_BYTES_PER_KEY_HEAD * T * H + SEG_TABLE_BYTES_PER_HEAD * H + Tq * H * (256 + 512)
    lflop = LLOYD_FLOP_PER_TOKEN_HEAD * th
    return {
        "keys": {"bound": "hbm", "ms": round(kms, 4), "GBps": round(kbytes / kms / 1e6, 1),
                 "frac": round(kbytes / kms / 1e6 / HBM_PEAK_GBPS, 4), "bytes_per_call": int(kbytes),
                 "token_heads_per_s": round(th / (kms * 1e-3), 1)},
        "values": {"bound": "hbm", "ms": round(vals, 4), "GBps": round(vbytes / vals / 1e6, 1),
                   "frac": round(vbytes / vals / 1e6 / HBM_PEAK_GBPS, 4), "bytes_per_call": int(vbytes)},
        "lloyd_build": {"bound": "mfma", "iterations": iters, "ms": round(lbuild, 4),
                        "ms_per_iteration": round(lbuild / iters, 4),
                        "TFLOPs_equivalent": round(iters * lflop / lbuild / 1e9, 1),
                        "frac_equivalent": round(iters * lflop / lbuild / 1e9 / MFMA_F16_PEAK_TFLOPS, 4),
                        "note": "the seeded table build of the step (one tensor, all heads): two full iterations, "
                                "then iterations that re-assign only the tokens whose distance bounds no longer "
                                "settle their centroid; the rate counts the GEMM FLOPs of that many full "
                                "assignments"},
        "attention": {"bound": "mfma", "ms": round(ams, 4), "TFLOPs": round(aflop / ams / 1e9, 1),
                      "frac": round(aflop / ams / 1e9 / MFMA_F16_PEAK_TFLOPS, 4),
                      "compressed_GBps": round(abytes / ams / 1e6, 1)},
        "stats_and_basis": {"bound": "latency", "ms": round(stats, 4)},
    }


def _pool_worker_init():
    """Worker set-up: the oracle's BLAS on one thread per worker."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_keys_unit(args):
    """One (layer, head) unit of the CPU baseline: the oracle's statistics and
    Jacobi basis from the layer's Queries, its Forgy table over the head's
    tokens, then its QSAC + PSAC key quantization of `rows` tokens, timed."""
    import numpy as np
    from oracle import lloyd as OL, quantize as Qz, stats as OS
    K, Q, rows, seed, head = args
    S, n = OS.update(np.zeros((D, D)), 0, Q.astype(np.float64))
    basis = OS.principal_basis(S, n)
    wts = OS.channel_weights(S, n)
    C0 = OL.lloyd(K.astype(np.float64), 256, 0, seed=seed, head=head)
    t0 = time.perf_counter()
    o = Qz.quantize_keys(K[:rows].astype(np.float64), C0, wts, basis["U_bf16"], M=8, flags=3)
    dt = time.perf_counter() - t0
    return {"head": head, "seconds": dt, "rows": rows, "table": C0, "w": wts, "U": basis["U_bf16"],
            "idx": o["idx"], "q": o["q"], "scale_bits": o["scale_bits"], "zero": o["zero"], "Cq": o["Cq"],
            "c_scale_bits": o["c_scale_bits"], "dq": o["info"]["dq"]}


def start_cpu_pool():
    """The oracle's worker pool, started before anything touches the GPU (its
    workers come from a fork server that never initialises the device)."""
    import multiprocessing as mp
    n = max(1, min(len(os.sched_getaffinity(0)), 16))
    ctx = mp.get_context("forkserver")
    return ctx.Pool(n, initializer=_pool_worker_init), n


def _near_tie(k, C, w, o_j, g_j, dq, M, rel=1e-6):
    """Whether a GPU centroid choice g_j that differs from the oracle's o_j is a
    near-tie of the oracle's own scores: QSAC scores S within `rel`, or, when
    the GPU's choice lies outside the oracle's M nearest by d_Q, the d_Q values
    at that boundary within `rel`."""
    import numpy as np
    from oracle import quantize as Qz
    Wg = np.asarray(w, np.float64).reshape(-1, 64).sum(axis=1)

    def S_of(j):
        _, _, R = Qz.group_ranges(Qz.residual(np.asarray(k, np.float64)[None], np.asarray(C)[j][None]))
        return float(Qz.qsac_score(R, Wg)[0])
    so, sg = S_of(o_j), S_of(g_j)
    if abs(sg - so) <= rel * max(so, 1e-300):
        return True
    order = np.argsort(dq, kind="stable")
    if g_j not in order[:M]:
        dm = dq[order[M - 1]]
        return abs(dq[g_j] - dm) <= rel * max(dm, 1e-300)
    return False


def cpu_baseline_depth(pool, workers, qwm, torch, step, rows=4096):
    """The oracle, untuned, on a bounded sample of the depth workload's key
    quantization: `workers` (layer 0, head) units in parallel, each the first
    `rows` tokens of one head.  Also a parity sample: the GPU's key call on the
    same heads with the oracle's tables, weights and basis, compared with the
    oracle's outputs (indices, codes, scales, zero-points, C)."""
    import numpy as np
    from oracle import formats as F
    K, _, Q = step.layers[0]
    heads = list(range(min(workers, step.H)))
    Kh = K[:, heads].float().cpu().numpy()
    Qh = Q[:, heads].float().cpu().numpy()
    units = [(np.ascontiguousarray(Kh[:, i]), np.ascontiguousarray(Qh[:, i]), rows, 1, h) for i, h in enumerate(heads)]
    t0 = time.perf_counter()
    res = pool.map(_oracle_keys_unit, units)
    wall = time.perf_counter() - t0
    cpu_s = sum(r["seconds"] for r in res)
    token_heads = rows * len(heads)
    keys_wall = max(r["seconds"] for r in res)
    value = token_heads / keys_wall / step.H          # token positions across all heads
    # parity sample: the GPU key call on the sampled heads with the oracle's inputs
    Kd = K[:rows, heads].contiguous()
    tab = torch.from_numpy(np.stack([r["table"] for r in res]).astype(np.float32)).to(torch.bfloat16).cuda()
    wt = torch.from_numpy(np.stack([r["w"] for r in res]).astype(np.float32)).cuda()
    Ub = torch.from_numpy(np.stack([r["U"] for r in res]).astype(np.float32)).to(torch.bfloat16).cuda()
    kp = qwm.quantize_keys(Kd, tab, wt, Ub, M=8, flags=3)
    torch.cuda.synchronize()
    gidx = kp.idx.cpu().numpy()
    gcodes = kp.codes.cpu().numpy()
    gscale = kp.scale.cpu().numpy().view(np.uint16)
    gz = kp.zeros.cpu().numpy()
    gc = kp.c.cpu().numpy()
    mism = near = code_bad = c_lsb2 = 0
    c_lsb1 = 0
    for i, r in enumerate(res):
        o_idx = r["idx"].astype(np.int64)
        g_idx = gidx[i].astype(np.int64)
        bad = np.nonzero(o_idx != g_idx)[0]
        mism += len(bad)
        for t in bad:
            near += int(_near_tie(Kh[t, i], r["table"], r["w"], int(o_idx[t]), int(g_idx[t]), r["dq"][t], 8))
        same = o_idx == g_idx
        q = F.unpack_codes(gcodes[i], 128)
        zz = F.unpack_zeros(gz[i][: (rows + 1) // 2], rows)
        code_bad += int(np.sum(np.any(q[same] != r["q"][same], axis=1) | np.any(gscale[i][same] != r["scale_bits"][same], axis=1)
                               | np.any(zz[same] != r["zero"][same], axis=1)))
        dc = np.abs(gc[i].astype(np.int64) - r["Cq"].astype(np.int64))[same]
        c_lsb1 += int(np.sum(dc == 1))
        c_lsb2 += int(np.sum(dc > 1))
    return {
        "cpu_baseline": {"value": round(value, 2), "unit": "tokens/s", "cores": workers, "kind": "oracle",
                         "sample": f"key quantization (QSAC + PSAC, M = 8) of the first {rows:,} tokens of heads "
                                   f"0-{len(heads) - 1} of layer 0 of the depth cache, one (layer, head) unit per "
                                   f"worker process ({workers} workers, BLAS 1 thread each); tokens/s = token-heads/s "
                                   f"/ {step.H} heads, from the slowest unit's time",
                         "token_heads_per_s": round(token_heads / keys_wall, 1), "cpu_seconds": round(cpu_s, 2),
                         "wall_s_with_setup": round(wall, 2)},
        "parity_sample": {"token_heads": token_heads, "idx_mismatches": mism, "near_ties": near,
                          "mismatches_beyond_near_ties": mism - near, "codec_mismatches_on_equal_idx": code_bad,
                          "c_off_by_1_lsb": c_lsb1, "c_off_by_more": c_lsb2,
                          "note": "GPU qwm_quantize_keys on the sampled heads with the oracle's own Forgy table, "
                                  "weights and basis, against the oracle's outputs"},
    }


def rollout_ablations(qwm, torch, datagen, chunks=40):
    """The causal rollout (H = 24, 40 chunks of 1,560 tokens, drawn on the
    device) under each ablation: per-ablation tokens/s and the top-1 shift
    rate against attention over the bf16 keys."""
    import numpy as np
    Kd, Vd, Qd = datagen.device_layer("rollout", 0)
    H, T = Kd.shape[1], 1560
    refs = []
    for t in range(chunks):
        sl = slice(t * T, (t + 1) * T)
        refs.append(qwm.reference_top1(Qd[sl], Kd[: sl.stop]))
    names = {0: "nearest", 1: "qsac", 2: "psac", 3: "qsac+psac"}
    out = {}
    for flags in (0, 1, 2, 3):
        for _ in range(2):
            st = qwm.QueryStats(H)
            segs, prev, tops = [], None, []
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for t in range(chunks):
                sl = slice(t * T, (t + 1) * T)
                K, V = Kd[sl], Vd[sl]
                if prev is None:
                    Ck = qwm.build_centroids(K, 10, seed=1)
                    Cv = qwm.build_centroids(V, 10, seed=2)
                    U = None
                    kp = qwm.quantize_keys(K, Ck, None, None, M=8, flags=flags)
                else:
                    Ck = qwm.build_centroids(K, 3, init=prev[0])
                    Cv = qwm.build_centroids(V, 3, init=prev[1])
                    U = st.U.clone() if flags & 2 else None
                    kp = qwm.quantize_keys(K, Ck, st.w if flags & 1 else None, U, M=8, flags=flags)
                vp = qwm.quantize_values(V, Cv)
                segs.append((kp, vp, Ck, Cv, U))
                _, _, top1 = qwm.attention(Qd[sl], qwm.segment_array(segs), want_top1=True)
                tops.append(top1)
                qwm.update_query_stats(Qd[sl], st, compute_basis=True)
                prev = (Ck, Cv)
            torch.cuda.synchronize()
            secs = time.perf_counter() - t0
        rates = [float((tops[t] != refs[t]).float().mean().item()) for t in range(chunks)]
        out[names[flags]] = {"tokens_per_s": round(chunks * T / secs, 1), "seconds": round(secs, 4),
                             "shift_rate": round(float(np.mean(rates[1:])), 5),
                             "shift_rate_cold_start": round(rates[0], 5)}
    out["workload"] = (f"rollout: H={H}, d=128, {chunks} chunks x {T:,} tokens drawn on the device, causal "
                       f"statistics, 10 seeded + 3 warm Lloyd iterations per chunk, attention of each chunk's "
                       f"Queries over the cache so far; shift = top-1 key differs from the top-1 over the bf16 keys")
    return out


def rank_sweep(qwm, torch, step, ranks=(8, 16, 32)):
    """The pages' PSAC rank ablation on layer 0 of the depth cache: basis,
    QSAC + PSAC keys and attention at each rank, with the stored bits per
    token-head (K + V, dense coefficients) and the extra bits per cached
    element over rank 8 (the pages report +0.1341 and +0.2569 bit going from
    8 to 16 on two models)."""
    K, V, Q = step.layers[0]
    H, T = step.H, step.T
    Ck, Cv, vp = step.Ck[0], step.Cv[0], step.vp[0]
    out = {}

    def timed(fn, n=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for r in ranks:
        st = qwm.QueryStats(H, r=r)
        t_stats = timed(lambda: (st.reset(), qwm.update_query_stats(Q, st, compute_basis=True)))
        kp = qwm.PackedChunk(T, H, True, r=r)
        t_keys = timed(lambda: qwm.quantize_keys(K, Ck, st.w, st.U, M=8, flags=3, out=kp))
        segs = qwm.segment_array([(kp, vp, Ck, Cv, st.U)])
        t_attn = timed(lambda: qwm.attention(Q, segs))
        bits = (kp.nbytes() + vp.nbytes()) * 8 / (H * T)
        out[str(r)] = {"stats_and_basis_ms": round(t_stats, 4), "keys_ms": round(t_keys, 4),
                       "attention_ms": round(t_attn, 4), "bits_per_token_head": round(bits, 2),
                       "extra_bits_per_element_vs_r8": round((bits - 680.0) / 256.0, 4),
                       "eig_iterations_max": int(st.iters.abs().max().item())}
    out["note"] = ("rank 8: subspace-iteration basis and coefficients fused into the selection kernel; ranks 16 "
                   "and 32: one-sided Jacobi basis and an exact fp64 coefficient pass; the attention kernel takes "
                   "one PSAC k-step for ranks up to 16 and two for 32")
    return out


def storage_refinements(qwm, torch, step):
    """The storage refinements on layer 0 of the depth cache: the keep test
    (diagonal in the key kernel, and the full e^T M e form as a pass), the
    per-head dense / sparse coefficient layout, and two-level INT8 + FP16
    group scales; resident bits per token-head and the attention time over
    each stored form."""
    K, V, Q = step.layers[0]
    H, T = step.H, step.T
    st, Ck, Cv = step.st[0], step.Ck[0], step.Cv[0]

    def timed(fn, n=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    out = {}
    vp = qwm.quantize_values(V, Cv)
    for name, flags, full in (("plain", 3, False), ("keep_diagonal", 7, False), ("keep_full", 3, True)):
        kp = qwm.quantize_keys(K, Ck, st.w, st.U, M=8, flags=flags)
        ms_keep = timed(lambda: qwm.psac_keep_full(K, Ck, st, st.U, kp)) if full else None
        kept = float((kp.c_scale != 0).float().mean().item())
        dense_bytes = kp.nbytes()
        ms_compact = timed(lambda: qwm.compact_coefficients(kp))
        lay = kp.layouts()
        seg = qwm.segment_array([(kp, vp, Ck, Cv, st.U)])
        ms_attn = timed(lambda: qwm.attention(Q, seg))
        out[name] = {"kept_fraction": round(kept, 5), "sparse_heads": sum(1 for l in lay if l[0] == 1),
                     "key_bytes_dense": int(dense_bytes), "key_bytes_stored": int(kp.nbytes()),
                     "compact_ms": round(ms_compact, 4), "attention_ms": round(ms_attn, 4)}
        if full:
            out[name]["keep_full_pass_ms"] = round(ms_keep, 4)
    # two-level scales on keys and values
    kp = qwm.quantize_keys(K, Ck, st.w, st.U, M=8, flags=3)
    vp2 = qwm.quantize_values(V, Cv)
    ms_two = timed(lambda: (qwm.two_level_scales(K, Ck, kp, st.w, st.U, flags=3),
                            qwm.two_level_scales(V, Cv, vp2)), n=1)
    seg = qwm.segment_array([(kp, vp2, Ck, Cv, st.U)])
    ms_attn = timed(lambda: qwm.attention(Q, seg))
    bits = (kp.nbytes() + vp2.nbytes()) * 8 / (H * T)
    out["two_level"] = {"bits_per_token_head": round(bits, 2), "convert_ms": round(ms_two, 4),
                        "attention_ms": round(ms_attn, 4),
                        "ratio_per_token_vs_bf16": round(4096 / bits, 3)}
    return out


def run_depth(args, qwm, torch, datagen, pool):
    import numpy as np
    log(f"drawing {args.layers} depth layers on the device")
    step = FullDepth(qwm, torch, datagen, args.layers, f_energy=args.f_energy)
    torch.cuda.synchronize()
    log("timing")
    ms, keys_ms, attn_ms, wall, diag_step = depth_timed(step, torch, args.steps, args.warmup)
    L, H, T, Tq = step.L, step.H, step.T, step.queries
    keys_total_s = float(keys_ms.sum()) * 1e-3
    value = L * T * args.steps / keys_total_s
    config = {"workload": f"full-depth memory case: {L} layers x H={H} heads x d=128, {T:,} cached tokens per "
                          f"layer (bf16 K+V {L * H * T * 2 * D * 2 / 2 ** 30:.2f} GiB resident), {Tq:,} Queries per "
                          f"layer; per layer: statistics + basis, 10 seeded Lloyd iterations for K and for V, "
                          f"QSAC+PSAC keys (M=8, r=8, 256 centroids), values, attention over the layer's 2-bit cache",
              "layers": L, "heads": H, "tokens_per_layer": T, "queries_per_layer": Tq}
    if args.f_energy is not None:
        config["f_energy"] = args.f_energy
    res = base_result(args, value, ms, "bf16", config)
    res["value_definition"] = ("token positions (all heads) quantized per second by qwm_quantize_keys "
                               "(QSAC+PSAC), summed over the HIP-event times of every key call of the timed steps")
    res["step_tokens_per_s"] = round(L * T / (ms * 1e-3), 1)
    flops = ATTN_FLOP_PER_QKH * Tq * T * H
    am = float(attn_ms.mean())
    ach = flops / (am * 1e-3) / 1e12
    abytes = PACKED_BYTES_PER_KEY_HEAD * T * H + SEG_TABLE_BYTES_PER_HEAD * H + Tq * H * (256 + 512)
    res["roofline"] = {"kernel": "qwm_attention (fused dequant + PSAC + online softmax; the call's kernels: "
                                 "attention_tables_kernel, attention_kernel, attention_combine_kernel)",
                       "bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4), "traffic": attention_traffic(DEPTH_TRAFFIC_FILE),
                       "flop_per_launch": int(flops), "avg_launch_ms": round(am, 4), "launches": int(len(attn_ms)),
                       "algorithmic_bytes_per_launch": int(abytes),
                       "compressed_GBps": round(abytes / (am * 1e-3) / 1e9, 1)}
    kb = KEY_BYTES_PER_TOKEN_HEAD * T * H + KEY_TABLE_BYTES_PER_HEAD * H
    km = float(keys_ms.mean())
    res["keys"] = {"avg_call_ms": round(km, 4), "calls": int(len(keys_ms)), "token_heads_per_call": T * H,
                   "GBps": round(kb / (km * 1e-3) / 1e9, 1), "hbm_frac": round(kb / (km * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   "algorithmic_bytes_per_call": int(kb)}
    res["stage_rooflines"] = stage_rooflines(torch, qwm, step, keys_ms, attn_ms)
    packed, tables = step.resident_bytes()
    bf16 = L * H * T * 2 * D * 2
    res["resident"] = {"packed_bytes": int(packed), "table_bytes": int(tables),
                       "GiB": round((packed + tables) / 2 ** 30, 3), "bf16_GiB": round(bf16 / 2 ** 30, 3),
                       "ratio": round(bf16 / (packed + tables), 3), "ratio_without_tables": round(bf16 / packed, 3),
                       "bits_per_token_head": round(packed * 8 / (L * H * T), 2)}
    res["device_counters_per_step"] = {"nonfinite_rows": int(diag_step[0]), "exact_fallbacks": int(diag_step[1]),
                                       "scale_saturations": int(diag_step[2])}
    res["wall_s_timed"] = round(wall, 3)
    if not args.no_extras:
        log("rank sweep")
        res["rank_sweep"] = rank_sweep(qwm, torch, step)
        log("storage refinements")
        res["storage_refinements"] = storage_refinements(qwm, torch, step)
    if not (args.no_rollout or args.no_extras):
        log("rollout ablations")
        res["rollout_ablations"] = rollout_ablations(qwm, torch, datagen)
    if pool is not None:
        log("timing the CPU oracle sample")
        res.update(cpu_baseline_depth(pool[0], pool[1], qwm, torch, step))
    return res


def cpu_baseline(w, nq, heads=6):
    """The oracle (untuned) on a bounded sample of the 480p step: the quantize
    side (statistics + Jacobi basis, 3 + 3 Lloyd iterations, QSAC + PSAC keys,
    values of the new chunk) for `heads` of the 12 heads, attention of `nq`
    Queries of head 0 over all 25 segments (seeded random packed contents);
    extrapolated to the whole step (12 heads, 1,560 Queries)."""
    import numpy as np
    from oracle import attention as OA, lloyd as OL, quantize as Qz, stats as OS
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    H, CHUNK, NCHUNK = w.H, w.chunk, w.n_chunks
    sl = w.chunk_slice(NCHUNK - 1)
    slp = w.chunk_slice(NCHUNK - 2)
    t_quant = 0.0
    tables = None
    for h in range(heads):
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
        Qz.quantize_keys(K, Ck, wts, basis["U_bf16"], M=8)
        Qz.quantize_values(Vv, Cv)
        t_quant += time.perf_counter() - t0
        if tables is None:
            tables = (Ck, Cv, basis["U_bf16"])
    rng = np.random.default_rng(5)
    segs = []
    Ck, Cv, U = tables
    for s in range(NCHUNK):
        q = rng.integers(0, 4, (CHUNK, 128)).astype(np.uint8)
        z = rng.integers(0, 4, (CHUNK, 2)).astype(np.uint8)
        sc = rng.uniform(0.01, 0.2, (CHUNK, 2)).astype(np.float16).astype(np.float64)
        segs.append(dict(k_idx=rng.integers(0, 256, CHUNK), k_q=q, k_scale=sc, k_zero=z,
                         k_Cq=rng.integers(-127, 128, (CHUNK, 8)), k_cs=np.full(CHUNK, 1e-3),
                         k_centroids=Ck, U=U, v_idx=rng.integers(0, 256, CHUNK), v_q=q,
                         v_scale=sc, v_zero=z, v_centroids=Cv))
    Qs = w.Q[sl, 0][:nq].astype(np.float64)
    t1 = time.perf_counter()
    OA.cache_attention(Qs, segs, 1 / np.sqrt(D))
    t_attn = time.perf_counter() - t1
    step_s = t_quant * H / heads + t_attn * H * CHUNK / nq
    return {"value": round(CHUNK / step_s, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"quantize side of the step for {heads} of {H} heads: stats + Jacobi basis, 3 + 3 Lloyd "
                      f"iterations, QSAC + PSAC keys and values of the 1,560-token chunk ({t_quant:.2f} s); "
                      f"attention of {nq} Queries of one head over 39,000 keys ({t_attn:.2f} s); extrapolated "
                      f"to {H} heads and 1,560 Queries",
            "seconds_sampled": round(t_quant + t_attn, 2)}


def keys_bulk(qwm, torch, Kall, table, st):
    """Key quantization of many tokens in one call (QSAC + PSAC): HBM rate."""
    H = Kall.shape[1]
    kb = qwm.PackedChunk(Kall.shape[0], H, True)
    for _ in range(2):
        qwm.quantize_keys(Kall, table, st.w, st.U, M=8, flags=3, out=kb)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    nb = 5
    for _ in range(nb):
        qwm.quantize_keys(Kall, table, st.w, st.U, M=8, flags=3, out=kb)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / nb
    byts = KEY_BYTES_PER_TOKEN_HEAD * Kall.shape[0] * H + KEY_TABLE_BYTES_PER_HEAD * H
    return {"tokens": int(Kall.shape[0]), "token_heads": int(Kall.shape[0]) * H, "ms": round(ms, 4),
            "tokens_per_s": round(Kall.shape[0] / (ms * 1e-3), 1),
            "GBps": round(byts / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def keys_keep_test(qwm, torch, Kall, table, st):
    """Bulk key quantization with the PSAC keep test (flags QSAC | PSAC | KEEP):
    time, and the fraction of tokens that keep their coefficients."""
    H = Kall.shape[1]
    kb = qwm.PackedChunk(Kall.shape[0], H, True)
    flags = qwm.QWM_QSAC | qwm.QWM_PSAC | qwm.QWM_PSAC_KEEP
    qwm.quantize_keys(Kall, table, st.w, st.U, M=8, flags=flags, out=kb)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        qwm.quantize_keys(Kall, table, st.w, st.U, M=8, flags=flags, out=kb)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    kept = float((kb.c_scale != 0).float().mean().item())
    return {"ms": round(ms, 4), "tokens_per_s": round(Kall.shape[0] / (ms * 1e-3), 1), "kept_fraction": round(kept, 4)}


def keys_m_sweep(qwm, torch, Kall, table, st, Ms=(4, 8, 16, 256)):
    """The pages' candidate-count ablation (QSAC's M): bulk key quantization
    (QSAC + PSAC) at each M, same tokens and tables."""
    H = Kall.shape[1]
    kb = qwm.PackedChunk(Kall.shape[0], H, True)
    diag = qwm.new_diag()
    out = {}
    for M in Ms:
        qwm.quantize_keys(Kall, table, st.w, st.U, M=M, flags=3, out=kb)
        torch.cuda.synchronize()
        diag.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            qwm.quantize_keys(Kall, table, st.w, st.U, M=M, flags=3, out=kb, diag=diag)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        out[str(M)] = {"ms": round(ms, 4), "tokens_per_s": round(Kall.shape[0] / (ms * 1e-3), 1),
                       "exact_fallbacks": int(diag.tolist()[1]) // 3}
    return out


def keys_full_matrix(qwm, torch, K, table, st, M=8):
    """The pages' full-matrix ablation of QSAC (candidates by the Query
    second-moment matrix instead of its diagonal), QSAC + PSAC on the new chunk,
    beside the diagonal call on the same tokens; also the share of tokens whose
    centroid the full form changes."""
    H = K.shape[1]
    kd = qwm.PackedChunk(K.shape[0], H, True)
    kf = qwm.PackedChunk(K.shape[0], H, True)
    out = {"workload": f"{K.shape[0]} tokens x {H} heads, M={M}"}
    for name, call in (("diagonal", lambda: qwm.quantize_keys(K, table, st.w, st.U, M=M, flags=3, out=kd)),
                       ("full", lambda: qwm.quantize_keys_fullq(K, table, st.S, st.n, st.w, st.U, M=M, flags=3,
                                                                out=kf))):
        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        out[name] = {"ms": round(ms, 4), "token_heads_per_s": round(K.shape[0] * H / (ms * 1e-3), 1)}
    out["idx_changed_fraction"] = round(float((kd.idx != kf.idx).float().mean().item()), 4)
    return out


def prq_codec(qwm, torch, X, stages=(1, 2, 3), iters=10):
    """QVG's progressive residual quantization as a second codec workload: all
    stages (seeded Lloyd on each stage's residual, nearest assignment, fp32
    residual) and the last stage's INT2 codes, for 1 to 3 stages."""
    out = {}
    for S in stages:
        qwm.prq_quantize(X, S, iters=iters, seed=1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            qwm.prq_quantize(X, S, iters=iters, seed=1)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        out[str(S)] = {"ms": round(ms, 4), "token_heads_per_s": round(X.shape[0] * X.shape[1] / (ms * 1e-3), 1)}
    out["workload"] = f"{X.shape[0]} tokens x {X.shape[1]} heads, {iters} seeded Lloyd iterations per stage"
    return out


def decode_ab(qwm, torch, step, fused_ms):
    """The pages' read path for comparison: decode every packed chunk to BF16
    (K_hat with PSAC, V_hat), then dense attention over the decoded rows, against
    the fused dequantizing attention timed in the step."""
    H, total = step.H, step.total
    Kd = torch.empty(total, H, D, dtype=torch.bfloat16, device="cuda")
    Vd = torch.empty_like(Kd)
    Q = step.Q[step.sl_new]

    def decode_all():
        pos = 0
        for (kp, vp, kc, vc, U) in step.all_segs():
            qwm.decode_segment(kp, vp, kc, vc, U, Kd[pos:pos + kp.T], Vd[pos:pos + kp.T])
            pos += kp.T

    def dense():
        qwm.attention(Q, None, active=(Kd, Vd))

    for f in (decode_all, dense):
        f()
    torch.cuda.synchronize()
    res = {}
    for name, f in (("decode_ms", decode_all), ("dense_attention_ms", dense)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            f()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / 5, 4)
    res["decode_plus_dense_ms"] = round(res["decode_ms"] + res["dense_attention_ms"], 4)
    res["fused_ms"] = round(fused_ms, 4)
    res["decoded_bytes"] = int(2 * total * H * D * 2)
    res["note"] = ("decoder: every chunk's BF16 K_hat (PSAC included) and V_hat written to HBM, then the same "
                   "attention kernel reads them as one BF16 chunk; fused: dequantization into LDS inside attention")
    return res


def timed_steps(step, torch, steps, warmup):
    import numpy as np
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    diags = [step.diag] + ([step.vdiag] if hasattr(step, "vdiag") else [])
    for d in diags:
        d.zero_()
    step.run()
    torch.cuda.synchronize()
    diag_step = sum(d for d in diags).tolist()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        step.run(evs[i])
    if hasattr(step, "join"):
        step.join()      # work the timed steps launched on side streams
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_end) / steps
    stage = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(step.stage_names)}
    return ms, stage, wall, diag_step


def roofline(step, attn_ms):
    flops = ATTN_FLOP_PER_QKH * step.queries * step.total * step.H
    achieved = flops / (attn_ms * 1e-3) / 1e12
    attn_bytes = PACKED_BYTES_PER_KEY_HEAD * step.total * step.H + SEG_TABLE_BYTES_PER_HEAD * step.H * step.nch \
        + step.queries * step.H * (256 + 512)
    return {"kernel": "attention (fused dequant + PSAC + online softmax; the call includes the fp16 table "
                      "conversion and the split merge)",
            "bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
            "flop_per_launch": flops, "avg_launch_ms": round(attn_ms, 4),
            "algorithmic_bytes_per_launch": int(attn_bytes),
            "compressed_GBps": round(attn_bytes / (attn_ms * 1e-3) / 1e9, 1)}


def base_result(args, metric_value, ms, dtype, config):
    return {
        "metric": "Key tokens/s quantized (QSAC+PSAC) + compressed-cache attention MFMA %/HBM GB/s",
        "value": round(metric_value, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic", "config": config,
    }


def run_stream_or_pass(args, qwm, torch, w):
    if args.workload in ("480p", "720p"):
        log(f"prefilling {w.n_chunks - 1} chunks")
        step = Stream(qwm, torch, w)
        config = {"workload": f"{args.workload}-shaped single layer, streaming step: H={w.H}, d=128, "
                              f"{w.n_chunks - 1} cached chunks + 1 new chunk of {w.chunk:,} tokens "
                              f"({w.chunk * w.n_chunks:,} keys in {w.n_chunks} segments), {w.chunk:,} queries; "
                              f"M=8, r=8, 256 centroids, 3 warm Lloyd iterations",
                  "heads": w.H, "chunk_tokens": w.chunk, "cached_keys": w.chunk * w.n_chunks, "queries": w.chunk}
    else:
        step = OnePass(qwm, torch, w)
        config = {"workload": f"{args.workload}: one pass over {w.T:,} tokens x {w.H} heads ({w.dtype}), "
                              f"{w.Q.shape[0]:,} queries; 10 seeded Lloyd iterations, M=8, r=8",
                  "heads": w.H, "tokens": w.T, "queries": int(w.Q.shape[0])}
    if args.f_energy is not None:
        config["f_energy"] = args.f_energy
    torch.cuda.synchronize()
    log("timing")
    ms, stage, wall, diag_step = timed_steps(step, torch, args.steps, args.warmup)
    res = base_result(args, step.new_tokens / (ms * 1e-3), ms, "f32" if w.dtype == "f32" else "bf16", config)
    res["roofline"] = roofline(step, stage["attention"])
    if args.workload == "480p":
        res["roofline"]["traffic"] = attention_traffic()
    res["stages_ms"] = {k: round(v, 4) for k, v in stage.items()}
    if isinstance(step, Stream):
        # the overlapped step against the same calls made one after another on one
        # stream: the attention output must be bit-identical
        out = step.run()
        step.join()
        torch.cuda.synchronize()
        dsegs = qwm.segment_array(step.all_segs())
        total = dsegs.total
        ref, _, _ = qwm.attention(step.Q[step.sl_new], dsegs)
        torch.cuda.synchronize()
        res["step_check_max_abs_diff"] = float((out - ref).abs().max().item())
        res["keys_step"] = {"token_heads": step.chunk * step.H,
                            "ms": round(stage["keys"], 4)}
        res["keys_bulk"] = keys_bulk(qwm, torch, step.K[: (step.nch - 1) * step.chunk], step.prev[0], step.st)
        if not args.no_decode_ab:
            res["decode_ab"] = decode_ab(qwm, torch, step, stage["attention"])
            res["keys_m_sweep"] = keys_m_sweep(qwm, torch, step.K[: (step.nch - 1) * step.chunk], step.prev[0],
                                               step.st)
            res["prq_codec"] = prq_codec(qwm, torch, step.K[step.sl_new])
            res["keys_full_matrix"] = keys_full_matrix(qwm, torch, step.K[step.sl_new], step.prev[0], step.st)
            res["keys_keep_test"] = keys_keep_test(qwm, torch, step.K[: (step.nch - 1) * step.chunk], step.prev[0],
                                                   step.st)
    else:
        res["keys_bulk"] = keys_bulk(qwm, torch, step.K, step.Ck, step.st)
    res["wall_s_timed"] = round(wall, 3)
    res["exact_fallbacks_per_step"] = int(diag_step[1])
    res["nonfinite_rows_per_step"] = int(diag_step[0])
    res["eig_iterations"] = step.st.iters.tolist()
    if args.workload == "480p" and not args.no_cpu_baseline:
        log("timing the CPU oracle sample")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_queries)
    return res


def run_rollout(args, qwm, torch, w):
    """Causal rollout for every ablation: tokens/s and the token-shift rate
    (fraction of (head, Query) pairs whose top-1 key under the quantized cache
    differs from the top-1 over the bf16 keys)."""
    import numpy as np
    dev = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()
    Kd, Vd, Qd = dev(w.K), dev(w.V), dev(w.Q)
    H, T, nch = w.H, w.chunk, w.n_chunks
    names = {0: "nearest", 1: "qsac", 2: "psac", 3: "qsac+psac"}
    refs = []
    for t in range(nch):
        sl = w.chunk_slice(t)
        refs.append(qwm.reference_top1(Qd[sl], Kd[: sl.stop]))
    torch.cuda.synchronize()
    out = {}
    for flags in (0, 1, 2, 3):
        for _ in range(2):                        # the first pass warms up, the second is timed
            st = qwm.QueryStats(H)
            segs, prev, tops = [], None, []
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for t in range(nch):
                sl = w.chunk_slice(t)
                K, V = Kd[sl], Vd[sl]
                if prev is None:
                    Ck = qwm.build_centroids(K, 10, seed=1)
                    Cv = qwm.build_centroids(V, 10, seed=2)
                    U = None
                    kp = qwm.quantize_keys(K, Ck, None, None, M=8, flags=flags)
                else:
                    Ck = qwm.build_centroids(K, 3, init=prev[0])
                    Cv = qwm.build_centroids(V, 3, init=prev[1])
                    U = st.U.clone() if flags & 2 else None
                    kp = qwm.quantize_keys(K, Ck, st.w if flags & 1 else None, U, M=8, flags=flags)
                vp = qwm.quantize_values(V, Cv)
                segs.append((kp, vp, Ck, Cv, U))
                dsegs = qwm.segment_array(segs)
                total = dsegs.total
                _, _, top1 = qwm.attention(Qd[sl], dsegs, want_top1=True)
                tops.append(top1)
                qwm.update_query_stats(Qd[sl], st, compute_basis=True)   # causal: feeds the next chunks
                prev = (Ck, Cv)
            torch.cuda.synchronize()
            secs = time.perf_counter() - t0
        rates = [float((tops[t] != refs[t]).float().mean().item()) for t in range(nch)]
        out[names[flags]] = {"tokens_per_s": round(nch * T / secs, 1), "seconds": round(secs, 4),
                             "shift_rate": round(float(np.mean(rates[1:])), 5),
                             "shift_rate_cold_start": round(rates[0], 5)}
        log(f"  {names[flags]}: {out[names[flags]]}")
    config = {"workload": f"rollout: H={H}, d=128, {nch} chunks x {T:,} tokens, causal statistics, 10 seeded + "
                          f"3 warm Lloyd iterations per chunk, attention of each chunk's Queries over the cache so far",
              "heads": H, "chunk_tokens": T, "chunks": nch}
    best = out["qsac+psac"]
    res = base_result(args, best["tokens_per_s"], best["seconds"] * 1e3 / nch, "bf16", config)
    res["steps"], res["warmup"] = nch, 1
    res["ablations"] = out
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU path is not "
              f"part of this build", file=sys.stderr)
        sys.exit(2)
    pool = None
    if args.workload == "depth" and not args.no_cpu_baseline:
        pool = start_cpu_pool()          # before anything touches the GPU
    import torch
    import bit_kv_cache_head_amd as qwm
    import datagen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(torch)
    if args.workload == "depth":
        res = run_depth(args, qwm, torch, datagen, pool)
    else:
        log(f"generating the {args.workload} workload")
        w = datagen.make_workload(args.workload, f_energy=args.f_energy)
        if args.workload == "rollout":
            res = run_rollout(args, qwm, torch, w)
        else:
            res = run_stream_or_pass(args, qwm, torch, w)
    if pool is not None:
        pool[0].close()
        pool[0].join()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
