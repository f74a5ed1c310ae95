"""Seeded synthetic Key/Value/Query streams shaped like a video world model's KV cache.

This module is shared by the CPU oracle and by the GPU tests/bench.  It holds
only the synthetic *input distribution*; none of the quantization method's
arithmetic lives here.

What it imitates (QuantWM, arXiv 2609.26425 v2):
  * Keys/Values cluster strongly (the centroid-residual representation of the
    preliminaries section, and the 256-centroid setting of the experimental
    setup), and clusters drift slowly from frame to frame.
  * Query energy is concentrated: the top-8 eigen-directions of the Query
    second moment hold 60-71 % of the energy (Sec. 4.2; Fig. 4 and Fig. 8).
  * Shapes follow the 480p / 720p, 93-frame setting: 24 latent frames of
    30x52 = 1,560 or 45x80 = 3,600 tokens, head dim 128 (Sec. 5.1, Fig. 6).

Recipe (per layer, head and tensor):
  K/V:  sigma_c = exp(U(ln 0.25, ln 4)) per channel; frame-0 cluster means
        mu0[j, c] = sigma_c * N(0, 1) for j < 256; every later frame adds
        N(0, drift^2) to every mean; each token picks a cluster uniformly and
        adds noise * N(0, I).
  Q:    Sigma = U diag(lam) U^T with U a Haar-random orthogonal matrix and
        lam_i proportional to rho^i (trace = d); rho is chosen so that the top-8
        share of the trace equals the requested fraction f.
Streams are independent: each (config, layer, head, stream) has its own
numpy PCG64 generator seeded from SeedSequence([seed, cfg, layer, head, stream]).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

D_HEAD = 128
N_CLUSTERS = 256
FRAME_480P = 30 * 52      # 1,560 tokens per latent frame
FRAME_720P = 45 * 80      # 3,600 tokens per latent frame

_STREAM_K, _STREAM_V, _STREAM_Q = 1, 2, 3


def rng_for(seed: int, cfg: int, layer: int, head: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, layer, head, stream])))


def rho_for_energy(f: float, r: int = 8, d: int = D_HEAD) -> float:
    """Decay rate rho with (1 - rho^r) / (1 - rho^d) = f (geometric spectrum)."""
    if not (r / d < f < 1.0):
        raise ValueError("energy fraction out of range")
    lo, hi = 1e-9, 1.0 - 1e-12
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        val = (1.0 - mid ** r) / (1.0 - mid ** d)
        if val > f:       # too concentrated -> larger rho
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def query_spectrum(f: float, d: int = D_HEAD) -> np.ndarray:
    rho = rho_for_energy(f, 8, d)
    lam = rho ** np.arange(d, dtype=np.float64)
    return lam * (d / lam.sum())


def haar_orthogonal(rng: np.random.Generator, d: int = D_HEAD) -> np.ndarray:
    g = rng.standard_normal((d, d))
    qm, rm = np.linalg.qr(g)
    return qm * np.sign(np.diag(rm))[None, :]


def cluster_stream(rng: np.random.Generator, n_tokens: int, frame_tokens: int, *,
                   d: int = D_HEAD, n_clusters: int = N_CLUSTERS,
                   drift: float = 0.05, noise: float = 0.1) -> np.ndarray:
    """[n_tokens, d] float64 tokens from drifting Gaussian clusters."""
    sigma = np.exp(rng.uniform(math.log(0.25), math.log(4.0), size=d))
    means = sigma[None, :] * rng.standard_normal((n_clusters, d))
    out = np.empty((n_tokens, d), dtype=np.float64)
    t = 0
    frame = 0
    while t < n_tokens:
        if frame > 0:
            means = means + drift * rng.standard_normal((n_clusters, d))
        m = min(frame_tokens, n_tokens - t)
        assign = rng.integers(0, n_clusters, size=m)
        out[t:t + m] = means[assign] + noise * rng.standard_normal((m, d))
        t += m
        frame += 1
    return out


def query_stream(rng: np.random.Generator, n_tokens: int, f: float, d: int = D_HEAD) -> np.ndarray:
    """[n_tokens, d] float64 queries ~ N(0, Sigma) with top-8 energy fraction f."""
    u = haar_orthogonal(rng, d)
    lam = query_spectrum(f, d)
    z = rng.standard_normal((n_tokens, d))
    return (z * np.sqrt(lam)[None, :]) @ u.T


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array whose values are x rounded to bfloat16 (round to nearest even).

    Input preparation only: the generated caches are handed over as bf16,
    like a model's activations.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits(x_bf16_valued: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of a float32 array that already holds bf16 values."""
    a = np.ascontiguousarray(x_bf16_valued, dtype=np.float32).view(np.uint32)
    if np.any(a & 0xFFFF):
        raise ValueError("array is not bf16-valued")
    return (a >> 16).astype(np.uint16)


@dataclass
class Workload:
    """One synthetic workload.  Arrays are float32 [T, H, d] (bf16-valued unless dtype == 'f32')."""
    name: str
    dtype: str                 # 'bf16' or 'f32'
    chunk: int                 # tokens per chunk (frame)
    n_chunks: int
    heads: list
    layer: int
    f_energy: float
    K: np.ndarray = field(repr=False)
    V: np.ndarray = field(repr=False)
    Q: np.ndarray = field(repr=False)

    @property
    def H(self) -> int:
        return len(self.heads)

    @property
    def T(self) -> int:
        return self.K.shape[0]

    def chunk_slice(self, t: int) -> slice:
        return slice(t * self.chunk, min((t + 1) * self.chunk, self.T))


# name -> (cfg id, H, dtype, tokens per chunk, chunks, queries, energy fraction)
CONFIGS = {
    "tiny":   (1, 1, "f32", 4096, 1, 512, 0.65),
    "480p":   (2, 12, "bf16", FRAME_480P, 25, None, 0.65),
    "720p":   (3, 40, "bf16", FRAME_720P, 25, None, 0.60),
    "depth":  (4, 40, "bf16", 28000, 1, 1560, 0.65),
    "rollout": (5, 24, "bf16", FRAME_480P, 40, None, 0.65),
}


def make_workload(name: str, *, seed: int = 0, layer: int = 0, heads=None, n_chunks=None,
                  chunk=None, n_queries=None, f_energy=None) -> Workload:
    """Generate a workload.  `heads`, `n_chunks`, `chunk` and `n_queries` allow
    smaller slices of the same distributions (a head's streams do not depend on
    which other heads are generated)."""
    cfg_id, H, dtype, tpc, nch, nq, f = CONFIGS[name]
    heads = list(range(H)) if heads is None else list(heads)
    tpc = tpc if chunk is None else chunk
    nch = nch if n_chunks is None else n_chunks
    f = f if f_energy is None else f_energy
    T = tpc * nch
    # one-shot configs: fixed query count; streaming configs: one query per token
    nq = (T if nq is None else nq) if n_queries is None else n_queries
    # frames: tiny = a single frame without drift; depth = 1,560-token frames
    frame = {"tiny": T, "depth": FRAME_480P}.get(name, tpc)
    Hn = len(heads)
    K = np.empty((T, Hn, D_HEAD), np.float32)
    V = np.empty((T, Hn, D_HEAD), np.float32)
    Q = np.empty((nq, Hn, D_HEAD), np.float32)
    for i, h in enumerate(heads):
        K[:, i] = cluster_stream(rng_for(seed, cfg_id, layer, h, _STREAM_K), T, frame)
        V[:, i] = cluster_stream(rng_for(seed, cfg_id, layer, h, _STREAM_V), T, frame)
        Q[:, i] = query_stream(rng_for(seed, cfg_id, layer, h, _STREAM_Q), nq, f)
    if dtype == "bf16":
        K, V, Q = round_to_bf16(K), round_to_bf16(V), round_to_bf16(Q)
    return Workload(name=name, dtype=dtype, chunk=tpc, n_chunks=nch, heads=heads, layer=layer,
                    f_energy=f, K=K, V=V, Q=Q)


# ---------------------------------------------------------------------------
# The same recipe drawn on the GPU.  The full-depth cache (40 layers x 40 heads
# x 28,000 tokens, about 21 GiB of bf16 K and V) is too large to draw with the
# numpy streams above in a benchmark's time, so its layers are drawn on the
# device by torch's Philox generator: same distributions (cluster means,
# per-frame drift, uniform cluster choice, noise; Haar basis and geometric
# Query spectrum), different random numbers from the numpy streams.  One
# generator per (config, layer, stream) draws all heads of the layer at once.
# ---------------------------------------------------------------------------
def _torch_seed(seed: int, cfg: int, layer: int, stream: int) -> int:
    s = np.random.SeedSequence([seed, cfg, layer, 1000 + stream]).generate_state(2, dtype=np.uint32)
    return int(s[0]) | (int(s[1] & 0x7FFFFFFF) << 32)


def _device_clusters(g, H: int, n_tokens: int, frame_tokens: int, device, drift: float = 0.05,
                     noise: float = 0.1):
    """[n_tokens, H, d] bf16 tokens from drifting Gaussian clusters (all heads)."""
    import torch
    f32 = torch.float32
    sigma = torch.exp(torch.empty(H, 1, D_HEAD, dtype=f32, device=device)
                      .uniform_(math.log(0.25), math.log(4.0), generator=g))
    means = sigma * torch.randn(H, N_CLUSTERS, D_HEAD, dtype=f32, device=device, generator=g)
    out = torch.empty(n_tokens, H, D_HEAD, dtype=torch.bfloat16, device=device)
    t = 0
    frame = 0
    while t < n_tokens:
        if frame > 0:
            means = means + drift * torch.randn(H, N_CLUSTERS, D_HEAD, dtype=f32, device=device, generator=g)
        m = min(frame_tokens, n_tokens - t)
        assign = torch.randint(0, N_CLUSTERS, (H, m), device=device, generator=g)
        x = torch.gather(means, 1, assign[:, :, None].expand(H, m, D_HEAD))
        x = x + noise * torch.randn(H, m, D_HEAD, dtype=f32, device=device, generator=g)
        out[t:t + m] = x.transpose(0, 1).to(torch.bfloat16)
        t += m
        frame += 1
    return out


def device_layer(name: str, layer: int, *, seed: int = 0, f_energy=None, device="cuda", heads=None,
                 n_tokens=None, n_queries=None):
    """(K, V [T, H, d], Q [nq, H, d]) bf16 device tensors of one layer of a
    workload, drawn on the device (see above).  heads / n_tokens / n_queries
    shrink the draw (a smaller draw is not a slice of the full one)."""
    import torch
    cfg_id, H, dtype, tpc, nch, nq, f = CONFIGS[name]
    if dtype != "bf16":
        raise ValueError("device_layer draws the bf16 workloads")
    f = f if f_energy is None else f_energy
    T = tpc * nch if n_tokens is None else n_tokens
    H = H if heads is None else heads
    nq = (T if nq is None else nq) if n_queries is None else n_queries
    frame = {"depth": FRAME_480P}.get(name, tpc)
    gens = {}
    for stream in (_STREAM_K, _STREAM_V, _STREAM_Q):
        g = torch.Generator(device=device)
        g.manual_seed(_torch_seed(seed, cfg_id, layer, stream))
        gens[stream] = g
    K = _device_clusters(gens[_STREAM_K], H, T, frame, device)
    V = _device_clusters(gens[_STREAM_V], H, T, frame, device)
    # Haar bases (QR of a Gaussian with the sign of R's diagonal fixed), fp64 on the host
    gq = torch.Generator()
    gq.manual_seed(_torch_seed(seed, cfg_id, layer, _STREAM_Q + 10))
    G = torch.randn(H, D_HEAD, D_HEAD, dtype=torch.float64, generator=gq)
    qm, rm = torch.linalg.qr(G)
    U = (qm * torch.sign(torch.diagonal(rm, dim1=1, dim2=2))[:, None, :]).to(torch.float32).to(device)
    lam = torch.from_numpy(query_spectrum(f)).to(torch.float32).to(device)
    z = torch.randn(H, nq, D_HEAD, dtype=torch.float32, device=device, generator=gens[_STREAM_Q])
    q = torch.matmul(z * torch.sqrt(lam)[None, None, :], U.transpose(1, 2).contiguous())   # [H, nq, d]
    Q = q.transpose(0, 1).contiguous().to(torch.bfloat16)
    return K, V, Q
