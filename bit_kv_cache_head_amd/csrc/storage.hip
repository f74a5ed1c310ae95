// Refinements of the stored format: two-level group scales (rainbus digest,
// method step (3): group scales in INT8 under an FP16 second level), the keep
// test of the PSAC coefficients with the full Query second moment (method
// step (4); the method section's objective e^T M e), and the per-chunk choice
// of the smaller of a dense and a sparse coefficient layout (QuantWM v2
// App. D.1).  Each works on a chunk the quantizers have already stored.
#include "common.hpp"
#include "psac.hpp"

namespace qwm {

__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// ---------------------------------------------------------------------------
// Two-level scales.  Per (chunk, head, group g) the second-level scale s2_g is
// the smallest power of two p >= 2^-24 with 255 p >= the largest stored fp16
// step of the group; each token's INT8 code is q = min(ceil(s / p), floor(65504 / p))
// and its effective step q p, an exact fp16 value.  Grid H, 256 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scale2_kernel(const uint16_t* __restrict__ scale, int64_t T,
                                                     uint16_t* __restrict__ scale2) {
  const int h = blockIdx.x, tid = threadIdx.x;
  float m0 = 0.f, m1 = 0.f;
  const uint32_t* sh = reinterpret_cast<const uint32_t*>(scale + (int64_t)h * T * 2);
  for (int64_t t = tid; t < T; t += 256) {
    const uint32_t v = sh[t];
    m0 = fmaxf(m0, f16_bits_to_f32(v & 0xFFFFu));
    m1 = fmaxf(m1, f16_bits_to_f32(v >> 16));
  }
  for (int o = 32; o > 0; o >>= 1) {
    m0 = fmaxf(m0, __shfl_xor(m0, o, 64));
    m1 = fmaxf(m1, __shfl_xor(m1, o, 64));
  }
  __shared__ float red[2][4];
  if ((tid & 63) == 0) { red[0][tid >> 6] = m0; red[1][tid >> 6] = m1; }
  __syncthreads();
  if (tid < 2) {
    float m = fmaxf(fmaxf(red[tid][0], red[tid][1]), fmaxf(red[tid][2], red[tid][3]));
    uint32_t bits = 0u;
    if (m > 0.f) {
      int e = -24;
      while (255.0f * ldexpf(1.0f, e) < m) ++e;   // exact: powers of two times 255
      bits = f32_to_f16_bits(ldexpf(1.0f, e));
    }
    scale2[h * 2 + tid] = (uint16_t)bits;
  }
}

struct TwoLevelArgs {
  const void* x; int32_t dtype; int64_t T; int64_t st, sh; int32_t H;
  const uint16_t* mu; const float* w; const uint16_t* U; uint32_t flags; int32_t r;
  const uint8_t* idx; const uint16_t* scale; const uint16_t* scale2;
  uint8_t* codes; uint8_t* zeros; int64_t zstride; uint8_t* scale_q;
  int8_t* cq; uint16_t* cscale; qwm_diag* diag;
};

// Re-encodes every token with its effective step (one wave per token, lane l
// holds channels 2 l and 2 l + 1, groups split at lane 32): codes,
// zero-points, INT8 step codes, and for keys the PSAC coefficients of the new
// error E = x - (mu + r_hat) in fp64.  RR: rank (0 for values).
template <int RR>
__global__ __launch_bounds__(256) void two_level_kernel(TwoLevelArgs a) {
  const int lane = threadIdx.x & 63, g = lane >> 5;
  const int64_t id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (id >= (int64_t)a.H * a.T) return;
  const int h = (int)(id / a.T);
  const int64_t tok = id % a.T, base = id;
  const int64_t rowoff = (int64_t)h * a.sh + tok * a.st + 2 * lane;
  float x0, x1;
  if (a.dtype == QWM_F32) {
    const float* xr = static_cast<const float*>(a.x) + rowoff;
    x0 = xr[0]; x1 = xr[1];
  } else {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.x) + rowoff);
    x0 = bf16_bits_to_f32(v & 0xFFFFu); x1 = bf16_bits_to_f32(v >> 16);
  }
  const bool bad = __any(!(__builtin_isfinite(x0) && __builtin_isfinite(x1)));
  const uint32_t mw = *reinterpret_cast<const uint32_t*>(a.mu + ((int64_t)h * NC + a.idx[base]) * D + 2 * lane);
  const float m0 = bf16_bits_to_f32(mw & 0xFFFFu), m1 = bf16_bits_to_f32(mw >> 16);
  const float r0 = x0 - m0, r1 = x1 - m1;                       // fl32 residual
  float lo = fminf(0.f, fminf(r0, r1)), hi = fmaxf(0.f, fmaxf(r0, r1));
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, o, 64));
    hi = fmaxf(hi, __shfl_xor(hi, o, 64));
  }
  (void)hi;
  const float s = f16_bits_to_f32(a.scale[base * 2 + g]);
  const float p = f16_bits_to_f32(a.scale2[h * 2 + g]);
  int q = 0;
  if (!bad && p > 0.f) {
    q = (int)ceilf(s / p);                                      // exact: p is a power of two
    const int qmax = (int)floorf(65504.0f / p);
    q = q < qmax ? q : qmax;
  }
  const float st = (float)q * p;                                // exact fp16 value
  int z = 0, c0 = 0, c1 = 0;
  if (st > 0.f) {
    z = rne_quot(-lo, st);
    z = z < 0 ? 0 : (z > 3 ? 3 : z);
    c0 = rne_quot(r0, st) + z; c0 = c0 < 0 ? 0 : (c0 > 3 ? 3 : c0);
    c1 = rne_quot(r1, st) + z; c1 = c1 < 0 ? 0 : (c1 > 3 ? 3 : c1);
  }
  // byte b = channels 4b .. 4b + 3 = lanes 2b, 2b + 1
  const uint32_t pair = (uint32_t)c0 | ((uint32_t)c1 << 2);
  const uint32_t other = __shfl_xor(pair, 1, 64);
  if ((lane & 1) == 0) a.codes[base * 32 + (lane >> 1)] = (uint8_t)(pair | (other << 4));
  const int z1 = __shfl(z, 32, 64);
  if ((lane & 31) == 0) a.scale_q[base * 2 + g] = (uint8_t)q;
  if (lane == 0) {
    const uint32_t nib = (uint32_t)(z | (z1 << 2));
    uint8_t* zb = a.zeros + (int64_t)h * a.zstride + (tok >> 1);
    uint32_t* word = reinterpret_cast<uint32_t*>(reinterpret_cast<uintptr_t>(zb) & ~(uintptr_t)3);
    const int sh = 8 * (int)(reinterpret_cast<uintptr_t>(zb) & 3) + 4 * (int)(tok & 1);
    atomicAnd(word, ~(0xFu << sh));      // the neighbour token owns the other nibble
    atomicOr(word, nib << sh);
  }
  if constexpr (RR > 0) {
    int8_t* cq = a.cq + base * RR;
    if (bad || !(a.flags & QWM_PSAC) || a.U == nullptr) {
      if (lane < RR) cq[lane] = 0;
      if (lane == 0) a.cscale[base] = 0;
      return;
    }
    const double e0 = (double)x0 - ((double)m0 + (double)st * (double)(c0 - z));
    const double e1 = (double)x1 - ((double)m1 + (double)st * (double)(c1 - z));
    const bool wts = (a.flags & QWM_QSAC) && a.w != nullptr;
    psac_token<RR>(e0, e1, lane, a.U + (int64_t)h * D * RR, (a.flags & QWM_PSAC_KEEP) != 0,
                   wts ? (double)a.w[h * D + 2 * lane] : 1.0, wts ? (double)a.w[h * D + 2 * lane + 1] : 1.0,
                   cq, a.cscale + base, a.diag);
  }
}

// ---------------------------------------------------------------------------
// Keep test with the full second moment: a key keeps its coefficients iff the
// compensation D = U c_hat lowers e^T S e, i.e. iff
//   D^T S (D - 2 e) = c_hat^T (U^T S U) c_hat - 2 c_hat^T (U^T S e) < 0
// (S / n scaled by n > 0 decides the same).  keepfull_prep_kernel forms
// P = U^T S (r x 128) and A = P U (r x r) per head in fp64; keepfull_kernel
// recomputes each key's error from its stored codes and step and tests it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void keepfull_prep_kernel(const double* __restrict__ S, const uint16_t* __restrict__ U,
                                                            int32_t r, double* __restrict__ P, double* __restrict__ A) {
  const int h = blockIdx.x, tid = threadIdx.x;
  const double* Sh = S + (int64_t)h * D * D;
  const uint16_t* Uh = U + (int64_t)h * D * r;
  double* Ph = P + (int64_t)h * r * D;
  for (int e = tid; e < r * D; e += 256) {
    const int i = e / D, c = e % D;
    double v = 0.0;
    for (int k = 0; k < D; ++k) v = fma((double)bf16_bits_to_f32(Uh[k * r + i]), Sh[k * D + c], v);
    Ph[e] = v;
  }
  __syncthreads();
  for (int e = tid; e < r * r; e += 256) {
    const int i = e / r, j = e % r;
    double v = 0.0;
    for (int c = 0; c < D; ++c) v = fma(Ph[i * D + c], (double)bf16_bits_to_f32(Uh[c * r + j]), v);
    A[(int64_t)h * r * r + e] = v;
  }
}

struct KeepFullArgs {
  const void* x; int32_t dtype; int64_t T; int64_t st, sh; int32_t H;
  const uint16_t* mu; const int64_t* n; int32_t r;
  const uint8_t* idx; const uint8_t* codes; const uint16_t* scale; const uint8_t* scale_q; const uint16_t* scale2;
  const uint8_t* zeros; int64_t zstride;
  int8_t* cq; uint16_t* cscale; const double* P; const double* A;
};

template <int RR>
__global__ __launch_bounds__(256) void keepfull_kernel(KeepFullArgs a) {
  const int lane = threadIdx.x & 63, g = lane >> 5;
  const int64_t id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (id >= (int64_t)a.H * a.T) return;
  const int h = (int)(id / a.T);
  const int64_t tok = id % a.T, base = id;
  const uint16_t csb = a.cscale[base];
  if (csb == 0 || a.n[h] <= 0) return;            // nothing kept, or no statistics
  const int64_t rowoff = (int64_t)h * a.sh + tok * a.st + 2 * lane;
  double x0, x1;
  if (a.dtype == QWM_F32) {
    const float* xr = static_cast<const float*>(a.x) + rowoff;
    x0 = xr[0]; x1 = xr[1];
  } else {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.x) + rowoff);
    x0 = bf16_bits_to_f32(v & 0xFFFFu); x1 = bf16_bits_to_f32(v >> 16);
  }
  const uint32_t mw = *reinterpret_cast<const uint32_t*>(a.mu + ((int64_t)h * NC + a.idx[base]) * D + 2 * lane);
  const double m0 = bf16_bits_to_f32(mw & 0xFFFFu), m1 = bf16_bits_to_f32(mw >> 16);
  const uint32_t cb = a.codes[base * 32 + (lane >> 1)] >> (4 * (lane & 1));
  const int q0 = (int)(cb & 3u), q1 = (int)((cb >> 2) & 3u);
  const double stp = a.scale2 ? (double)a.scale_q[base * 2 + g] * (double)f16_bits_to_f32(a.scale2[h * 2 + g])
                              : (double)f16_bits_to_f32(a.scale[base * 2 + g]);
  const int z = (a.zeros[(int64_t)h * a.zstride + (tok >> 1)] >> (4 * (int)(tok & 1) + 2 * g)) & 3;
  const double e0 = x0 - (m0 + stp * (double)(q0 - z));
  const double e1 = x1 - (m1 + stp * (double)(q1 - z));
  const double* Ph = a.P + (int64_t)h * RR * D;
  const double* Ah = a.A + (int64_t)h * RR * RR;
  const double cs = (double)f16_bits_to_f32(csb);
  double ch[RR], y[RR];
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    ch[i] = cs * (double)a.cq[base * RR + i];
    y[i] = wave_sum_d(Ph[i * D + 2 * lane] * e0 + Ph[i * D + 2 * lane + 1] * e1);   // (U^T S e)_i
  }
  double delta = 0.0;
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    double t = 0.0;
#pragma unroll
    for (int j = 0; j < RR; ++j) t = fma(Ah[i * RR + j], ch[j], t);
    delta = fma(ch[i], t - 2.0 * y[i], delta);
  }
  if (!(delta < 0.0)) {
    if (lane < RR) a.cq[base * RR + lane] = 0;
    if (lane == 0) a.cscale[base] = 0;
  }
}

// ---------------------------------------------------------------------------
// Dense / sparse coefficient layout, one block of 1,024 threads per head: the
// kept keys (nonzero coefficient scale) are counted 64 at a time by ballots;
// the smaller layout takes its bytes from the arena with one atomic add and
// its place goes into the head's directory entry.  Sparse: a bitmap of 64-key
// words, the kept count before each word, the kept rows and scales in key
// order; dense: every row and scale.  Sections start on 16-byte boundaries.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int64_t al16(int64_t n) { return (n + 15) & ~(int64_t)15; }
__host__ __device__ __forceinline__ int64_t dense_layout_bytes(int64_t T, int r) { return al16(T * r) + al16(T * 2); }
__host__ __device__ __forceinline__ int64_t sparse_layout_bytes(int64_t T, int64_t count, int r) {
  const int64_t nw = (T + 63) / 64;
  return al16(nw * 8) + al16(nw * 4) + al16(count * r) + al16(count * 2);
}

struct CompactArgs {
  const int8_t* c; const uint16_t* cs; int64_t T; int32_t H, r;
  qwm_cdir* dir; uint8_t* arena; int64_t arena_bytes; unsigned long long* used; qwm_diag* diag;
};

__global__ __launch_bounds__(1024) void compact_kernel(CompactArgs a) {
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t T = a.T, nw = (T + 63) / 64;
  const uint16_t* csh = a.cs + (int64_t)h * T;
  const int8_t* ch = a.c + (int64_t)h * T * a.r;
  __shared__ int64_t wcnt[16];
  __shared__ int64_t total_s, base_s;
  __shared__ int layout_s;
  // pass 1: kept keys in all
  int64_t cnt = 0;
  for (int64_t w = wv; w < nw; w += 16) {
    const int64_t t = w * 64 + lane;
    const uint64_t m = __ballot(t < T && csh[t] != 0);
    cnt += __popcll(m);
  }
  if (lane == 0) wcnt[wv] = cnt;
  __syncthreads();
  if (tid == 0) {
    int64_t tot = 0;
    for (int i = 0; i < 16; ++i) tot += wcnt[i];
    const int64_t db = dense_layout_bytes(T, a.r), sb = sparse_layout_bytes(T, tot, a.r);
    const int sparse = sb < db ? 1 : 0;
    const int64_t bytes = sparse ? sb : db;
    const int64_t base = (int64_t)atomicAdd(a.used, (unsigned long long)bytes);
    const bool fits = base + bytes <= a.arena_bytes;
    layout_s = fits ? sparse : -1;
    total_s = tot;
    base_s = base;
    a.dir[h].layout = fits ? sparse : QWM_LAYOUT_OVERFLOW;
    a.dir[h].count = (int32_t)tot;
    a.dir[h].offset = base;
    if (!fits && a.diag) atomicAdd((unsigned long long*)&a.diag->layout_overflows, 1ull);
  }
  __syncthreads();
  const int layout = layout_s;
  if (layout < 0) return;
  uint8_t* out = a.arena + base_s;
  const int r = a.r;
  if (layout == 0) {
    // dense: rows, then scales
    for (int64_t i = tid; i < T * r / 8; i += 1024)
      reinterpret_cast<uint2*>(out)[i] = reinterpret_cast<const uint2*>(ch)[i];
    uint16_t* cso = reinterpret_cast<uint16_t*>(out + al16(T * r));
    for (int64_t t = tid; t < T; t += 1024) cso[t] = csh[t];
    return;
  }
  uint64_t* bm = reinterpret_cast<uint64_t*>(out);
  uint32_t* pre = reinterpret_cast<uint32_t*>(out + al16(nw * 8));
  int8_t* co = reinterpret_cast<int8_t*>(out + al16(nw * 8) + al16(nw * 4));
  uint16_t* cso = reinterpret_cast<uint16_t*>(out + al16(nw * 8) + al16(nw * 4) + al16(total_s * r));
  // pass 2: 16 words per round, in order; the kept count before each word is
  // the running carry plus the counts of the round's lower words
  __shared__ int32_t rc[16];
  int64_t carry = 0;
  for (int64_t w0 = 0; w0 < nw; w0 += 16) {
    const int64_t w = w0 + wv;
    const int64_t t = w * 64 + lane;
    const bool kept = w < nw && t < T && csh[t] != 0;
    const uint64_t m = __ballot(kept);
    if (lane == 0) rc[wv] = __popcll(m);
    __syncthreads();
    int64_t before = carry;
    for (int i = 0; i < wv; ++i) before += rc[i];
    if (w < nw) {
      if (lane == 0) { bm[w] = m; pre[w] = (uint32_t)before; }
      if (kept) {
        const int64_t e = before + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const int8_t* src = ch + t * r;
        int8_t* dst = co + e * r;
        for (int k = 0; k < r; k += 8) *reinterpret_cast<uint2*>(dst + k) = *reinterpret_cast<const uint2*>(src + k);
        cso[e] = csh[t];
      }
    }
    int64_t round = 0;
    for (int i = 0; i < 16; ++i) round += rc[i];
    __syncthreads();
    carry += round;
  }
}

}  // namespace qwm

namespace qwm_host {
using namespace qwm;

size_t keepfull_ws_bytes(int32_t H, int32_t r) {
  return (size_t)((H * (int64_t)r * D * 8 + 255) & ~(int64_t)255) + (size_t)H * r * r * 8;
}

int64_t coefficient_layout_bytes(int32_t layout, int64_t T, int64_t count, int32_t r) {
  return layout == QWM_LAYOUT_SPARSE ? sparse_layout_bytes(T, count, r) : dense_layout_bytes(T, r);
}

qwm_status launch_two_level(const qwm_tokens* x, const uint16_t* centroids, const float* w, const uint16_t* U,
                            uint32_t flags, const qwm_packed* io, bool keys, uint8_t* scale_q, uint16_t* scale2,
                            qwm_diag* diag, hipStream_t stream) {
  hipLaunchKernelGGL(scale2_kernel, dim3(x->H), dim3(256), 0, stream, io->scale, x->T, scale2);
  qwm_status s = check_launch("second-level scales");
  if (s != QWM_OK) return s;
  TwoLevelArgs a{};
  a.x = x->ptr; a.dtype = x->dtype; a.T = x->T; a.st = x->stride_t; a.sh = x->stride_h; a.H = x->H;
  a.mu = centroids; a.w = (flags & QWM_QSAC) ? w : nullptr; a.U = U; a.flags = flags; a.r = io->r;
  a.idx = io->idx; a.scale = io->scale; a.scale2 = scale2;
  a.codes = io->codes; a.zeros = io->zeros; a.zstride = zeros_stride(x->T); a.scale_q = scale_q;
  a.cq = io->c; a.cscale = io->c_scale; a.diag = diag;
  const dim3 grid((unsigned)(((int64_t)x->H * x->T + 3) / 4));
  if (!keys) hipLaunchKernelGGL(two_level_kernel<0>, grid, dim3(256), 0, stream, a);
  else if (io->r == 8) hipLaunchKernelGGL(two_level_kernel<8>, grid, dim3(256), 0, stream, a);
  else if (io->r == 16) hipLaunchKernelGGL(two_level_kernel<16>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(two_level_kernel<32>, grid, dim3(256), 0, stream, a);
  return check_launch("two-level re-encoding");
}

qwm_status launch_keep_full(const qwm_tokens* k, const uint16_t* centroids, const double* S, const int64_t* n,
                            const uint16_t* U, const qwm_packed* io, const uint8_t* scale_q, const uint16_t* scale2,
                            void* ws, hipStream_t stream) {
  const int r = io->r;
  double* P = static_cast<double*>(ws);
  double* A = reinterpret_cast<double*>(static_cast<char*>(ws) + ((k->H * (int64_t)r * D * 8 + 255) & ~(int64_t)255));
  hipLaunchKernelGGL(keepfull_prep_kernel, dim3(k->H), dim3(256), 0, stream, S, U, r, P, A);
  qwm_status s = check_launch("keep test projections");
  if (s != QWM_OK) return s;
  KeepFullArgs a{};
  a.x = k->ptr; a.dtype = k->dtype; a.T = k->T; a.st = k->stride_t; a.sh = k->stride_h; a.H = k->H;
  a.mu = centroids; a.n = n; a.r = r;
  a.idx = io->idx; a.codes = io->codes; a.scale = io->scale; a.scale_q = scale_q; a.scale2 = scale2;
  a.zeros = io->zeros; a.zstride = zeros_stride(k->T); a.cq = io->c; a.cscale = io->c_scale; a.P = P; a.A = A;
  const dim3 grid((unsigned)(((int64_t)k->H * k->T + 3) / 4));
  if (r == 8) hipLaunchKernelGGL(keepfull_kernel<8>, grid, dim3(256), 0, stream, a);
  else if (r == 16) hipLaunchKernelGGL(keepfull_kernel<16>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(keepfull_kernel<32>, grid, dim3(256), 0, stream, a);
  return check_launch("full-form keep test");
}

qwm_status launch_compact(const qwm_packed* keys, qwm_cdir* dir, uint8_t* arena, int64_t arena_bytes,
                          int64_t* arena_used, qwm_diag* diag, hipStream_t stream) {
  CompactArgs a{};
  a.c = keys->c; a.cs = keys->c_scale; a.T = keys->T; a.H = keys->H; a.r = keys->r;
  a.dir = dir; a.arena = arena; a.arena_bytes = arena_bytes;
  a.used = reinterpret_cast<unsigned long long*>(arena_used); a.diag = diag;
  hipLaunchKernelGGL(compact_kernel, dim3(keys->H), dim3(1024), 0, stream, a);
  return check_launch("coefficient layout");
}

}  // namespace qwm_host
