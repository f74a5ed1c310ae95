// Lloyd iterations with distance bounds and exact integer member sums.
//
// The centroid tables are QVG's k-means tables (QVG summary Sec. 2A; QuantWM
// v2 Sec. 2): every token goes to its nearest centroid, then every centroid
// becomes the bf16 mean of its members.  Two facts make the later iterations
// cheap without changing any result:
//
//  * Distance bounds (the triangle inequality, as in Hamerly's k-means).  A
//    token carries an upper bound u on its distance to its centroid a and a
//    lower bound l on its distance to every other centroid.  When the means
//    move by delta_j, u + delta_a < l - max_{j != a} delta_j proves that a is
//    still the strictly nearest centroid, and the token is not looked at.  All
//    bounds are rounded outward, so a skipped token is one whose exact
//    nearest centroid cannot have changed.
//
//  * Integer member sums.  Channel c of a head is summed in fixed point, in
//    units of 2^(emax_c - P) (emax_c: the largest binary exponent of the
//    channel's values, P = min(62 - bit length of T, 48)).  Every value of the channel
//    is then a whole number of units, unless it is finer than the unit (the
//    head is then flagged and takes the fp64 member-sum path of quantize.hip),
//    and no sum of T values leaves 64 bits.  Integer sums do not depend on the
//    order of the additions, so an iteration adds the tokens that joined a
//    cluster and subtracts those that left, in any order, and holds the exact
//    sum.  The new centroid is bf16(fl64(sum) / n), which equals the plain
//    fp64 mean whenever the fp64 sum is exact.
#include <climits>

#include "lloyd.hpp"

namespace qwm {


__global__ __launch_bounds__(256) void lloyd_fill_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

// frexp exponent of a nonzero finite float (x = m 2^e, 1/2 <= |m| < 1)
__device__ __forceinline__ int frexp_e(float v) { return __builtin_amdgcn_frexp_expf(v); }

// ---------------------------------------------------------------------------
// Exponent ranges.  Grid (H, nb), 256 threads: 16 lanes per row (8 channels
// each), rows of head blockIdx.x strided over the grid's y.  Rows with a
// non-finite channel take no part (the build excludes them).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lloyd_scan_kernel(const void* __restrict__ x, int32_t dtype, int64_t T,
                                                         int64_t st, int64_t sh, int32_t* __restrict__ emax,
                                                         int32_t* __restrict__ emin) {
  __shared__ int32_t smax[D], smin[D];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, l16 = tid & 15, grp = tid >> 4;
  if (tid < D) { smax[tid] = INT_MIN; smin[tid] = INT_MAX; }
  __syncthreads();
  int lmax[8], lmin[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { lmax[i] = INT_MIN; lmin[i] = INT_MAX; }
  // a round covers 4 rows per lane group (loads in flight together); every
  // lane runs the same number of rounds, so the ballots see whole rows
  constexpr int RW = 4;
  const int64_t step = (int64_t)gridDim.y * 16 * RW;
  const int64_t rounds = (T + step - 1) / step;
  for (int64_t rd = 0; rd < rounds; ++rd) {
    float v[RW][8];
    bool live[RW];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
      const int64_t t = rd * step + ((int64_t)blockIdx.y * RW + q) * 16 + grp;
      live[q] = t < T;
      const int64_t tc = live[q] ? t : 0;
      if (dtype == QWM_BF16) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + h * sh + tc * st + 8 * l16);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          v[q][i] = (i & 1) ? __uint_as_float(w[i >> 1] & 0xFFFF0000u) : __uint_as_float(w[i >> 1] << 16);
      } else {
        const float* xr = static_cast<const float*>(x) + h * sh + tc * st + 8 * l16;
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(xr);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(xr + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[q][i] = w0[i]; v[q][4 + i] = w1[i]; }
      }
    }
#pragma unroll
    for (int q = 0; q < RW; ++q) {
      bool ok = true;
#pragma unroll
      for (int i = 0; i < 8; ++i) ok = ok && ((__float_as_uint(v[q][i]) & 0x7F800000u) != 0x7F800000u);
      const uint64_t bm = __ballot(ok);
      const bool row_ok = live[q] && (((bm >> (lane & 48)) & 0xFFFFull) == 0xFFFFull);
      if (row_ok) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (v[q][i] != 0.0f) {
            const int e = frexp_e(v[q][i]);
            lmax[i] = e > lmax[i] ? e : lmax[i];
            lmin[i] = e < lmin[i] ? e : lmin[i];
          }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (lmax[i] != INT_MIN) atomicMax(&smax[8 * l16 + i], lmax[i]);
    if (lmin[i] != INT_MAX) atomicMin(&smin[8 * l16 + i], lmin[i]);
  }
  __syncthreads();
  if (tid < D) {
    if (smax[tid] != INT_MIN) atomicMax(&emax[h * D + tid], smax[tid]);
    if (smin[tid] != INT_MAX) atomicMin(&emin[h * D + tid], smin[tid]);
  }
}

// Per head: flagged when some channel holds a nonzero value finer than the
// fixed-point unit (frexp exponent below emax - P + MB).  Grid H, 128 threads.
__global__ __launch_bounds__(128) void lloyd_flag_kernel(const int32_t* __restrict__ emax,
                                                         const int32_t* __restrict__ emin,
                                                         int32_t* __restrict__ hflag, int32_t P, int32_t MB) {
  const int h = blockIdx.x, c = threadIdx.x;
  const int32_t hi = emax[h * D + c], lo = emin[h * D + c];
  const bool bad = lo != INT_MAX && (int64_t)lo < (int64_t)hi - P + MB;
  const int any = __syncthreads_or(bad);
  if (c == 0) hflag[h] = any ? 1 : 0;
}

// ---------------------------------------------------------------------------
// Recorded changes: one wave per changed token, 2 channels per lane; the row
// is added to its new centroid's sums and taken from its old one's.
// ---------------------------------------------------------------------------
template <int MB>
__global__ __launch_bounds__(256) void lloyd_changes_kernel(const void* __restrict__ x, int64_t T, int64_t st,
                                                            int64_t sh, const int32_t* __restrict__ emax,
                                                            const int32_t* __restrict__ hflag,
                                                            const uint2* __restrict__ chg,
                                                            const int32_t* __restrict__ chg_cnt,
                                                            int64_t* __restrict__ sums, int32_t* __restrict__ cnt,
                                                            int32_t P) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = *chg_cnt;
  for (int i = blockIdx.x * 4 + wv; i < n; i += gridDim.x * 4) {
    const uint2 c = chg[i];
    const int64_t id = c.x;
    const int h = (int)(id / T);
    const int64_t t = id - (int64_t)h * T;
    if (hflag[h]) continue;
    const int old = (int)(c.y & 0xFFu), nw = (int)((c.y >> 8) & 0xFFu);
    uint32_t bits[2];
    if constexpr (MB == 8) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(x) + h * sh + t * st + 2 * lane);
      bits[0] = w & 0xFFFFu; bits[1] = w >> 16;
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const float*>(x) + h * sh + t * st + 2 * lane);
      bits[0] = w.x; bits[1] = w.y;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int ch = 2 * lane + k;
      const int32_t e = emax[h * D + ch];
      const int64_t f = to_fixed<MB>(bits[k], e == INT_MIN ? 0 : P - e);
      if (f != 0) {
        atomicAdd(reinterpret_cast<unsigned long long*>(&sums[((int64_t)h * NC + nw) * D + ch]), (unsigned long long)f);
        atomicAdd(reinterpret_cast<unsigned long long*>(&sums[((int64_t)h * NC + old) * D + ch]), (unsigned long long)(-f));
      }
    }
    if (lane == 0) {
      atomicAdd(&cnt[h * NC + nw], 1);
      atomicSub(&cnt[h * NC + old], 1);
    }
  }
}

// ---------------------------------------------------------------------------
// New means and their moves: one wave per (head, centroid), 2 channels per
// lane.  delta = ||new - old|| (fp64, exact squares of bf16 differences),
// rounded up to fp32.  Flagged heads are left to the fp64 path.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lloyd_finalize_kernel(const int32_t* __restrict__ emax,
                                                             const int32_t* __restrict__ hflag,
                                                             const int64_t* __restrict__ sums,
                                                             const int32_t* __restrict__ cnt,
                                                             float* __restrict__ delta, const uint16_t* cur,
                                                             uint16_t* out, int32_t H, int32_t P) {
  const int lane = threadIdx.x & 63;
  const int unit = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (unit >= H * NC) return;
  const int h = unit / NC;
  if (hflag[h]) return;
  const int32_t n = cnt[unit];
  const uint16_t* src = cur + (int64_t)unit * D + 2 * lane;
  uint16_t* dst = out + (int64_t)unit * D + 2 * lane;
  const uint32_t o0 = src[0], o1 = src[1];
  uint32_t n0 = o0, n1 = o1;
  if (n > 0) {
    const int64_t* s = sums + (int64_t)unit * D + 2 * lane;
    const int32_t e0 = emax[h * D + 2 * lane], e1 = emax[h * D + 2 * lane + 1];
    const double m0 = s[0] == 0 ? 0.0 : ldexp((double)s[0], e0 - P);
    const double m1 = s[1] == 0 ? 0.0 : ldexp((double)s[1], e1 - P);
    n0 = f64_to_bf16_bits(m0 / (double)n);
    n1 = f64_to_bf16_bits(m1 / (double)n);
  }
  // reads of the old row come before the write (cur may be out)
  __builtin_amdgcn_wave_barrier();
  dst[0] = (uint16_t)n0;
  dst[1] = (uint16_t)n1;
  const double d0 = (double)bf16_bits_to_f32(n0) - (double)bf16_bits_to_f32(o0);
  const double d1 = (double)bf16_bits_to_f32(n1) - (double)bf16_bits_to_f32(o1);
  const double d2 = wave_sum_d(d0 * d0 + d1 * d1);
  if (lane == 0) delta[unit] = (float)sqrt(d2) * (1.0f + 1.0f / 1048576.0f);
}

// ---------------------------------------------------------------------------
// Bounds after a mean update.  Grid (H, nb), 256 threads; a block takes
// chunks of 1,024 consecutive tokens (4 per thread, loads issued together).
// The head's largest move delta1 (centroid i1) and second largest delta2
// first; then per token: u += delta_a, l -= (a == i1 ? delta2 : delta1),
// rounded outward; the token is listed for the next assignment unless u < l.
// Listed tokens gather in LDS and take their place in the head's list with
// one atomic per chunk.  Every token of a flagged head is listed; excluded
// rows never are.
// ---------------------------------------------------------------------------
constexpr int LB_CHUNK = 1024;

__global__ __launch_bounds__(256) void lloyd_bounds_kernel(int64_t T, const uint8_t* __restrict__ assign,
                                                           const uint32_t* __restrict__ excl, int64_t excl_words,
                                                           const int32_t* __restrict__ hflag,
                                                           const float* __restrict__ delta, float* __restrict__ ub,
                                                           float* __restrict__ lb, int32_t* __restrict__ wl,
                                                           int32_t* __restrict__ wl_cnt) {
  __shared__ float sd[NC];
  __shared__ float top[3];
  __shared__ int32_t lst[LB_CHUNK];
  __shared__ int32_t nl, gbase;
  const int h = blockIdx.x, tid = threadIdx.x;
  sd[tid] = delta[h * NC + tid];
  __syncthreads();
  if (tid < 64) {
    // (largest, its index, second largest) over four values per lane, then across the wave
    float m1 = -1.0f, m2 = -1.0f;
    int i1 = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float v = sd[tid + 64 * q];
      if (v > m1) { m2 = m1; m1 = v; i1 = tid + 64 * q; }
      else if (v > m2) m2 = v;
    }
    for (int o = 32; o > 0; o >>= 1) {
      const float b1 = __shfl_xor(m1, o, 64), b2 = __shfl_xor(m2, o, 64);
      const int bi = __shfl_xor(i1, o, 64);
      const float lo = fminf(m1, b1);
      if (b1 > m1 || (b1 == m1 && bi < i1)) { m1 = b1; i1 = bi; }
      m2 = fmaxf(lo, fmaxf(m2, b2));
    }
    if (tid == 0) { top[0] = m1; top[1] = m2; top[2] = __int_as_float(i1); }
  }
  __syncthreads();
  const float d1 = top[0], d2 = top[1];
  const int i1 = __float_as_int(top[2]);
  const bool flagged = hflag[h] != 0;
  const int64_t nchunk = (T + LB_CHUNK - 1) / LB_CHUNK;
  for (int64_t ch = blockIdx.y; ch < nchunk; ch += gridDim.y) {
    if (tid == 0) nl = 0;
    __syncthreads();
    uint32_t ew[4];
    int a[4];
    float u[4], l[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t t = ch * LB_CHUNK + 256 * k + tid;
      const int64_t o = (int64_t)h * T + (t < T ? t : 0);
      ew[k] = excl[h * excl_words + ((t < T ? t : 0) >> 5)];
      a[k] = assign[o];
      u[k] = ub[o];
      l[k] = lb[o];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t t = ch * LB_CHUNK + 256 * k + tid;
      if (t >= T || ((ew[k] >> (t & 31)) & 1u)) continue;
      bool push = flagged;
      if (!flagged) {
        const float uu = (u[k] + sd[a[k]]) * (1.0f + 1.0f / 4194304.0f);
        const float ll = (l[k] - (a[k] == i1 ? d2 : d1)) * (1.0f - 1.0f / 4194304.0f);
        if (uu < ll) {
          const int64_t o = (int64_t)h * T + t;
          ub[o] = uu;
          lb[o] = ll;
        } else {
          push = true;
        }
      }
      if (push) lst[atomicAdd(&nl, 1)] = (int32_t)t;
    }
    __syncthreads();
    if (tid == 0 && nl > 0) gbase = atomicAdd(&wl_cnt[h], nl);
    __syncthreads();
    for (int i = tid; i < nl; i += 256) wl[(int64_t)h * T + gbase + i] = lst[i];
    __syncthreads();   // lst and nl are reused by the next chunk
  }
}

}  // namespace qwm

namespace qwm_host {
using namespace qwm;

static constexpr size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t lloyd_state_bytes(int64_t T, int32_t H) {
  const size_t h = (size_t)H, t = (size_t)T;
  return al256(4 * h * D) * 2 + al256(4 * h) + al256(8 * h * NC * D) + al256(4 * h * NC) * 2 + al256(4 * h * t) * 3 +
         al256(4 * (h + 1)) + al256(8 * h * t);
}

LloydState lloyd_state_carve(char*& p, int64_t T, int32_t H, int32_t dtype) {
  auto take = [&](size_t n) { char* r = p; p += al256(n); return r; };
  const size_t h = (size_t)H, t = (size_t)T;
  LloydState s{};
  s.emax = reinterpret_cast<int32_t*>(take(4 * h * D));
  s.emin = reinterpret_cast<int32_t*>(take(4 * h * D));
  s.hflag = reinterpret_cast<int32_t*>(take(4 * h));
  s.sums = reinterpret_cast<int64_t*>(take(8 * h * NC * D));
  s.cnt = reinterpret_cast<int32_t*>(take(4 * h * NC));
  s.delta = reinterpret_cast<float*>(take(4 * h * NC));
  s.ub = reinterpret_cast<float*>(take(4 * h * t));
  s.lb = reinterpret_cast<float*>(take(4 * h * t));
  s.wl = reinterpret_cast<int32_t*>(take(4 * h * t));
  s.wl_cnt = reinterpret_cast<int32_t*>(take(4 * (h + 1)));
  s.chg_cnt = s.wl_cnt + H;
  s.chg = reinterpret_cast<uint2*>(take(8 * h * t));
  int bl = 0;
  for (int64_t v = T; v > 0; v >>= 1) ++bl;
  s.P = 62 - bl < 48 ? 62 - bl : 48;
  s.MB = dtype == QWM_BF16 ? 8 : 24;
  return s;
}

static void fill(int32_t* p, int64_t n, int32_t v, hipStream_t stream) {
  const int64_t nb = (n + 255) / 256;
  hipLaunchKernelGGL(lloyd_fill_kernel, dim3((unsigned)(nb < 1024 ? (nb < 1 ? 1 : nb) : 1024)), dim3(256), 0,
                     stream, p, n, v);
}

qwm_status lloyd_scan(const qwm_tokens* x, const LloydState& s, hipStream_t stream) {
  fill(s.emax, (int64_t)x->H * D, INT_MIN, stream);
  fill(s.emin, (int64_t)x->H * D, INT_MAX, stream);
  int64_t nb = (x->T + 16 * 64 - 1) / (16 * 64);   // about 64 rows per block
  nb = nb < 1 ? 1 : (nb > 64 ? 64 : nb);
  hipLaunchKernelGGL(lloyd_scan_kernel, dim3(x->H, (unsigned)nb), dim3(256), 0, stream, x->ptr, x->dtype, x->T,
                     x->stride_t, x->stride_h, s.emax, s.emin);
  hipLaunchKernelGGL(lloyd_flag_kernel, dim3(x->H), dim3(D), 0, stream, s.emax, s.emin, s.hflag, s.P, s.MB);
  return check_launch("Lloyd exponent scan");
}

qwm_status lloyd_bounds(const qwm_tokens* x, const uint8_t* assign, const uint32_t* excl, int64_t excl_words,
                        const LloydState& s, hipStream_t stream) {
  int64_t nb = (x->T + LB_CHUNK - 1) / LB_CHUNK;
  nb = nb < 1 ? 1 : (nb > 4096 ? 4096 : nb);
  hipLaunchKernelGGL(lloyd_bounds_kernel, dim3(x->H, (unsigned)nb), dim3(256), 0, stream, x->T, assign, excl,
                     excl_words, s.hflag, s.delta, s.ub, s.lb, s.wl, s.wl_cnt);
  return check_launch("Lloyd bounds");
}

qwm_status lloyd_apply_changes(const qwm_tokens* x, const LloydState& s, hipStream_t stream) {
  if (x->dtype == QWM_BF16)
    hipLaunchKernelGGL(lloyd_changes_kernel<8>, dim3(1024), dim3(256), 0, stream, x->ptr, x->T, x->stride_t,
                       x->stride_h, s.emax, s.hflag, s.chg, s.chg_cnt, s.sums, s.cnt, s.P);
  else
    hipLaunchKernelGGL(lloyd_changes_kernel<24>, dim3(1024), dim3(256), 0, stream, x->ptr, x->T, x->stride_t,
                       x->stride_h, s.emax, s.hflag, s.chg, s.chg_cnt, s.sums, s.cnt, s.P);
  return check_launch("Lloyd changes");
}

qwm_status lloyd_finalize(const qwm_tokens* x, const LloydState& s, const uint16_t* cur, uint16_t* out,
                          hipStream_t stream) {
  const int64_t units = (int64_t)x->H * NC;
  hipLaunchKernelGGL(lloyd_finalize_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, s.emax, s.hflag,
                     s.sums, s.cnt, s.delta, cur, out, x->H, s.P);
  return check_launch("Lloyd means");
}

}  // namespace qwm_host
