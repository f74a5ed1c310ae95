// Query statistics and principal Query basis (QuantWM Sec. 4.1-4.2, method
// step (1) and (4), App. C.3 cold start, App. D.1 incremental statistics).
//
//   S_h += sum_t q_t q_t^T   (fp64 running sum; each 16-token MFMA partial is
//                             exact-product fp32 and is folded into fp64)
//   n_h += T,  w_h = diag(S_h) / n_h  (w = 1 while n_h = 0)
//   U_r = top-8 eigenvectors of S_h / n_h (fp64 block subspace iteration with
//         Rayleigh-Ritz), stored in bf16; eigenvalues descending, the
//         largest-magnitude entry of each vector positive.
#include "common.hpp"

namespace qwm {

// ---------------------------------------------------------------------------
// Gram update, bf16 Queries, MFMA.  Grid (4, H): block (b, h) owns the
// 32-row stripe b of S_h; wave w owns the 32x32 tile (b, w).
// ---------------------------------------------------------------------------
constexpr int GRAM_TOK = 64;

__global__ __launch_bounds__(256) void gram_bf16_kernel(const uint16_t* __restrict__ q, int64_t T,
                                                        int64_t st, int64_t sh, double* __restrict__ S) {
  const int b = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hl = lane >> 5;
  __shared__ uint16_t qt[D][GRAM_TOK + 8];   // transposed tile [channel][token]
  double acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0;
  const uint16_t* qh = q + (int64_t)h * sh;
  for (int64_t t0 = 0; t0 < T; t0 += GRAM_TOK) {
    // stage 64 tokens: thread -> (token tid/4, channels 32*(tid%4) .. +32)
    {
      const int tk = tid >> 2, c0 = (tid & 3) * 32;
      const int64_t t = t0 + tk;
      if (t < T) {
        const u32x4* src = reinterpret_cast<const u32x4*>(qh + t * st + c0);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          u32x4 x = src[v];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qt[c0 + 8 * v + 2 * e][tk] = (uint16_t)(x[e] & 0xFFFFu);
            qt[c0 + 8 * v + 2 * e + 1][tk] = (uint16_t)(x[e] >> 16);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 32; ++c) qt[c0 + c][tk] = 0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < GRAM_TOK / 16; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&qt[32 * b + (lane & 31)][16 * ks + 8 * hl]);
      const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&qt[32 * w + (lane & 31)][16 * ks + 8 * hl]);
      f32x16 c = {};
      c = mfma_bf16(a, bb, c);   // products of bf16 values are exact in fp32
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += (double)c[i];
    }
    __syncthreads();
  }
  double* Sh = S + (int64_t)h * D * D;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 32 * b + c_row(i, hl), col = 32 * w + (lane & 31);
    Sh[row * D + col] += acc[i];
  }
}

// Gram update for fp32 Queries: plain fp64 FMAs (products of fp32 values are
// exact in fp64).  Grid (64, H), 256 threads, one S entry per thread.
__global__ __launch_bounds__(256) void gram_f32_kernel(const float* __restrict__ q, int64_t T, int64_t st,
                                                       int64_t sh, double* __restrict__ S) {
  const int h = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;   // 0 .. 16383
  const int i = e >> 7, j = e & 127;
  const float* qh = q + (int64_t)h * sh;
  double s = 0.0;
  for (int64_t t = 0; t < T; ++t) s = fma((double)qh[t * st + i], (double)qh[t * st + j], s);
  S[(int64_t)h * D * D + e] += s;
}

// n += T; w = diag(S)/n (w = 1 while n == 0).  Grid H, 128 threads.
__global__ void finalize_kernel(const double* __restrict__ S, int64_t* __restrict__ n, float* __restrict__ w,
                                int64_t T) {
  const int h = blockIdx.x, c = threadIdx.x;
  const int64_t nn = n[h] + T;
  __syncthreads();
  const double sc = S[(int64_t)h * D * D + c * D + c];
  w[h * D + c] = nn > 0 ? (float)(sc / (double)nn) : 1.0f;
  if (c == 0) n[h] = nn;
}

// ---------------------------------------------------------------------------
// Principal basis: block subspace iteration (P = 16 columns) in fp64, warm-
// started from the stored basis; each round is ORTH_PER_ROUND x POWER_STEPS
// products with A (Cholesky-QR re-orthonormalization in between) followed by a
// Rayleigh-Ritz step and a residual test on the top-8 Ritz pairs.  One 256-thread block per head; thread t holds row t/2, columns
// 64*(t%2) .. +64 of A = S/n in registers.
// ---------------------------------------------------------------------------
constexpr int P = 16;
constexpr int EIG_ROUNDS = 24;      // Rayleigh-Ritz checks
constexpr int POWER_STEPS = 3;      // products with A between re-orthonormalizations
constexpr int ORTH_PER_ROUND = 3;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct EigShared {
  double X[D][P + 1];
  double Y[D][P + 1];
  double Hm[P][P + 1];
  double W[P][P + 1];
  double G[P][P + 1];
  double red[8][P];
  double cs[P / 2][2];
  double theta[P];
  double trace;
  int conv;
};

// Y = A X
__device__ __forceinline__ void matvec(const double (&a)[64], EigShared& sm, int tid) {
  const int i = tid >> 1, half = tid & 1;
  double acc[P];
#pragma unroll
  for (int j = 0; j < P; ++j) acc[j] = 0.0;
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    const double av = a[c];
    const double* xr = sm.X[64 * half + c];
#pragma unroll
    for (int j = 0; j < P; ++j) acc[j] = fma(av, xr[j], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < P; ++j) acc[j] += __shfl_xor(acc[j], 1, 64);
  if (half == 0) {
#pragma unroll
    for (int j = 0; j < P; ++j) sm.Y[i][j] = acc[j];
  }
  __syncthreads();
}

// G = Y^T Y, or Hm = X^T Y when xty; one entry per thread, four independent
// partial sums so the LDS loads and fp64 FMAs overlap.
__device__ __forceinline__ void gram16(EigShared& sm, int tid, bool xty) {
  const int a = tid >> 4, b = tid & 15;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
#pragma unroll 4
  for (int i = 0; i < D; i += 4) {
    const double* L0 = xty ? sm.X[i] : sm.Y[i];
    const double* L1 = xty ? sm.X[i + 1] : sm.Y[i + 1];
    const double* L2 = xty ? sm.X[i + 2] : sm.Y[i + 2];
    const double* L3 = xty ? sm.X[i + 3] : sm.Y[i + 3];
    s0 = fma(L0[a], sm.Y[i][b], s0);
    s1 = fma(L1[a], sm.Y[i + 1][b], s1);
    s2 = fma(L2[a], sm.Y[i + 2][b], s2);
    s3 = fma(L3[a], sm.Y[i + 3][b], s3);
  }
  const double s = (s0 + s1) + (s2 + s3);
  if (xty) sm.Hm[a][b] = s; else sm.G[a][b] = s;
  __syncthreads();
}

// Cholesky of G (upper factor in G's upper triangle) by wave 0, lane = column.
__device__ void cholesky16(EigShared& sm, int tid) {
  if (tid < 64) {
    const int j = tid;
    double col[P];   // column j of the factor
#pragma unroll
    for (int p = 0; p < P; ++p) col[p] = 0.0;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      // r_kk from lane k
      double dkk = 0.0;
      if (j == k) {
        double s = sm.G[k][k];
#pragma unroll
        for (int p = 0; p < P; ++p) if (p < k) s -= col[p] * col[p];
        dkk = sqrt(fmax(s, 1e-300));
        col[k] = dkk;
      }
      dkk = __shfl(dkk, k, 64);
      // column k of the factor, broadcast entry by entry
      double ck[P];
#pragma unroll
      for (int p = 0; p < P; ++p) ck[p] = __shfl(col[p], k, 64);
      if (j > k && j < P) {
        double s = sm.G[k][j];
#pragma unroll
        for (int p = 0; p < P; ++p) if (p < k) s -= ck[p] * col[p];
        col[k] = s / dkk;
      }
    }
    if (j < P) {
#pragma unroll
      for (int p = 0; p < P; ++p) sm.G[p][j] = col[p];
    }
  }
  __syncthreads();
}

// X = Y R^{-1} (R upper, in G), rows in parallel.
__device__ __forceinline__ void solve_rows(EigShared& sm, int tid, bool into_x) {
  if (tid < D) {
    double x[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
      double s = sm.Y[tid][j];
#pragma unroll
      for (int p = 0; p < P; ++p) if (p < j) s -= x[p] * sm.G[p][j];
      x[j] = s / sm.G[j][j];
    }
#pragma unroll
    for (int j = 0; j < P; ++j) {
      if (into_x) sm.X[tid][j] = x[j]; else sm.Y[tid][j] = x[j];
    }
  }
  __syncthreads();
}

// X = orth(Y) by two rounds of Cholesky QR.
__device__ void orthonormalize(EigShared& sm, int tid) {
  gram16(sm, tid, false);
  cholesky16(sm, tid);
  solve_rows(sm, tid, false);   // Y <- Y R^-1
  gram16(sm, tid, false);
  cholesky16(sm, tid);
  solve_rows(sm, tid, true);    // X <- Y R^-1
}

// Cyclic Jacobi on the 16x16 symmetric Hm (parallel round-robin ordering),
// accumulating W.  All threads call; thread 0..7 own the 8 rotations of a round.
__device__ void jacobi16(EigShared& sm, int tid) {
  if (tid < P * P) {
    const int a = tid >> 4, b = tid & 15;
    sm.W[a][b] = (a == b) ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 8; ++sweep) {
    // convergence: off-diagonal mass
    if (tid == 0) {
      double off = 0.0, tot = 0.0;
      for (int a = 0; a < P; ++a)
        for (int b = 0; b < P; ++b) {
          const double v = sm.Hm[a][b] * sm.Hm[a][b];
          tot += v;
          if (a != b) off += v;
        }
      sm.conv = (off <= 1e-24 * tot) ? 1 : 0;
    }
    __syncthreads();
    if (sm.conv) break;
    for (int round = 0; round < P - 1; ++round) {
      // round-robin pairing of 16 indices: position 0 fixed, others rotate
      if (tid < P / 2) {
        auto pos = [&](int k) { return k == 0 ? 0 : 1 + (k - 1 + round) % (P - 1); };
        int p = pos(tid), q = pos(P - 1 - tid);
        if (p > q) { int t = p; p = q; q = t; }
        const double apq = sm.Hm[p][q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double theta = (sm.Hm[q][q] - sm.Hm[p][p]) / (2.0 * apq);
          const double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
          c = 1.0 / sqrt(t * t + 1.0);
          s = t * c;
        }
        sm.cs[tid][0] = c;
        sm.cs[tid][1] = s;
      }
      __syncthreads();
      // column update (Hm <- Hm J, W <- W J): thread -> (pair, row)
      double hp = 0, hq = 0, wp = 0, wq = 0;
      int p = 0, q = 0, row = 0;
      const bool act = tid < (P / 2) * P;
      if (act) {
        const int k = tid >> 4;
        row = tid & 15;
        auto pos = [&](int kk) { return kk == 0 ? 0 : 1 + (kk - 1 + round) % (P - 1); };
        p = pos(k); q = pos(P - 1 - k);
        if (p > q) { int t = p; p = q; q = t; }
        const double c = sm.cs[k][0], s = sm.cs[k][1];
        const double ap = sm.Hm[row][p], aq = sm.Hm[row][q];
        hp = c * ap - s * aq; hq = s * ap + c * aq;
        const double vp = sm.W[row][p], vq = sm.W[row][q];
        wp = c * vp - s * vq; wq = s * vp + c * vq;
      }
      __syncthreads();
      if (act) { sm.Hm[row][p] = hp; sm.Hm[row][q] = hq; sm.W[row][p] = wp; sm.W[row][q] = wq; }
      __syncthreads();
      // row update (Hm <- J^T Hm): thread -> (pair, column)
      if (act) {
        const int k = tid >> 4, col = tid & 15;
        const double c = sm.cs[k][0], s = sm.cs[k][1];
        const double ap = sm.Hm[p][col], aq = sm.Hm[q][col];
        hp = c * ap - s * aq; hq = s * ap + c * aq;
        row = col;
      }
      __syncthreads();
      if (act) { sm.Hm[p][row] = hp; sm.Hm[q][row] = hq; }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(256) void eig_kernel(const double* __restrict__ S, const int64_t* __restrict__ n,
                                                  uint16_t* __restrict__ U, float* __restrict__ lambda,
                                                  float* __restrict__ energy, int32_t* __restrict__ iters) {
  const int h = blockIdx.x, tid = threadIdx.x;
  __shared__ EigShared sm;
  const int64_t nn = n[h];
  uint16_t* Uh = U + (int64_t)h * D * R;
  if (nn <= 0) {
    for (int e = tid; e < D * R; e += 256) Uh[e] = 0;
    if (tid < R) lambda[h * R + tid] = 0.f;
    if (tid == 0) { energy[h] = 0.f; if (iters) iters[h] = 0; }
    return;
  }
  const double inv_n = 1.0 / (double)nn;
  const double* Sh = S + (int64_t)h * D * D;
  double a[64];
  {
    const int i = tid >> 1, half = tid & 1;
#pragma unroll
    for (int c = 0; c < 64; ++c) {
      // symmetric by construction: use the upper triangle
      const int col = 64 * half + c;
      const double v = (i <= col) ? Sh[i * D + col] : Sh[col * D + i];
      a[c] = v / (double)nn;
    }
  }
  if (tid == 0) {
    double tr = 0.0;
    for (int c = 0; c < D; ++c) tr += Sh[c * D + c] / (double)nn;
    sm.trace = tr;
  }
  (void)inv_n;
  // start: previous basis (if any) in columns 0..7, hashed vectors elsewhere
  {
    int mine = 0;
    for (int e = tid; e < D * R; e += 256) mine |= (Uh[e] != 0);
    const bool have_prev = __syncthreads_or(mine) != 0;
    for (int e = tid; e < D * P; e += 256) {
      const int i = e / P, j = e % P;
      double v;
      if (j < R && have_prev) {
        v = (double)bf16_bits_to_f32(Uh[i * R + j]);
        v += 1e-3 * ((double)(mix64(0x51ull * (e + 1)) >> 11) * (1.0 / 9007199254740992.0) - 0.5);
      } else {
        v = (double)(mix64(0x9E37ull * (e + 7) + (uint64_t)h) >> 11) * (1.0 / 9007199254740992.0) - 0.5;
      }
      sm.Y[i][j] = v;
    }
  }
  __syncthreads();
  orthonormalize(sm, tid);
  int it = 0, converged = 0;
  for (it = 1; it <= EIG_ROUNDS; ++it) {
    // subspace iteration: POWER_STEPS products with A per orthonormalization
    for (int o = 0; o < ORTH_PER_ROUND; ++o) {
      for (int p = 0; p < POWER_STEPS; ++p) {
        matvec(a, sm, tid);                 // Y = A X
        if (p + 1 < POWER_STEPS) {
          for (int e = tid; e < D * P; e += 256) sm.X[e / P][e % P] = sm.Y[e / P][e % P];
          __syncthreads();
        }
      }
      orthonormalize(sm, tid);              // X = orth(Y)
    }
    matvec(a, sm, tid);                     // Y = A X
    {
      gram16(sm, tid, true);            // Hm = X^T A X
      if (tid < P * P) {
        const int r = tid >> 4, c = tid & 15;
        const double v = 0.5 * (sm.Hm[r][c] + sm.Hm[c][r]);
        sm.G[r][c] = v;
      }
      __syncthreads();
      if (tid < P * P) sm.Hm[tid >> 4][tid & 15] = sm.G[tid >> 4][tid & 15];
      __syncthreads();
      jacobi16(sm, tid);
      // sort Ritz values descending (thread 0), permutation into red[0][*]
      if (tid == 0) {
        int order[P];
        for (int j = 0; j < P; ++j) order[j] = j;
        for (int x = 1; x < P; ++x)
          for (int y = x; y > 0 && sm.Hm[order[y]][order[y]] > sm.Hm[order[y - 1]][order[y - 1]]; --y) {
            int t = order[y]; order[y] = order[y - 1]; order[y - 1] = t;
          }
        for (int j = 0; j < P; ++j) { sm.theta[j] = sm.Hm[order[j]][order[j]]; sm.red[0][j] = (double)order[j]; }
      }
      __syncthreads();
      // X <- X W(:, order), Y <- Y W(:, order)
      {
        double xr[P], yr[P];
#pragma unroll
        for (int j = 0; j < P; ++j) { xr[j] = 0.0; yr[j] = 0.0; }
        if (tid < D) {
          for (int k = 0; k < P; ++k) {
            const double xk = sm.X[tid][k], yk = sm.Y[tid][k];
#pragma unroll
            for (int j = 0; j < P; ++j) {
              const double wkj = sm.W[k][(int)sm.red[0][j]];
              xr[j] = fma(xk, wkj, xr[j]);
              yr[j] = fma(yk, wkj, yr[j]);
            }
          }
        }
        __syncthreads();
        if (tid < D) {
#pragma unroll
          for (int j = 0; j < P; ++j) { sm.X[tid][j] = xr[j]; sm.Y[tid][j] = yr[j]; }
        }
      }
      __syncthreads();
      // residuals of the top R Ritz pairs
      if (tid < D) {
        double rs[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const double r = sm.Y[tid][j] - sm.theta[j] * sm.X[tid][j];
          rs[j] = r * r;
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
          double v = rs[j];
          for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
          if ((tid & 63) == 0) sm.red[1 + (tid >> 6)][j] = v;
        }
      }
      __syncthreads();
      if (tid == 0) {
        int ok = 1;
        const double scale = fabs(sm.theta[0]) > 0 ? fabs(sm.theta[0]) : 1.0;
        for (int j = 0; j < R; ++j) {
          const double res = sqrt(sm.red[1][j] + sm.red[2][j]);
          if (!(res <= 1e-9 * scale)) ok = 0;
        }
        sm.conv = ok;
      }
      __syncthreads();
      if (sm.conv) { converged = 1; break; }
    }
    orthonormalize(sm, tid);            // X = orth(Y), continue from the rotated basis
  }
  // outputs: sign rule, bf16, eigenvalues, energy
  if (tid < R) {
    const int j = tid;
    int imax = 0;
    double vmax = -1.0;
    for (int i = 0; i < D; ++i) {
      const double v = fabs(sm.X[i][j]);
      if (v > vmax) { vmax = v; imax = i; }
    }
    sm.red[3][j] = sm.X[imax][j] < 0 ? -1.0 : 1.0;
    lambda[h * R + j] = (float)sm.theta[j];
  }
  __syncthreads();
  for (int e = tid; e < D * R; e += 256) {
    const int i = e / R, j = e % R;
    Uh[e] = (uint16_t)f64_to_bf16_bits(sm.red[3][j] * sm.X[i][j]);
  }
  if (tid == 0) {
    double top = 0.0;
    for (int j = 0; j < R; ++j) top += sm.theta[j];
    energy[h] = (float)(top / sm.trace);
    if (iters) iters[h] = converged ? it : -it;
  }
}

}  // namespace qwm

// ---------------------------------------------------------------------------
// Host entry points (declared in api.hip).
// ---------------------------------------------------------------------------
namespace qwm_host {
using namespace qwm;

qwm_status launch_stats(const qwm_tokens* q, const qwm_qstats* st, int32_t compute_basis, hipStream_t stream) {
  if (q->T > 0) {
    if (q->dtype == QWM_BF16) {
      hipLaunchKernelGGL(gram_bf16_kernel, dim3(4, q->H), dim3(256), 0, stream,
                         static_cast<const uint16_t*>(q->ptr), q->T, q->stride_t, q->stride_h, st->S);
    } else {
      hipLaunchKernelGGL(gram_f32_kernel, dim3(64, q->H), dim3(256), 0, stream,
                         static_cast<const float*>(q->ptr), q->T, q->stride_t, q->stride_h, st->S);
    }
    qwm_status s = check_launch("query stats gram");
    if (s != QWM_OK) return s;
  }
  hipLaunchKernelGGL(finalize_kernel, dim3(st->H), dim3(D), 0, stream, st->S, st->n, st->w, q->T);
  qwm_status s = check_launch("query stats finalize");
  if (s != QWM_OK) return s;
  if (compute_basis) {
    hipLaunchKernelGGL(eig_kernel, dim3(st->H), dim3(256), 0, stream, st->S, st->n, st->U, st->lambda,
                       st->energy, st->iters);
    s = check_launch("principal basis");
  }
  return s;
}
}  // namespace qwm_host
