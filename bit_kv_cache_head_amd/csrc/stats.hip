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
// started from the stored basis.  Each round is ORTH_PER_ROUND x POWER_STEPS
// products with A (Cholesky-QR re-orthonormalization in between), then a
// Rayleigh-Ritz step and a residual test on the top-8 Ritz pairs.
//
// One 256-thread block per head.  The products A X and the 16x16 Gram
// matrices run on the fp64 MFMA (v_mfma_f64_16x16x4, IEEE fp64 FMAs); wave w
// keeps rows 32w .. 32w+31 of A = S/n in registers as MFMA A-fragments.
// Lane layout of the 16x16x4 fp64 MFMA: A[i][k] from lane i + 16k, B[k][j]
// from lane j + 16k, result D[i][j] in lane j + 16 (i % 4), register i / 4.
// ---------------------------------------------------------------------------
constexpr int P = 16;
constexpr int PP = P + 1;             // padded row
constexpr int EIG_ROUNDS = 24;        // Rayleigh-Ritz checks
constexpr int POWER_STEPS = 3;        // products with A between re-orthonormalizations
constexpr int ORTH_PER_ROUND = 4;
// Residual test |A x - theta x| <= EIG_RESIDUAL * theta_1: the eigenvector error
// it leaves (~ residual / eigen-gap, ~1e-6 here) is at the level of the
// statistics' own rounding (fp32 partial sums of bf16 products, 1e-6
// relative) and far below half a bf16 ulp of the stored basis.
constexpr double EIG_RESIDUAL = 1e-7;

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f64x4 mfma_f64(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct EigShared {
  double X[D][PP];        // orthonormal block
  double Y[D][PP];        // products
  double Z[D][PP];        // second product buffer
  double part[4][P][PP];  // per-wave Gram partials
  double Hm[P][PP];
  double W[P][PP];
  double G[P][PP];
  double rd[P];           // reciprocals of G's diagonal (solve_rows)
  double cs[P / 2][2];
  double theta[P];
  double red[4][P];
  int order[P];
  double trace;
};

// dst = A src (128 x 16).
__device__ __forceinline__ void matvec(const double (&a)[2][32], const double (*src)[PP], double (*dst)[PP],
                                       int tid) {
  const int l = tid & 63, wv = tid >> 6;
  f64x4 c0 = {0.0, 0.0, 0.0, 0.0}, c1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const double bv = src[4 * s + (l >> 4)][l & 15];
    c0 = mfma_f64(a[0][s], bv, c0);
    c1 = mfma_f64(a[1][s], bv, c1);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    dst[32 * wv + (l >> 4) + 4 * r][l & 15] = c0[r];
    dst[32 * wv + 16 + (l >> 4) + 4 * r][l & 15] = c1[r];
  }
  __syncthreads();
}

// out = L^T R (16 x 16); wave w sums rows 32w .. 32w+31, partials added in a fixed order.
__device__ __forceinline__ void gram16(EigShared& sm, const double (*L)[PP], const double (*Rm)[PP],
                                       double (*out)[PP], int tid) {
  const int l = tid & 63, wv = tid >> 6;
  f64x4 c0 = {0.0, 0.0, 0.0, 0.0}, c1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < 8; s += 2) {
    const int r0 = 32 * wv + 4 * s + (l >> 4);
    c0 = mfma_f64(L[r0][l & 15], Rm[r0][l & 15], c0);
    c1 = mfma_f64(L[r0 + 4][l & 15], Rm[r0 + 4][l & 15], c1);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) sm.part[wv][(l >> 4) + 4 * r][l & 15] = c0[r] + c1[r];
  __syncthreads();
  {
    const int i = tid >> 4, j = tid & 15;
    out[i][j] = (sm.part[0][i][j] + sm.part[1][i][j]) + (sm.part[2][i][j] + sm.part[3][i][j]);
  }
  __syncthreads();
}

// Upper Cholesky factor of G + shift*I into G's upper triangle, by wave 0
// (lane j = column j).  shift_rel > 0 adds shift_rel * trace(G) to the
// diagonal (shifted Cholesky-QR: keeps the factorization finite when the
// block is numerically rank deficient).
__device__ void cholesky16(EigShared& sm, int tid, double shift_rel) {
  if (tid < 64) {
    const int j = tid;
    double shift = 0.0;
    if (shift_rel > 0.0) {
      double dj = (j < P) ? sm.G[j][j] : 0.0;
      shift = shift_rel * wave_sum_d(dj);
    }
    double col[P];
#pragma unroll
    for (int p = 0; p < P; ++p) col[p] = 0.0;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      double dkk = 0.0;
      if (j == k) {
        double s = sm.G[k][k] + shift;
#pragma unroll
        for (int p = 0; p < P; ++p) if (p < k) s -= col[p] * col[p];
        dkk = sqrt(fmax(s, 1e-300));
        col[k] = dkk;
      }
      dkk = __shfl(dkk, k, 64);
      double ck[P];
#pragma unroll
      for (int p = 0; p < P; ++p) ck[p] = (p < k) ? __shfl(col[p], k, 64) : 0.0;
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

// dst = src R^{-1} (R upper, in G), one row per thread; src == dst allowed.
// The 16 pivot reciprocals are formed once (sm.rd) and multiplied.
__device__ __forceinline__ void solve_rows(EigShared& sm, const double (*src)[PP], double (*dst)[PP], int tid) {
  if (tid < P) sm.rd[tid] = 1.0 / sm.G[tid][tid];
  __syncthreads();
  if (tid < D) {
    double x[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
      double s = src[tid][j];
#pragma unroll
      for (int p = 0; p < P; ++p) if (p < j) s -= x[p] * sm.G[p][j];
      x[j] = s * sm.rd[j];
    }
#pragma unroll
    for (int j = 0; j < P; ++j) dst[tid][j] = x[j];
  }
  __syncthreads();
}

// dst = orth(src) by `passes` rounds of Cholesky QR, the first one shifted;
// the intermediate passes overwrite src.  After the shifted pass (shift s =
// 3e-12 trace) column j has squared norm ~ r_j^2 / (r_j^2 + s), r_j being its
// component orthogonal to the earlier columns, so a column well below 1 is a
// direction the block does not really span (A rank deficient, e.g. fewer
// Queries than columns, leaves only rounding noise there, and that noise is
// nearly the same in every column).  Such columns are replaced by fresh hashed
// vectors so that the next pass sees a full-rank block.  `salt` varies the
// replacements from call to call.
__device__ void orthonormalize(EigShared& sm, double (*src)[PP], double (*dst)[PP], int passes, int tid,
                               int& salt, int h) {
  for (int ps = 0; ps < passes; ++ps) {
    gram16(sm, src, src, sm.G, tid);
    if (ps == 1) {
      uint32_t weak = 0;
#pragma unroll
      for (int j = 0; j < P; ++j) weak |= (!(sm.G[j][j] >= 0.1) ? 1u : 0u) << j;   // NaN counts as weak
      if (weak) {                       // uniform: every thread read the same diagonal
        ++salt;
        for (int e = tid; e < D * P; e += 256) {
          const int i = e / P, j = e % P;
          if ((weak >> j) & 1u)
            src[i][j] = (double)(mix64(0xC0FFEEull * (uint64_t)salt + 0x9E37ull * (uint64_t)e +
                                       ((uint64_t)h << 40)) >> 11) * (1.0 / 9007199254740992.0) - 0.5;
        }
        __syncthreads();
        gram16(sm, src, src, sm.G, tid);
        cholesky16(sm, tid, 3e-12);     // the new columns are not orthogonal yet: shift once more
        solve_rows(sm, src, src, tid);
        gram16(sm, src, src, sm.G, tid);
      }
    }
    cholesky16(sm, tid, ps == 0 ? 3e-12 : 0.0);
    solve_rows(sm, src, ps + 1 == passes ? dst : src, tid);
  }
}

// Cyclic Jacobi on the symmetric 16x16 Hm (parallel round-robin ordering,
// eight disjoint rotations per round), accumulating W.  Runs in wave 0; the
// rotations of one round touch disjoint entries, so each lane updates the
// entries it read.
__device__ __forceinline__ int rr_pos(int k, int round) { return k == 0 ? 0 : 1 + (k - 1 + round) % (P - 1); }

__device__ void jacobi16(EigShared& sm, int tid) {
  if (tid < 64) {
    const int l = tid;
    for (int e = l; e < P * P; e += 64) sm.W[e >> 4][e & 15] = ((e >> 4) == (e & 15)) ? 1.0 : 0.0;
    wave_sync();
    for (int sweep = 0; sweep < 10; ++sweep) {
      double off = 0.0, tot = 0.0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = l + 64 * u;
        const double v = sm.Hm[e >> 4][e & 15];
        tot += v * v;
        if ((e >> 4) != (e & 15)) off += v * v;
      }
      off = wave_sum_d(off);
      tot = wave_sum_d(tot);
      if (off <= 1e-24 * tot) break;
      for (int round = 0; round < P - 1; ++round) {
        if (l < P / 2) {
          int p = rr_pos(l, round), q = rr_pos(P - 1 - l, round);
          if (p > q) { const int t = p; p = q; q = t; }
          const double apq = sm.Hm[p][q];
          double c = 1.0, sn = 0.0;
          if (apq != 0.0) {
            const double theta = (sm.Hm[q][q] - sm.Hm[p][p]) / (2.0 * apq);
            const double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
            c = 1.0 / sqrt(t * t + 1.0);
            sn = t * c;
          }
          sm.cs[l][0] = c;
          sm.cs[l][1] = sn;
        }
        wave_sync();
        // columns: Hm <- Hm J, W <- W J; task (pair k, row)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = l + 64 * u, k = e >> 4, row = e & 15;
          int p = rr_pos(k, round), q = rr_pos(P - 1 - k, round);
          if (p > q) { const int t = p; p = q; q = t; }
          const double c = sm.cs[k][0], sn = sm.cs[k][1];
          const double ap = sm.Hm[row][p], aq = sm.Hm[row][q];
          const double vp = sm.W[row][p], vq = sm.W[row][q];
          sm.Hm[row][p] = c * ap - sn * aq;
          sm.Hm[row][q] = sn * ap + c * aq;
          sm.W[row][p] = c * vp - sn * vq;
          sm.W[row][q] = sn * vp + c * vq;
        }
        wave_sync();
        // rows: Hm <- J^T Hm; task (pair k, column)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = l + 64 * u, k = e >> 4, col = e & 15;
          int p = rr_pos(k, round), q = rr_pos(P - 1 - k, round);
          if (p > q) { const int t = p; p = q; q = t; }
          const double c = sm.cs[k][0], sn = sm.cs[k][1];
          const double ap = sm.Hm[p][col], aq = sm.Hm[q][col];
          sm.Hm[p][col] = c * ap - sn * aq;
          sm.Hm[q][col] = sn * ap + c * aq;
        }
        wave_sync();
      }
    }
    // Ritz values in descending order (rank by counting; ties by index)
    if (l < P) {
      const double v = sm.Hm[l][l];
      int rank = 0;
#pragma unroll
      for (int m = 0; m < P; ++m) {
        const double o = sm.Hm[m][m];
        rank += (o > v) || (o == v && m < l);
      }
      sm.order[rank] = l;
      sm.theta[rank] = v;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void eig_kernel(const double* __restrict__ S, const int64_t* __restrict__ n,
                                                  uint16_t* __restrict__ U, float* __restrict__ lambda,
                                                  float* __restrict__ energy, int32_t* __restrict__ iters) {
  const int h = blockIdx.x, tid = threadIdx.x, l = tid & 63, wv = tid >> 6;
  __shared__ EigShared sm;
  const int64_t nn = n[h];
  uint16_t* Uh = U + (int64_t)h * D * R;
  if (nn <= 0) {
    for (int e = tid; e < D * R; e += 256) Uh[e] = 0;
    if (tid < R) lambda[h * R + tid] = 0.f;
    if (tid == 0) { energy[h] = 0.f; if (iters) iters[h] = 0; }
    return;
  }
  const double* Sh = S + (int64_t)h * D * D;
  // A = S / n as MFMA A-fragments: a[t][s] = A[32w + 16t + l%16][4s + l/16]
  // (symmetric by construction: read the upper triangle)
  double a[2][32];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const int i = 32 * wv + 16 * t + (l & 15), c = 4 * s + (l >> 4);
      const double v = (i <= c) ? Sh[i * D + c] : Sh[c * D + i];
      a[t][s] = v / (double)nn;
    }
  }
  if (tid < 64) {
    double tr = 0.0;
    for (int c = l; c < D; c += 64) tr += Sh[c * D + c] / (double)nn;
    tr = wave_sum_d(tr);
    if (l == 0) sm.trace = tr;
  }
  // start: previous basis (if any) in columns 0..7, hashed vectors elsewhere.
  // A stored basis with a non-finite entry (e.g. never initialised) is ignored.
  {
    int mine = 0, bad = 0;
    for (int e = tid; e < D * R; e += 256) {
      mine |= (Uh[e] != 0);
      bad |= !is_finite_f(bf16_bits_to_f32(Uh[e]));
    }
    const bool have_prev = __syncthreads_or(mine) != 0 && __syncthreads_or(bad) == 0;
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
  int salt = 0;
  orthonormalize(sm, sm.Y, sm.X, 2, tid, salt, h);
  int it = 0, converged = 0;
  for (it = 1; it <= EIG_ROUNDS; ++it) {
    for (int o = 0; o < ORTH_PER_ROUND; ++o) {
      // POWER_STEPS products, ping-ponging so that the last lands in Y
      const double (*src)[PP] = sm.X;
#pragma unroll
      for (int p = 0; p < POWER_STEPS; ++p) {
        double (*dst)[PP] = ((POWER_STEPS - 1 - p) % 2 == 0) ? sm.Y : sm.Z;
        matvec(a, src, dst, tid);
        src = dst;
      }
      // between power steps one (shifted) Cholesky-QR pass keeps the block well
      // conditioned; the last one before Rayleigh-Ritz is a full second pass
      orthonormalize(sm, sm.Y, sm.X, o + 1 == ORTH_PER_ROUND ? 2 : 1, tid, salt, h);
    }
    matvec(a, sm.X, sm.Y, tid);                   // Y = A X
    // Rayleigh-Ritz: Hm = sym(X^T A X), eigen-decomposed by Jacobi
    gram16(sm, sm.X, sm.Y, sm.G, tid);
    {
      const int r = tid >> 4, c = tid & 15;
      sm.Hm[r][c] = 0.5 * (sm.G[r][c] + sm.G[c][r]);
    }
    __syncthreads();
    jacobi16(sm, tid);
    // X <- X W(:, order), Y <- Y W(:, order)
    if (tid < D) {
      double xr[P], yr[P];
#pragma unroll
      for (int j = 0; j < P; ++j) { xr[j] = 0.0; yr[j] = 0.0; }
      for (int k = 0; k < P; ++k) {
        const double xk = sm.X[tid][k], yk = sm.Y[tid][k];
#pragma unroll
        for (int j = 0; j < P; ++j) {
          const double wkj = sm.W[k][sm.order[j]];
          xr[j] = fma(xk, wkj, xr[j]);
          yr[j] = fma(yk, wkj, yr[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < P; ++j) { sm.X[tid][j] = xr[j]; sm.Y[tid][j] = yr[j]; }
    }
    __syncthreads();
    // residuals |A x_j - theta_j x_j| of the top R Ritz pairs (rows split over waves 0, 1)
    if (tid < D) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const double r = sm.Y[tid][j] - sm.theta[j] * sm.X[tid][j];
        const double v = wave_sum_d(r * r);
        if (l == 0) sm.red[wv][j] = v;
      }
    }
    __syncthreads();
    {
      const double scale = fabs(sm.theta[0]) > 0 ? fabs(sm.theta[0]) : 1.0;
      int ok = 1;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const double res = sqrt(sm.red[0][j] + sm.red[1][j]);
        ok &= (res <= EIG_RESIDUAL * scale) ? 1 : 0;
      }
      if (ok) { converged = 1; break; }   // uniform: every thread reads the same values
    }
    orthonormalize(sm, sm.Y, sm.X, 2, tid, salt, h);  // continue from A X_rot
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

// ---------------------------------------------------------------------------
// Principal basis for the rank ablation (r = 16, 32): one-sided (Hestenes)
// Jacobi in fp64 on W = S / n + tau I, tau = trace / d > 0, one block per head.
// Column pairs are rotated until every pair is orthogonal; then the columns
// are (lambda_i + tau) v_i, so their norms order the eigenvalues and their
// directions are the eigenvectors (the shift keeps every column away from
// zero, so a rank-deficient M still yields an orthonormal basis).  Rounds
// follow the circle method: 127 rounds of 64 disjoint pairs cover every pair
// once per sweep.  Thread (pair tid / 4, rows 32 (tid % 4) .. +32).  W lives in
// LDS column-major with a 2-double pad per column, so the 16 columns a wave
// touches at one row offset fall on distinct banks.
// ---------------------------------------------------------------------------
constexpr int JW = D + 2;             // doubles per stored column
constexpr int JACOBI_SWEEPS = 30;
constexpr double JACOBI_TOL = 1e-11;  // |w_p . w_q| <= tol ||w_p|| ||w_q|| for every pair

__device__ __forceinline__ int circle_player(int m, int round) {
  return m == 0 ? 0 : 1 + (m - 1 + round) % (D - 1);
}

__global__ __launch_bounds__(256) void jacobi_eig_kernel(const double* __restrict__ S, const int64_t* __restrict__ n,
                                                         uint16_t* __restrict__ U, float* __restrict__ lambda,
                                                         float* __restrict__ energy, int32_t* __restrict__ iters,
                                                         int32_t r) {
  const int h = blockIdx.x, tid = threadIdx.x;
  __shared__ double W[D * JW];
  __shared__ double nrm[D];
  __shared__ int order[D];
  __shared__ double trace_s;
  __shared__ int rotated;
  const int64_t nn = n[h];
  uint16_t* Uh = U + (int64_t)h * D * r;
  if (nn <= 0) {
    for (int e = tid; e < D * r; e += 256) Uh[e] = 0;
    if (tid < r) lambda[h * r + tid] = 0.f;
    if (tid == 0) { energy[h] = 0.f; if (iters) iters[h] = 0; }
    return;
  }
  const double* Sh = S + (int64_t)h * D * D;
  if (tid < 64) {
    double tr = 0.0;
    for (int c = tid; c < D; c += 64) tr += Sh[c * D + c] / (double)nn;
    tr = wave_sum_d(tr);
    if (tid == 0) trace_s = tr;
  }
  __syncthreads();
  const double tau = trace_s > 0.0 ? trace_s / D : 1.0;
  for (int e = tid; e < D * D; e += 256) {
    const int c = e / D, i = e % D;   // column c, row i (symmetric: read the upper triangle)
    const double v = (i <= c) ? Sh[i * D + c] : Sh[c * D + i];
    W[c * JW + i] = v / (double)nn + (i == c ? tau : 0.0);
  }
  __syncthreads();
  const int pr = tid >> 2, part = tid & 3, r0 = 32 * part;
  if (tid == 0) rotated = 0;
  __syncthreads();
  int sweep = 0;
  for (sweep = 1; sweep <= JACOBI_SWEEPS; ++sweep) {
    for (int round = 0; round < D - 1; ++round) {
      const int p = circle_player(pr, round), q = circle_player(D - 1 - pr, round);
      double* wp = W + p * JW + r0;
      double* wq = W + q * JW + r0;
      double al = 0.0, be = 0.0, ga = 0.0;
#pragma unroll 8
      for (int i = 0; i < 32; ++i) {
        const double x = wp[i], y = wq[i];
        al = fma(x, x, al);
        be = fma(y, y, be);
        ga = fma(x, y, ga);
      }
      // the pair's four threads are consecutive lanes of one wave
      al += __shfl_xor(al, 1, 64); be += __shfl_xor(be, 1, 64); ga += __shfl_xor(ga, 1, 64);
      al += __shfl_xor(al, 2, 64); be += __shfl_xor(be, 2, 64); ga += __shfl_xor(ga, 2, 64);
      if (fabs(ga) > JACOBI_TOL * sqrt(al * be)) {
        // rotation that makes the pair orthogonal (smaller of the two angles)
        const double zeta = (be - al) / (2.0 * ga);
        const double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
        const double c = 1.0 / sqrt(1.0 + t * t), sn = c * t;
#pragma unroll 8
        for (int i = 0; i < 32; ++i) {
          const double x = wp[i], y = wq[i];
          wp[i] = c * x - sn * y;
          wq[i] = sn * x + c * y;
        }
        if (part == 0) rotated = 1;   // benign race: every writer stores 1
      }
      __syncthreads();
    }
    const int any = rotated;   // every thread reads the flag after the last round's barrier ...
    __syncthreads();
    if (tid == 0) rotated = 0;   // ... before it is cleared for the next sweep
    __syncthreads();
    if (!any) break;
  }
  // column norms = lambda + tau; order descending (lower column first on ties)
  if (tid < D) {
    double s2 = 0.0;
    for (int i = 0; i < D; ++i) s2 = fma(W[tid * JW + i], W[tid * JW + i], s2);
    nrm[tid] = sqrt(s2);
  }
  __syncthreads();
  if (tid < D) {
    const double v = nrm[tid];
    int rank = 0;
    for (int c = 0; c < D; ++c) rank += (nrm[c] > v || (nrm[c] == v && c < tid)) ? 1 : 0;
    order[rank] = tid;
  }
  __syncthreads();
  // outputs: the top r columns, normalised, largest-magnitude entry positive
  if (tid < r) {
    const int c = order[tid];
    int imax = 0;
    double vmax = -1.0;
    for (int i = 0; i < D; ++i) {
      const double v = fabs(W[c * JW + i]);
      if (v > vmax) { vmax = v; imax = i; }
    }
    const double sg = (W[c * JW + imax] < 0.0 ? -1.0 : 1.0) / nrm[c];
    for (int i = 0; i < D; ++i) Uh[i * r + tid] = (uint16_t)f64_to_bf16_bits(sg * W[c * JW + i]);
    lambda[h * r + tid] = (float)(nrm[c] - tau);
  }
  if (tid == 0) {
    double top = 0.0;
    for (int j = 0; j < r; ++j) top += nrm[order[j]] - tau;
    energy[h] = (float)(top / trace_s);
    if (iters) iters[h] = sweep <= JACOBI_SWEEPS ? sweep : -JACOBI_SWEEPS;
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
    if (st->r == R)
      hipLaunchKernelGGL(eig_kernel, dim3(st->H), dim3(256), 0, stream, st->S, st->n, st->U, st->lambda,
                         st->energy, st->iters);
    else
      hipLaunchKernelGGL(jacobi_eig_kernel, dim3(st->H), dim3(256), 0, stream, st->S, st->n, st->U, st->lambda,
                         st->energy, st->iters, st->r);
    s = check_launch("principal basis");
  }
  return s;
}
}  // namespace qwm_host
