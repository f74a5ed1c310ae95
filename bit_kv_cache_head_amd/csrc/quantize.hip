// Centroid choice, INT2 residual codec, PSAC coefficients and the Lloyd
// iteration (QuantWM Sec. 2 centroid-residual code, Sec. 4.1 QSAC, Sec. 4.2
// PSAC; method steps (2)-(4); App. D.1 packed storage).
//
// Every token's centroid choice is computed from one MFMA GEMM of the token
// against the per-head table m_j = bf16(-2 w (.) mu_j), augmented with
// B_j = ||mu_j||_w^2 split over three bf16 columns, so that
//     f_j ~ e_j = ||k - mu_j||_w^2 - ||k||_w^2
// with a certified error |f_j - e_j| <= c (||k||_w^2 + B_j).  A token whose
// choice the bound cannot certify (close runners-up, non-finite values) is
// sent to an exact fp64 path; no result depends on the approximation.
#include <atomic>
#include <climits>
#include <mutex>

#include "common.hpp"
#include "lloyd.hpp"
#include "psac.hpp"

namespace qwm {

enum { MODE_ASSIGN = 0, MODE_VALUES = 1, MODE_KEYS = 2 };

constexpr int PREP_PARTS = NC / 32;   // table-preparation blocks per head

constexpr int SEL_TOK = 128;     // tokens per block pass (4 waves x 32)
// Internal selection flag (above the public QWM_* bits): the key or value blocks of a
// head take its wave tiles from the per-head counters at counter + 4.
constexpr uint32_t SEL_HEAD_COUNTERS = 0x80000000u;

struct TablePrepArgs {
  const uint16_t* mu;   // [H][256][128] bf16
  const float* w;       // [H][128] or null (w = 1)
  uint16_t* aug;        // [H][256][4]   bf16  (B hi, mid, lo, 0)
  float* Bj;            // [H][256]
  float* Bmax;          // [H][PREP_PARTS] partial maxima of B (times 1 + 2^-16)
  double* Wg;           // [H][2]
  int32_t* counter;     // fallback work counter, then at counter + 4 the H wave-tile counters (all zeroed here)
  int32_t* zero; int32_t nzero;   // more counters zeroed here (Lloyd lists), or null
  int32_t H;
};

// Block (h, part): centroids 32 part .. +32 of head h; thread (centroid
// 32 part + tid / 8, channels 16 (tid % 8) .. +16).  B_j is summed over each
// thread's 16 channels in fp64 and then over the 8 threads of the centroid.
// Each block writes the maximum of its 32 B_j; block 0 the group weight sums.
__global__ __launch_bounds__(256) void prep_table_kernel(TablePrepArgs a) {
  const int h = blockIdx.x, part = blockIdx.y, tid = threadIdx.x;
  const int j = 32 * part + (tid >> 3), c0 = 16 * (tid & 7);
  __shared__ float ws[D];
  __shared__ float bm[4];
  if (tid < D) ws[tid] = a.w ? a.w[h * D + tid] : 1.0f;
  if (h == 0 && part == 0) {
    if (tid == 0) *a.counter = 0;
    for (int i = tid; i < a.H; i += 256) a.counter[4 + i] = 0;
  }
  if (h == 0 && part == 0 && a.zero)
    for (int i = tid; i < a.nzero; i += 256) a.zero[i] = 0;
  __syncthreads();
  const uint16_t* mj = a.mu + ((int64_t)h * NC + j) * D + c0;
  double B = 0.0;
  u32x4 v[2];
  v[0] = *reinterpret_cast<const u32x4*>(mj);
  v[1] = *reinterpret_cast<const u32x4*>(mj + 8);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = c0 + 8 * half + 2 * e;
      uint32_t lo16 = v[half][e] & 0xFFFFu, hi16 = v[half][e] >> 16;
      const float m0 = bf16_bits_to_f32(lo16), m1 = bf16_bits_to_f32(hi16);
      const float w0 = ws[c], w1 = ws[c + 1];
      B = fma((double)w0 * (double)m0, (double)m0, B);
      B = fma((double)w1 * (double)m1, (double)m1, B);
    }
  }
  // the centroid's 8 partial sums, in a fixed order
  B += __shfl_xor(B, 1, 64);
  B += __shfl_xor(B, 2, 64);
  B += __shfl_xor(B, 4, 64);
  if ((tid & 7) == 0) {
    const uint32_t bh = f64_to_bf16_bits(B);
    const double r1 = B - (double)bf16_bits_to_f32(bh);
    const uint32_t bmid = f64_to_bf16_bits(r1);
    const double r2 = r1 - (double)bf16_bits_to_f32(bmid);
    const uint32_t blo = f64_to_bf16_bits(r2);
    uint16_t* ag = a.aug + ((int64_t)h * NC + j) * 4;
    ag[0] = (uint16_t)bh; ag[1] = (uint16_t)bmid; ag[2] = (uint16_t)blo; ag[3] = 0;
    a.Bj[h * NC + j] = (float)B;
  }
  // block max of B over its 32 centroids; group weight sums over 64 channels
  // (fp64 sums of fp32 weights, exact for any sane spread of magnitudes)
  const float wmax = wave_max_f((float)B);
  const int lane = tid & 63, wv = tid >> 6;
  if (lane == 0) bm[wv] = wmax;
  double gsum = 0.0;
  if (part == 0 && wv < 2) gsum = wave_sum_d((double)ws[tid]);
  __syncthreads();
  if (tid == 0) a.Bmax[h * PREP_PARTS + part] = fmaxf(fmaxf(bm[0], bm[1]), fmaxf(bm[2], bm[3])) * (1.0f + 1.0f / 65536.0f);
  if (part == 0 && wv < 2 && lane == 0) a.Wg[2 * h + wv] = gsum;
}

struct SelectArgs {
  const void* x; int64_t T; int64_t st; int64_t sh; int32_t H;
  const uint16_t* aug; const float* Bj; const float* Bmax;
  const double* Wg;
  const uint16_t* mu;   // [H][256][128]
  const float* w;       // [H][128] or null
  const uint16_t* U;    // [H][128][8] or null
  int32_t M; uint32_t flags; float cb;  // cb: certified relative error coefficient
  // outputs
  uint8_t* idx;         // [H][T] (assignment for MODE_ASSIGN)
  uint8_t* codes; uint16_t* scale; uint8_t* zeros; int64_t zstride; int8_t* cq; uint16_t* cscale;
  // counter: the exact path's work counter; counter + 4 .. + 4 + H: the heads'
  // key or value wave-tile counters (SEL_HEAD_COUNTERS); both zeroed by the
  // table preparation
  int32_t* counter; int32_t* worklist;
  qwm_diag* diag;
  // full-matrix candidate distance: S [H][128][128] fp64, n [H], mu^T S mu [H][256]
  const double* qS; const int64_t* qn; const double* qB;
  // Lloyd: one bit per token, set for rows with a non-finite channel (they
  // take no part in the mean update); [H][excl_words] u32
  uint32_t* excl; int64_t excl_words;
  // Lloyd with distance bounds (MODE_ASSIGN): per token-head an upper bound on
  // the distance to the chosen centroid and a lower bound on the distance to
  // every other ([H][T], or null); after the first iteration only the tokens
  // of the per-head lists wl [H][T] (counts wl_cnt [H]) are assigned, and every
  // changed assignment is recorded as (h T + t, old | new << 8) in chg
  float* ub; float* lb;
  const int32_t* wl; const int32_t* wl_cnt;
  uint2* chg; int32_t* chg_cnt;
};

// Orders one wave's LDS writes before its later reads (and reads before later
// writes) of the same locations: the compiler keeps them in program order and
// one wave's LDS operations complete in order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int MU_ROW = D + 8;   // elements per staged centroid row (16 bytes of padding)
struct SelShared {
  uint16_t mu[NC * MU_ROW];    // centroid rows, padded: 16-byte chunk c of row j at chunk 17 j + c
  uint16_t aug[NC][4];
  float bj[NC];
  float w[D];
  float wm2[D];                // -2 w (exact)
  uint16_t ut[R][D];           // U^T (bf16)
  uint8_t idx[4][32];
  union {
    struct {                   // keys and values: the wave's 32 tokens, staged for coalesced stores
      uint8_t codes[4][32][32];
      uint16_t scale[4][32][2];
      uint8_t nib[4][32];
      int8_t cq[4][32][R];
      uint16_t cs[4][32];
    } k;
    struct {                   // Lloyd assignment: the wave's tokens, their bounds, certified or not
      int32_t tok[4][32];
      float ub[4][32];
      float lb[4][32];
      uint8_t fast[4][32];
    } l;
  };
};

// Two fp32 values as a bf16 pair (RNE; v_cvt_pk_bf16_f32), and its halves as fp32.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  bf16x2 p;
  p[0] = (__bf16)a;
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ float lo_bf16(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// f with its low byte replaced by byte b of jb (v_perm_b32, selector
// 0x07060500 + b: bytes 3..1 of f, then byte b of jb).
__device__ __forceinline__ float pack_idx(float f, uint32_t jb, int b) {
  return __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(f), jb, 0x07060500u + (uint32_t)b));
}

// Thresholds of the INT2 code: q = #{k : r > tau'_k}, k = 1..3.
struct GroupCodec {
  float s;       // step (fp16 value)
  int z;         // zero-point
  float t1, t2, t3;
  uint32_t sbits;
};

__device__ __forceinline__ GroupCodec make_codec(float lo, float hi, bool* sat) {
  GroupCodec g;
  const double Rg = (double)hi - (double)lo;
  g.sbits = fp16_up_div(Rg, 3.0f, sat);
  g.s = f16_bits_to_f32(g.sbits);
  if (g.s == 0.0f) {
    g.z = 0;
    g.t1 = g.t2 = g.t3 = __uint_as_float(0x7F800000u);   // +inf: every code 0
    return g;
  }
  int z = rne_quot(-lo, g.s);
  z = z < 0 ? 0 : (z > 3 ? 3 : z);
  g.z = z;
  float t[3];
#pragma unroll
  for (int k = 1; k <= 3; ++k) {
    const float tau = ((float)(k - z) - 0.5f) * g.s;        // exact
    // rne rounds the tie r == tau up to k - z iff k - z is even
    t[k - 1] = (((k - z) & 1) == 0) ? prev_float(tau) : tau;
  }
  g.t1 = t[0]; g.t2 = t[1]; g.t3 = t[2];
  return g;
}

__device__ __forceinline__ uint32_t code_of(float r, const GroupCodec& g) {
  return (uint32_t)(r > g.t1) + (uint32_t)(r > g.t2) + (uint32_t)(r > g.t3);
}

// Per-lane running list of the K smallest packed values (t[0] <= ... <= t[K-1]).
// ninf holds -inf in a register the compiler cannot see through, so that the
// last step stays one v_med3 (a min would first quiet its packed operand).
template <int K>
__device__ __forceinline__ void topk_insert(float (&t)[K], float x, float ninf) {
#pragma unroll
  for (int k = K - 1; k >= 1; --k) t[k] = __builtin_amdgcn_fmed3f(t[k - 1], t[k], x);
  t[0] = __builtin_amdgcn_fmed3f(ninf, t[0], x);
}

__device__ __forceinline__ void cswap(float& x, float& y) {
  const float lo = fminf(x, y), hi = fmaxf(x, y);
  x = lo;
  y = hi;
}

__device__ __forceinline__ float unpacked(float p) { return __uint_as_float(__float_as_uint(p) & 0xFFFFFF00u); }

// Residual statistics of the token against centroid j over the lane's 64
// channels (16 s + 8 hh + e): weighted squared distance and group ranges.
struct ResidStats {
  float d, lo0, hi0, lo1, hi1;
};

// 16-byte chunk c (channels 8c .. 8c+7) of centroid row j in the LDS table.
// Rows are 17 chunks apart: the 16 rows a quarter-wave reads at one chunk
// index fall on distinct bank groups, and a lane's chunk offsets are
// compile-time constants on top of its row base.
__device__ __forceinline__ u32x4 mu_chunk(const uint16_t* tab, int j, int c) {
  return reinterpret_cast<const u32x4*>(tab)[j * (MU_ROW / 8) + c];
}

// Residual statistics of the token kf (the lane's channels 16 s + 8 hh + e at
// kf[8 s + e]) against centroid j of the LDS table.
template <bool WEIGHTED>
__device__ __forceinline__ ResidStats resid_stats(const float (&kf)[64], const uint16_t* tab, int j, int hh,
                                                  const float* wsm) {
  // the weights are re-read from LDS per candidate instead of pinning 64 VGPRs
  asm volatile("" ::: "memory");
  ResidStats o{0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const u32x4 mv = mu_chunk(tab, j, 2 * s + hh);
    f32x4 w0 = {1.f, 1.f, 1.f, 1.f}, w1 = {1.f, 1.f, 1.f, 1.f};
    if (WEIGHTED) {
      w0 = *reinterpret_cast<const f32x4*>(wsm + 16 * s + 8 * hh);
      w1 = *reinterpret_cast<const f32x4*>(wsm + 16 * s + 8 * hh + 4);
    }
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t mw = mv[e >> 1];
      const float m = (e & 1) ? __uint_as_float(mw & 0xFFFF0000u) : __uint_as_float(mw << 16);
      const float r = kf[8 * s + e] - m;
      if (WEIGHTED) o.d = fmaf((e < 4 ? w0[e] : w1[e - 4]) * r, r, o.d);
      else o.d = fmaf(r, r, o.d);
      lo = fminf(lo, r);
      hi = fmaxf(hi, r);
    }
    if (s < 4) { o.lo0 = fminf(o.lo0, lo); o.hi0 = fmaxf(o.hi0, hi); }
    else { o.lo1 = fminf(o.lo1, lo); o.hi1 = fmaxf(o.hi1, hi); }
  }
  o.d = lanepair_sum(o.d);
  o.lo0 = lanepair_min(o.lo0); o.hi0 = lanepair_max(o.hi0);
  o.lo1 = lanepair_min(o.lo1); o.hi1 = lanepair_max(o.hi1);
  return o;
}

// Group ranges alone (the QSAC score S needs no distance): r = fl32(k - mu_j),
// lo/hi per 64-channel group, with the 0 the coded interval always holds.
__device__ __forceinline__ ResidStats resid_ranges(const float (&kf)[64], const uint16_t* tab, int j, int hh) {
  ResidStats o{0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const u32x4 mv = mu_chunk(tab, j, 2 * s + hh);
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t mw = mv[e >> 1];
      const float r0 = kf[8 * s + e] - __uint_as_float(mw << 16);
      const float r1 = kf[8 * s + e + 1] - __uint_as_float(mw & 0xFFFF0000u);
      lo = fminf(fminf(lo, r0), r1);
      hi = fmaxf(fmaxf(hi, r0), r1);
    }
    if (s < 4) { o.lo0 = fminf(o.lo0, lo); o.hi0 = fmaxf(o.hi0, hi); }
    else { o.lo1 = fminf(o.lo1, lo); o.hi1 = fmaxf(o.hi1, hi); }
  }
  o.lo0 = lanepair_min(o.lo0); o.hi0 = lanepair_max(o.hi0);
  o.lo1 = lanepair_min(o.lo1); o.hi1 = lanepair_max(o.hi1);
  return o;
}

constexpr float DREL = 1.0f / 65536.0f;   // relative error bound of the fp32 rescored distance

// QS: QSAC selection (keys with the QSAC flag and M > 1); otherwise nearest.
// WT: Query-weighted distances.
// KQ: GEMM values tracked per lane in QSAC selection (8 for M <= 8, 16 for
//     M <= 16: each lane holds half the centroids, so 2 KQ >= M candidates);
//     256 for M >= 256, where every centroid is a candidate and S is scored
//     for all of them.
//
// The GEMM's A operand is the exact bf16 centroid row mu_j, staged once per
// block in LDS (where the rescoring and the encoder read it too); the B operand
// is the token side t = -2 w (.) k, exact in bf16 for unweighted bf16 tokens and
// otherwise carried as a bf16 pair t_hi + t_lo (two MFMAs per k-step).
// select_range: tiles [t_begin, t_end) of head h (tokens, or entries of the
// head's list for Lloyd's bounded iterations; nlist of them), with the head's
// tables staged first.  Within the range the waves share only the staged
// tables, which they read, and each stages its own tokens' output, so the
// tiles need no block barrier; the range ends with one, so that a block may
// call it again for another head.
template <int MODE, bool F32, bool QS, bool WT, int KQ, bool BND, bool GDYN>
__device__ __forceinline__ void select_range(const SelectArgs a, SelShared& sm, const int h, const int64_t nlist,
                                             const int64_t t_begin, const int64_t t_end) {
  // KQ = 256: QSAC with M >= 256 (every centroid a candidate), scored exhaustively
  constexpr bool EXH = QS && KQ == NC;
  constexpr int KT = (QS && !EXH) ? KQ : 3;   // values tracked per lane (each lane holds half the centroids)
  constexpr bool SPLIT = F32 || WT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hh = lane >> 5, ln = lane & 31;
  const bool use_psac = (MODE == MODE_KEYS) && (a.flags & QWM_PSAC) && a.U != nullptr;
  const bool wlm = (MODE == MODE_ASSIGN) && a.wl != nullptr;

  // ---- stage the centroid rows, B_j, weights and U^T ----
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.mu + (int64_t)h * NC * D);
#pragma unroll 4
    for (int e = tid; e < NC * 16; e += 256) {
      const int j = e >> 4, c = e & 15;
      reinterpret_cast<u32x4*>(sm.mu)[j * (MU_ROW / 8) + c] = src[e];
    }
    const uint2* asrc = reinterpret_cast<const uint2*>(a.aug + (int64_t)h * NC * 4);
    reinterpret_cast<uint2*>(sm.aug)[tid] = asrc[tid];
    sm.bj[tid] = a.Bj[h * NC + tid] * (1.0f + 1.0f / 1048576.0f);   // upper bound of B_j
    if (tid < D) {
      const float wc = a.w ? a.w[h * D + tid] : 1.0f;
      sm.w[tid] = wc;
      sm.wm2[tid] = -2.0f * wc;
    }
    if (use_psac) {
      for (int e = tid; e < D * R; e += 256) sm.ut[e % R][e / R] = a.U[(int64_t)h * D * R + e];
    }
  }
  // block counter of the wave tiles handed out (in the padding of centroid row 0)
  int32_t* next_wt = reinterpret_cast<int32_t*>(sm.mu + D);
  if (tid == 0) *next_wt = 0;
  // GDYN with SEL_HEAD_COUNTERS: every block of the head draws from the head's
  // counter a.counter[4 + h] instead (a large call; a small one keeps fixed
  // block shares)
  int32_t* const gcnt = (GDYN && (a.flags & SEL_HEAD_COUNTERS)) ? a.counter + 4 + h : nullptr;
  __syncthreads();
  float Bmax = a.Bmax[h * PREP_PARTS];
#pragma unroll
  for (int p = 1; p < PREP_PARTS; ++p) Bmax = fmaxf(Bmax, a.Bmax[h * PREP_PARTS + p]);
  const double W0 = a.Wg[2 * h], W1 = a.Wg[2 * h + 1];
  const float cb = a.cb;

  // The block's range is cut into wave tiles of 32 list entries: wave tile u
  // (relative to the range) holds entries 32 (4 t_begin + u) + 0..31.  Wave w
  // starts with u = w; whenever a wave starts a tile it takes the next one from
  // the block counter (plus 4), so waves that finish early take more tiles.
  // With the head's counter (gcnt) the range is the whole head, and every wave
  // of every block on the head takes each of its tiles, the first included,
  // from that counter, so that blocks that get more of their CU take more.
  // nwt: wave tiles that hold at least one entry.
  const int64_t wt0 = 4 * t_begin;
  const int64_t nwt_r = 4 * (t_end - t_begin), nwt_l = (nlist + 31) / 32 - wt0;
  const int64_t nwt = nwt_r < nwt_l ? nwt_r : nwt_l;
  // The token of this lane in wave tile u; ok = false past the range or the list.
  auto lane_token = [&](int64_t u, bool& ok) __attribute__((always_inline)) -> int64_t {
    const int64_t e = (wt0 + u) * 32 + ln;
    ok = u < nwt && e < nlist;
    if (!wlm) return ok ? e : 0;
    return ok ? (int64_t)a.wl[(int64_t)h * a.T + e] : 0;
  };
  // Nearest-centroid modes (Lloyd assignment, values) have registers to spare:
  // each tile issues the next tile's bf16 token rows before its own work, so
  // their HBM latency passes under it.
  constexpr bool PF = !F32 && MODE != MODE_KEYS;
  u32x4 nrow[PF ? 8 : 1];
  auto fetch_rows = [&](int64_t t) __attribute__((always_inline)) {
    bool ok;
    const int64_t tk = lane_token(t, ok);
    const uint16_t* xr = static_cast<const uint16_t*>(a.x) + (int64_t)h * a.sh + tk * a.st;
#pragma unroll
    for (int s = 0; s < (PF ? 8 : 1); ++s)
      nrow[s] = ok ? *reinterpret_cast<const u32x4*>(xr + 16 * s + 8 * hh) : u32x4{0, 0, 0, 0};
  };
  const bool glob = GDYN && gcnt != nullptr;   // block-uniform
  constexpr int GCH = MODE == MODE_KEYS ? 1 : 2;   // wave tiles per draw from the head's counter
  int64_t u = __builtin_amdgcn_readfirstlane(wv);
  int64_t cend = 0;
  if constexpr (GDYN) {
    if (glob) {
      int32_t taken = 0;
      if (lane == 0) taken = atomicAdd(gcnt, 1);
      u = (int64_t)__builtin_amdgcn_readfirstlane(taken) * GCH;
      cend = u + GCH;
    }
  }
  if constexpr (PF) fetch_rows(u);
  while (u < nwt) {
    int32_t taken = 0;
    int64_t un;   // the wave's next tile
    if constexpr (GDYN) {
      if (GCH > 1 && glob && u + 1 < cend) {
        un = u + 1;
      } else {
        if (lane == 0) taken = glob ? atomicAdd(gcnt, 1) : atomicAdd(next_wt, 1);
        un = glob ? (int64_t)__builtin_amdgcn_readfirstlane(taken) * GCH : 4 + (int64_t)__builtin_amdgcn_readfirstlane(taken);
        cend = un + GCH;
      }
    } else {
      if (lane == 0) taken = atomicAdd(next_wt, 1);
      un = 4 + (int64_t)__builtin_amdgcn_readfirstlane(taken);
    }
    const int64_t tok0 = (wt0 + u) * 32;   // first list entry of the wave tile
    bool valid;
    const int64_t tok = lane_token(u, valid);
    const int64_t rowoff = (int64_t)h * a.sh + tok * a.st;

    // ---- the token in fp32: channels 16 s + 8 hh + e at kf[8 s + e] ----
    float kf[64];
    if (!F32) {
      const uint16_t* xr = static_cast<const uint16_t*>(a.x) + rowoff;
      u32x4 crow[PF ? 8 : 1];
      if constexpr (PF) {
#pragma unroll
        for (int s = 0; s < 8; ++s) crow[s] = nrow[s];
        fetch_rows(un);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        u32x4 v;
        if constexpr (PF) v = crow[s];
        else v = valid ? *reinterpret_cast<const u32x4*>(xr + 16 * s + 8 * hh) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          kf[8 * s + e] = (e & 1) ? __uint_as_float(v[e >> 1] & 0xFFFF0000u) : __uint_as_float(v[e >> 1] << 16);
      }
    } else {
      const float* xr = static_cast<const float*>(a.x) + rowoff;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const f32x4 v0 = valid ? *reinterpret_cast<const f32x4*>(xr + 16 * s + 8 * hh) : f32x4{0, 0, 0, 0};
        const f32x4 v1 = valid ? *reinterpret_cast<const f32x4*>(xr + 16 * s + 8 * hh + 4) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) { kf[8 * s + e] = v0[e]; kf[8 * s + 4 + e] = v1[e]; }
      }
    }
    // ---- GEMM B operand t = -2 w (.) k: bf16 t_hi (RNE) and, unless exact, the
    // bf16 t_lo of the remainder t - t_hi (exact in fp32) ----
    // The token norm A = sum_c w_c k_c^2 is gathered on the way as
    // -(1/2) sum_c t_c k_c (t_c = fl32(-2 w_c k_c), one fma per channel).
    bf16x8 th[8], tl[SPLIT ? 8 : 1];
    float An = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 hv, lv;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int c = 16 * s + 8 * hh + 2 * e2;
        const float x0 = kf[8 * s + 2 * e2], x1 = kf[8 * s + 2 * e2 + 1];
        const float t0 = WT ? sm.wm2[c] * x0 : -2.0f * x0;
        const float t1 = WT ? sm.wm2[c + 1] * x1 : -2.0f * x1;
        An = fmaf(t1, x1, fmaf(t0, x0, An));
        hv[e2] = pk_bf16(t0, t1);
        if (SPLIT) lv[e2] = pk_bf16(t0 - lo_bf16(hv[e2]), t1 - hi_bf16(hv[e2]));
      }
      th[s] = __builtin_bit_cast(bf16x8, hv);
      if (SPLIT) tl[SPLIT ? s : 0] = __builtin_bit_cast(bf16x8, lv);
    }
    bf16x8 kaug;
    {
      u32x4 v = {0, 0, 0, 0};
      if (hh == 0) { v[0] = 0x3F803F80u; v[1] = 0x3F80u; }   // (1, 1, 1, 0, ...)
      kaug = __builtin_bit_cast(bf16x8, v);
    }

    // ---- distance GEMM; each lane keeps its KT smallest (value | index) ----
    float t[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) t[k] = __builtin_inff();
    float ninf;
    asm volatile("v_mov_b32 %0, 0xff800000" : "=v"(ninf));
    // centroid indices of the lane's 16 values, four to a word: byte b of
    // jb0 + 8 q 0x01010101 is 32 ct + c_row(4 q + b, hh)
    uint32_t jb0 = (uint32_t)(4 * hh) * 0x01010101u + 0x03020100u;
#pragma unroll 1
    for (int ct = 0; ct < 8; ++ct) {
      f32x16 acc = {};
      const int j = 32 * ct + ln;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 af = __builtin_bit_cast(bf16x8, mu_chunk(sm.mu, j, 2 * s + hh));
        acc = mfma_bf16(af, th[s], acc);
        if (SPLIT) acc = mfma_bf16(af, tl[SPLIT ? s : 0], acc);
      }
      {
        u32x4 v = {0, 0, 0, 0};
        if (hh == 0) { const uint2 g = reinterpret_cast<const uint2*>(sm.aug)[j]; v[0] = g.x; v[1] = g.y; }
        acc = mfma_bf16(__builtin_bit_cast(bf16x8, v), kaug, acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) topk_insert<KT>(t, pack_idx(acc[i], jb0 + (uint32_t)(8 * (i >> 2)) * 0x01010101u, i & 3), ninf);
      jb0 += 32u * 0x01010101u;
    }
    // canonical per-token list: g[0..KT) = half 0, g[KT..2KT) = half 1 (identical on both lanes)
    float g[2 * KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const float o = lanepair_other(t[k], hh);
      g[k] = hh ? o : t[k];
      g[KT + k] = hh ? t[k] : o;
    }
    const float floor_unt = fminf(unpacked(g[KT - 1]), unpacked(g[2 * KT - 1]));   // every untracked value is >= this
    if (QS && !EXH) {
      // one ascending list of the 2 KT tracked values: half 1 reversed makes the
      // sequence bitonic; four half-cleaner stages sort it
#pragma unroll
      for (int k = 0; k < KT / 2; ++k) {
        const float x = g[KT + k];
        g[KT + k] = g[2 * KT - 1 - k];
        g[2 * KT - 1 - k] = x;
      }
#pragma unroll
      for (int d = KT; d >= 1; d >>= 1)
#pragma unroll
        for (int i = 0; i < 2 * KT; ++i)
          if ((i & d) == 0) cswap(g[i], g[i + d]);
    }
    float gmin = g[0];
    if ((!QS || EXH) && g[KT] < gmin) gmin = g[KT];

    // ---- token norm A = sum_c w_c k_c^2 ----
    const float A = lanepair_sum(-0.5f * An);
    const float A_hi = A * (1.0f + 1.0f / 32768.0f), A_lo = A * (1.0f - 1.0f / 32768.0f);
    // certified bounds on d_Q(j) = A + e_j from the GEMM value f_j:
    //   [lbA + f_j - cb B_j, ubA + f_j + cb B_j]
    const float lbA = A_lo * (1.0f - cb), ubA = A_hi * (1.0f + cb);
    const float L_unt = lbA + floor_unt - cb * Bmax;
#define QWM_LB(pv) (lbA + unpacked(pv) - cb * sm.bj[__float_as_uint(pv) & 0xFFu])
#define QWM_UB(pv) (ubA + unpacked(pv) + cb * sm.bj[__float_as_uint(pv) & 0xFFu])

    // |f_j| <= A + 2 B_j: with this bound finite no GEMM value (or partial sum) overflows
    bool fast = valid && __builtin_isfinite(gmin) && __builtin_isfinite(A) &&
                __builtin_isfinite(2.0f * (ubA + 2.0f * Bmax));
    int win = (int)(__float_as_uint(gmin) & 0xFFu);
    float wlo0 = 0.f, whi0 = 0.f, wlo1 = 0.f, whi1 = 0.f;   // group ranges of the winner
    bool have_w = false;                                   // ranges known for the winner
    float bu2 = 0.f, bl2 = 0.f;   // Lloyd: squared distance bounds, the winner's (upper) and every other's (lower)

    if (!QS) {
      // nearest centroid (weighted when QSAC runs with M == 1)
      float c0 = g[0], c1 = g[1], c2 = g[2], c3 = g[KT], c4 = g[KT + 1], c5 = g[KT + 2];
      cswap(c0, c3); cswap(c1, c4); cswap(c2, c5);
      cswap(c1, c3); cswap(c2, c4);
      cswap(c2, c3);
      cswap(c3, c4);
      cswap(c4, c5);
      cswap(c3, c4);
      const float ub0 = QWM_UB(c0);
      const bool by_bounds = (QWM_LB(c1) > ub0) && (QWM_LB(c2) > ub0) && (QWM_LB(c3) > ub0) &&
                             (QWM_LB(c4) > ub0) && (QWM_LB(c5) > ub0) && (L_unt > ub0);
      float d1 = __builtin_inff();   // smallest rescored distance
      const float cn[6] = {c0, c1, c2, c3, c4, c5};
      float dn[6];
      uint32_t evm = 0;
#pragma unroll
      for (int e = 0; e < 6; ++e) {
        dn[e] = 0.f;
        const bool need = fast && !by_bounds && (QWM_LB(cn[e]) <= d1 * (1.0f + DREL));
        if (!__any(need)) continue;
        const int j = (int)(__float_as_uint(cn[e]) & 0xFFu);
        const ResidStats rs = resid_stats<WT>(kf, sm.mu, j, hh, sm.w);
        if (need) {
          evm |= 1u << e;
          dn[e] = rs.d;
          if (!have_w || rs.d < d1 || (rs.d == d1 && j < win)) {
            d1 = rs.d; win = j;
            wlo0 = rs.lo0; whi0 = rs.hi0; wlo1 = rs.lo1; whi1 = rs.hi1; have_w = true;
          }
        }
      }
      if (fast && !by_bounds) {
        // every other tracked centroid (rescored or not) and every untracked one
        // must stay strictly above the winner
        const float hi1 = d1 * (1.0f + DREL);
        bool ok = have_w && (L_unt > hi1);
#pragma unroll
        for (int e = 0; e < 6; ++e) {
          const int j = (int)(__float_as_uint(cn[e]) & 0xFFu);
          const float lo = ((evm >> e) & 1u) ? dn[e] * (1.0f - DREL) : QWM_LB(cn[e]);
          ok = ok && (j == win || lo > hi1);
        }
        fast = ok;
      }
      if (MODE == MODE_ASSIGN && BND) {
        float l2 = L_unt;
#pragma unroll
        for (int e = 0; e < 6; ++e) {
          const int j = (int)(__float_as_uint(cn[e]) & 0xFFu);
          const float lo = ((evm >> e) & 1u) ? dn[e] * (1.0f - DREL) : QWM_LB(cn[e]);
          if (j != win) l2 = fminf(l2, lo);
        }
        bu2 = by_bounds ? ub0 : d1 * (1.0f + DREL);
        bl2 = l2;
      }
    } else if constexpr (EXH) {
      // QSAC with every centroid a candidate (M >= 256): the choice is the smallest (S, j)
      // over all of them, S from exact fp32 group ranges (nothing to certify)
      double Sbest = __builtin_inf();
#pragma unroll 1
      for (int j = 0; j < NC; ++j) {
        const ResidStats rs = resid_ranges(kf, sm.mu, j, hh);
        const double R0 = (double)rs.hi0 - (double)rs.lo0, R1 = (double)rs.hi1 - (double)rs.lo1;
        const double S = W0 * R0 * R0 + W1 * R1 * R1;
        if (!have_w || S < Sbest || (S == Sbest && j < win)) {
          Sbest = S; win = j;
          wlo0 = rs.lo0; whi0 = rs.hi0; wlo1 = rs.lo1; whi1 = rs.hi1; have_w = true;
        }
      }
      fast = fast && __builtin_isfinite(Sbest);
    } else {
      // QSAC.  Tracked candidate k is certainly outside the M nearest when M other
      // values are certainly smaller; the untracked ones must all be outside too.
      // Lb[k] is a lower bound on d_Q of slot k (raised to the rescored value once
      // the slot is scored); jp packs the slot's centroid index, four per word.
      // vectors, so that the scan below reads slot `it` by register indexing
      typedef float lbvec __attribute__((ext_vector_type(2 * KT)));
      typedef uint32_t jpvec __attribute__((ext_vector_type(2 * KT / 4)));
      lbvec Lb;
      jpvec jp;
      uint32_t outmask = 0;
      bool unt_out;
      {
        // UbM = the largest upper bound among the first M slots: M tracked
        // centroids certainly lie at or below it, so slot k is out when
        // Lb[k] > UbM, and every untracked centroid (d_Q >= L_unt) when
        // L_unt > UbM.  (The slots are in GEMM-value order, so UbM is the M-th
        // smallest upper bound up to the c B_j terms.)
        float UbM = a.M > 2 * KT ? __builtin_inff() : -__builtin_inff();   // M > 2 KT: no slot is out
#pragma unroll
        for (int k = 0; k < 2 * KT; ++k) {
          Lb[k] = QWM_LB(g[k]);
          if (k < a.M) UbM = fmaxf(UbM, QWM_UB(g[k]));
        }
#pragma unroll
        for (int q = 0; q < 2 * KT / 4; ++q) {
          uint32_t v = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) v |= (__float_as_uint(g[4 * q + e]) & 0xFFu) << (8 * e);
          jp[q] = v;
        }
#pragma unroll
        for (int k = 0; k < 2 * KT; ++k) outmask |= (Lb[k] > UbM ? 1u : 0u) << k;
        unt_out = L_unt > UbM;   // untracked centroids are all outside the M nearest
      }
      // score S for every possible member in ascending order of the GEMM value,
      // skipping candidates whose distance bound already exceeds the best S (S >= d_Q).
      // S needs only the group ranges; the winner's exact distance is taken once,
      // after the scan, for the membership test.
      double Sbest = __builtin_inf();
      float dwin = 0.f;
      // one slot per pass (`it` is wave-uniform: slot it is read by register indexing)
#pragma unroll 1
      for (int it = 0; it < 2 * KT; ++it) {
        const bool need = fast && !((outmask >> it) & 1u) && ((double)Lb[it] <= Sbest * (1.0 + 1.0 / 1048576.0));
        if (__any(need)) {
          const int j = (int)((jp[it >> 2] >> (8 * (it & 3))) & 0xFFu);
          const ResidStats rs = resid_ranges(kf, sm.mu, j, hh);
          if (need) {
            const double R0 = (double)rs.hi0 - (double)rs.lo0, R1 = (double)rs.hi1 - (double)rs.lo1;
            const double S = W0 * R0 * R0 + W1 * R1 * R1;
            if (!have_w || S < Sbest || (S == Sbest && j < win)) {
              Sbest = S; win = j;
              wlo0 = rs.lo0; whi0 = rs.hi0; wlo1 = rs.lo1; whi1 = rs.hi1; have_w = true;
            }
          }
        }
      }
      if (__any(fast)) {
        const ResidStats rw = resid_stats<WT>(kf, sm.mu, win, hh, sm.w);
        dwin = rw.d;
      }
      if (fast) {
        // the winner must be among the M nearest: count every centroid that may precede it
        const float dwin_hi = dwin * (1.0f + DREL);
        int before = 0;
#pragma unroll
        for (int k = 0; k < 2 * KT; ++k) {
          const int j = (int)((jp[k >> 2] >> (8 * (k & 3))) & 0xFFu);
          before += (j != win && Lb[k] <= dwin_hi) ? 1 : 0;
        }
        // untracked centroids either lie outside the M nearest or cannot beat the best S (S >= d_Q)
        const bool unt_ok = unt_out || ((double)L_unt > Sbest * (1.0 + 1.0 / 1048576.0));
        fast = have_w && __builtin_isfinite(Sbest) && unt_ok && (L_unt > dwin_hi) && (before <= a.M - 1);
      }
    }

    if (MODE == MODE_ASSIGN) {
      if (valid && hh == 0) {
        sm.l.tok[wv][ln] = (int32_t)tok;
        sm.l.fast[wv][ln] = fast ? 1 : 0;
        if (fast) {
          sm.idx[wv][ln] = (uint8_t)win;
          if (BND) {   // Euclidean distance bounds, rounded outward
            sm.l.ub[wv][ln] = sqrtf(bu2) * (1.0f + 1.0f / 1048576.0f);
            sm.l.lb[wv][ln] = sqrtf(fmaxf(bl2, 0.f)) * (1.0f - 1.0f / 1048576.0f);
          }
        } else {
          const int slot = atomicAdd(a.counter, 1);
          a.worklist[slot] = (int32_t)((int64_t)h * a.T + tok);
          sm.idx[wv][ln] = 0;
        }
      }
    } else {
      // ---- ranges of the winner (when the choice came from bounds alone) ----
      if (__any(!have_w)) {
        const ResidStats rs = resid_stats<WT>(kf, sm.mu, win, hh, sm.w);
        if (!have_w) { wlo0 = rs.lo0; whi0 = rs.hi0; wlo1 = rs.lo1; whi1 = rs.hi1; }
      }
      bool sat0 = false, sat1 = false;
      const GroupCodec g0 = make_codec(wlo0, whi0, &sat0);
      const GroupCodec g1 = make_codec(wlo1, whi1, &sat1);
      // codes, and PSAC's E = r - r_hat (exact in fp32) fed straight into C = E U on
      // MFMA (A = U^T, rows 0..7 valid; B = E split into three bf16 parts)
      f32x16 pacc = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const GroupCodec& g = s < 4 ? g0 : g1;
        const u32x4 mv = mu_chunk(sm.mu, win, 2 * s + hh);
        uint32_t bits = 0;
        float Ev[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t mwd = mv[e >> 1];
          const float m = (e & 1) ? __uint_as_float(mwd & 0xFFFF0000u) : __uint_as_float(mwd << 16);
          const float r = kf[8 * s + e] - m;
          const uint32_t q = code_of(r, g);
          bits |= q << (2 * e);
          Ev[e] = r - g.s * ((float)q - (float)g.z);
          if (F32 && use_psac) {
            // add the rounding error of r = fl32(k - mu) (TwoSum) so that E = k - mu - r_hat
            const float x = kf[8 * s + e];
            const float bv = r - x;
            Ev[e] += (x - (r - bv)) + (-m - bv);
          }
        }
        if (valid) *reinterpret_cast<uint16_t*>(&sm.k.codes[wv][ln][4 * s + 2 * hh]) = (uint16_t)bits;
        if (use_psac) {
          bf16x8 uf;
          if (ln < R) uf = *reinterpret_cast<const bf16x8*>(&sm.ut[ln][16 * s + 8 * hh]);
          else uf = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
          // E = b0 + b1 + b2 exactly: each part is the RNE bf16 of the remainder
          // left by the previous ones (the remainders are exact in fp32)
          u32x4 p0, p1, p2;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float ev0 = Ev[2 * e2], ev1 = Ev[2 * e2 + 1];
            p0[e2] = pk_bf16(ev0, ev1);
            const float r0 = ev0 - lo_bf16(p0[e2]), r1 = ev1 - hi_bf16(p0[e2]);
            p1[e2] = pk_bf16(r0, r1);
            p2[e2] = pk_bf16(r0 - lo_bf16(p1[e2]), r1 - hi_bf16(p1[e2]));
          }
          pacc = mfma_bf16(uf, __builtin_bit_cast(bf16x8, p0), pacc);
          pacc = mfma_bf16(uf, __builtin_bit_cast(bf16x8, p1), pacc);
          pacc = mfma_bf16(uf, __builtin_bit_cast(bf16x8, p2), pacc);
        }
      }
      if (valid && hh == 0) {
        if (fast) {
          sm.idx[wv][ln] = (uint8_t)win;
          sm.k.scale[wv][ln][0] = (uint16_t)g0.sbits;
          sm.k.scale[wv][ln][1] = (uint16_t)g1.sbits;
          sm.k.nib[wv][ln] = (uint8_t)(g0.z | (g1.z << 2));
          if ((sat0 || sat1) && a.diag) atomicAdd((unsigned long long*)&a.diag->scale_saturations,
                                                  (unsigned long long)((int)sat0 + (int)sat1));
        } else {
          const int slot = atomicAdd(a.counter, 1);
          a.worklist[slot] = (int32_t)((int64_t)h * a.T + tok);
          sm.idx[wv][ln] = 0;
          sm.k.nib[wv][ln] = 0;
          sm.k.scale[wv][ln][0] = 0;
          sm.k.scale[wv][ln][1] = 0;
        }
      }
      if (MODE == MODE_KEYS) {
        if (use_psac) {
          const f32x16 acc = pacc;
          // lane (token, hh) holds C[4 hh + 0..3] in acc[0..3]
          float m = fmaxf(fmaxf(fabsf(acc[0]), fabsf(acc[1])), fmaxf(fabsf(acc[2]), fabsf(acc[3])));
          m = lanepair_max(m);
          bool sat = false;
          uint32_t csb = fp16_up_div((double)m, 127.0f, &sat);
          if (sat && fast && valid && hh == 0 && a.diag)
            atomicAdd((unsigned long long*)&a.diag->scale_saturations, 1ull);
          const float cs = f16_bits_to_f32(csb);
          uint32_t packed = 0;
          float chat[4];   // c_s C_q of this lane's four coefficients
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            int qi = 0;
            if (cs > 0.f) {
              qi = rne_quot(acc[i], cs);
              qi = qi < -127 ? -127 : (qi > 127 ? 127 : qi);
            }
            packed |= ((uint32_t)(uint8_t)(int8_t)qi) << (8 * i);
            chat[i] = cs * (float)qi;   // exact (11 + 8 significant bits)
          }
          if (a.flags & QWM_PSAC_KEEP) {
            // Keep test (QuantWM method step (4)): the coefficients stay only if the
            // compensation D = (c_s C_q) U^T lowers the key's Query-weighted error
            // sum_c w_c e_c^2, i.e. iff sum_c w_c D_c (D_c - 2 E_c) < 0; E is
            // recomputed from the codes just written, the weights are those of
            // the centroid choice.
            float cr[R];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float o = lanepair_other(chat[i], hh);
              cr[i] = hh ? o : chat[i];
              cr[4 + i] = hh ? chat[i] : o;
            }
            float crit = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const GroupCodec& g = s < 4 ? g0 : g1;
              const u32x4 mv = mu_chunk(sm.mu, win, 2 * s + hh);
              u32x4 ur[R];
#pragma unroll
              for (int r2 = 0; r2 < R; ++r2) ur[r2] = *reinterpret_cast<const u32x4*>(&sm.ut[r2][16 * s + 8 * hh]);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t mwd = mv[e >> 1];
                const float mu = (e & 1) ? __uint_as_float(mwd & 0xFFFF0000u) : __uint_as_float(mwd << 16);
                const float x = kf[8 * s + e];
                const float r = x - mu;
                const uint32_t q = code_of(r, g);
                float E = r - g.s * ((float)q - (float)g.z);
                if (F32) {
                  const float bv = r - x;
                  E += (x - (r - bv)) + (-mu - bv);
                }
                float Dc = 0.f;
#pragma unroll
                for (int r2 = 0; r2 < R; ++r2) {
                  const uint32_t uw = ur[r2][e >> 1];
                  const float u = (e & 1) ? __uint_as_float(uw & 0xFFFF0000u) : __uint_as_float(uw << 16);
                  Dc = fmaf(cr[r2], u, Dc);
                }
                crit = fmaf(sm.w[16 * s + 8 * hh + e] * Dc, Dc - 2.0f * E, crit);
              }
            }
            crit = lanepair_sum(crit);
            if (!(crit < 0.f)) { packed = 0u; csb = 0u; }
          }
          if (valid) {
            *reinterpret_cast<uint32_t*>(&sm.k.cq[wv][ln][4 * hh]) = packed;
            if (hh == 0) sm.k.cs[wv][ln] = (uint16_t)csb;
          }
        } else if (valid) {
          *reinterpret_cast<uint32_t*>(&sm.k.cq[wv][ln][4 * hh]) = 0u;
          if (hh == 0) sm.k.cs[wv][ln] = 0;
        }
      }
    }
    // the staging rows are the wave's own: a wave-level barrier orders them
    wave_lds_sync();

    // ---- coalesced write-out of the wave's 32 tokens ----
    if (MODE == MODE_ASSIGN) {
      const int64_t left = nlist - tok0;
      const int nv = (int)(left < 32 ? (left > 0 ? left : 0) : 32);   // list entries of this wave
      const bool live = lane < nv;
      const int64_t o = (int64_t)h * a.T + (live ? (wlm ? (int64_t)sm.l.tok[wv][lane] : tok0 + lane) : 0);
      const bool certified = live && sm.l.fast[wv][lane];
      const uint32_t nw = live ? sm.idx[wv][lane] : 0u;
      const uint32_t old = (wlm && certified) ? a.idx[o] : nw;
      // changed assignments: one atomic per wave reserves their records
      const uint64_t cm = __ballot(old != nw);
      if (cm) {
        const int leader = __ffsll((long long)cm) - 1;
        int base = 0;
        if (lane == leader) base = atomicAdd(a.chg_cnt, __popcll(cm));
        base = __shfl(base, leader, 64);
        if (old != nw) a.chg[base + __popcll(cm & ((1ull << lane) - 1ull))] = make_uint2((uint32_t)o, old | (nw << 8));
      }
      if (certified) {
        a.idx[o] = (uint8_t)nw;
        if (BND) {
          a.ub[o] = sm.l.ub[wv][lane];
          a.lb[o] = sm.l.lb[wv][lane];
        }
      } else if (live && !wlm) {
        a.idx[o] = 0;   // the exact path fills it in
      }
    } else {
      const int64_t base = (int64_t)h * a.T + tok0;
      const int nv = (int)((a.T - tok0) < 32 ? (a.T - tok0) : 32);   // tokens of this wave
      if (nv > 0) {
        if (lane < nv) a.idx[base + lane] = sm.idx[wv][lane];
        {
          {
            const int t = lane >> 1, part = lane & 1;
            if (t < nv)
              *reinterpret_cast<u32x4*>(a.codes + (base + t) * 32 + 16 * part) =
                  *reinterpret_cast<const u32x4*>(&sm.k.codes[wv][t][16 * part]);
          }
          if (lane < nv)
            *reinterpret_cast<uint32_t*>(a.scale + (base + lane) * 2) =
                *reinterpret_cast<const uint32_t*>(&sm.k.scale[wv][lane][0]);
          if (2 * lane < nv) {
            const uint8_t lo = sm.k.nib[wv][2 * lane];
            const uint8_t hi = (2 * lane + 1 < nv) ? sm.k.nib[wv][2 * lane + 1] : 0;
            a.zeros[(int64_t)h * a.zstride + (tok0 >> 1) + lane] = (uint8_t)(lo | (hi << 4));
          }
          if (MODE == MODE_KEYS && a.cq != nullptr) {   // null: a later pass writes the coefficients
            if (lane < nv) {
              *reinterpret_cast<uint2*>(a.cq + (base + lane) * R) = *reinterpret_cast<const uint2*>(&sm.k.cq[wv][lane][0]);
              a.cscale[base + lane] = sm.k.cs[wv][lane];
            }
          }
        }
      }
    }
    wave_lds_sync();   // before the next tile's staging writes
    u = un;
  }
  __syncthreads();     // the block may stage another head's tables next
}

// Keys and values: the grid is one-dimensional.  Block b serves head b mod H;
// a head's blocks take its 32-token wave tiles from the head's counter
// a.counter[4 + h] (one tile per draw for keys, two for values), so that
// blocks that get more of their CU (a CU runs the block that arrived first
// ahead of its later partner) take more tiles.  The full Lloyd assignment:
// block (x, h) takes a fixed share of head h's tiles (its tiles are cheap, and
// the counter's atomics cost more than the balance gains).  FLAT (Lloyd's bounded
// iterations): all heads' lists, taken one after the other, form NT tiles,
// and block b takes tiles [b NT / G, (b + 1) NT / G) of them (G blocks), head by
// head, so that a short or uneven list still spreads over the whole grid.
// BND (Lloyd assignment): the distance bounds are written (a.ub, a.lb).
// Every variant runs two blocks per CU (the LDS allows two), KQ = 16 too: it
// would need about 320 registers per lane and spills instead, which still
// beats one wave per SIMD.
template <int MODE, bool F32, bool QS, bool WT, int KQ = 8, bool FLAT = false, bool BND = false>
__global__ __launch_bounds__(256, 2) void select_kernel(SelectArgs a) {
  __shared__ SelShared sm;
  if constexpr (FLAT) {
    int64_t nt = 0;
    for (int g = 0; g < a.H; ++g) nt += ((int64_t)a.wl_cnt[g] + SEL_TOK - 1) / SEL_TOK;
    const int64_t r0 = (int64_t)blockIdx.x * nt / gridDim.x;
    const int64_t r1 = (int64_t)(blockIdx.x + 1) * nt / gridDim.x;
    int64_t lo = 0;   // first tile of head g
    for (int g = 0; g < a.H && lo < r1; ++g) {
      const int64_t n = a.wl_cnt[g];
      const int64_t hi = lo + (n + SEL_TOK - 1) / SEL_TOK;
      if (hi > r0 && hi > lo)
        select_range<MODE, F32, QS, WT, KQ, BND, false>(a, sm, g, n, (lo > r0 ? lo : r0) - lo, (hi < r1 ? hi : r1) - lo);
      lo = hi;
    }
  } else if constexpr (MODE == MODE_KEYS || MODE == MODE_VALUES) {
    // one-dimensional grid, heads interleaved (block b serves head b mod H), so
    // that each head has blocks of every dispatch round; with SEL_HEAD_COUNTERS the blocks
    // of a head take its wave tiles from the head's counter, otherwise block
    // b / H of the head a fixed share of its tiles
    const int h = (int)(blockIdx.x % (unsigned)a.H);
    const int64_t ntile = (a.T + SEL_TOK - 1) / SEL_TOK;
    int64_t t_begin = 0, t_end = ntile;
    if (!(a.flags & SEL_HEAD_COUNTERS)) {
      const int64_t bph = gridDim.x / (unsigned)a.H, j = blockIdx.x / (unsigned)a.H;
      t_begin = j * ntile / bph;
      t_end = (j + 1) * ntile / bph;
    }
    if (t_begin >= t_end) return;   // block-uniform
    select_range<MODE, F32, QS, WT, KQ, BND, true>(a, sm, h, a.T, t_begin, t_end);
  } else {
    // block (x, h): a contiguous share of head h's tiles, equal to within one
    // tile across the head's gridDim.x blocks (the full Lloyd assignment)
    const int h = blockIdx.y;
    const int64_t ntile = (a.T + SEL_TOK - 1) / SEL_TOK;
    const int64_t t_begin = (int64_t)blockIdx.x * ntile / gridDim.x;
    const int64_t t_end = (int64_t)(blockIdx.x + 1) * ntile / gridDim.x;
    if (t_begin >= t_end) return;   // block-uniform
    select_range<MODE, F32, QS, WT, KQ, BND, false>(a, sm, h, a.T, t_begin, t_end);
  }
}

// ---------------------------------------------------------------------------
// Exact path for the tokens the fast path did not certify: plain fp64 scoring
// of all centroids, one wave per token.
// ---------------------------------------------------------------------------
// FULL: the full-matrix ablation of QSAC (QuantWM App. C.4): every token of
// head blockIdx.y (no worklist), candidates by the quadratic form
// (k - mu)^T S (k - mu) with S the head's Query second-moment sum (the
// positive factor 1 / n does not change the order; S = I before any Query),
// expanded as k^T S k - 2 (S k) . mu + mu^T S mu with the last term from
// fullq_bj_kernel; S sits in LDS for the whole block.
template <int MODE, bool F32, bool FULL = false>
__global__ __launch_bounds__(256) void fallback_kernel(SelectArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __shared__ double kx[4][D];
  __shared__ double wx[4][D];
  __shared__ double dq[4][NC];
  __shared__ uint8_t cand[4][NC];          // the M candidates in (d, j) order
  __shared__ double sq[FULL ? D * D : 1];   // S [c][r]
  __shared__ double tq[FULL ? 4 : 1][D];    // S k
  int count;
  if constexpr (FULL) {
    const int hb = blockIdx.y;
    const bool cold = a.qn[hb] <= 0;
    const double* Sh = a.qS + (int64_t)hb * D * D;
    for (int e = tid; e < D * D; e += 256) sq[e] = cold ? ((e / D == e % D) ? 1.0 : 0.0) : Sh[e];
    __syncthreads();
    count = (int)a.T;
  } else {
    count = *a.counter;
    if (blockIdx.x == 0 && tid == 0 && a.diag && count > 0)
      atomicAdd((unsigned long long*)&a.diag->exact_fallbacks, (unsigned long long)count);
  }
  const bool use_qsac = (MODE == MODE_KEYS) && (a.flags & QWM_QSAC);
  const bool use_psac = (MODE == MODE_KEYS) && (a.flags & QWM_PSAC) && a.U != nullptr;
  for (int item = blockIdx.x * 4 + wv; item < count; item += gridDim.x * 4) {
    const int64_t id = FULL ? (int64_t)blockIdx.y * a.T + item : (int64_t)a.worklist[item];
    const int h = (int)(id / a.T);
    const int64_t tok = id % a.T;
    const int64_t rowoff = (int64_t)h * a.sh + tok * a.st;
    // token row, 2 channels per lane
    double x0, x1;
    if (F32) {
      const float* xr = static_cast<const float*>(a.x) + rowoff;
      x0 = xr[2 * lane]; x1 = xr[2 * lane + 1];
    } else {
      const uint16_t* xr = static_cast<const uint16_t*>(a.x) + rowoff;
      x0 = bf16_bits_to_f32(xr[2 * lane]); x1 = bf16_bits_to_f32(xr[2 * lane + 1]);
    }
    const int bad = __any(!(__builtin_isfinite(x0) && __builtin_isfinite(x1)));
    const int64_t base = (int64_t)h * a.T + tok;
    if (bad) {
      if (MODE != MODE_ASSIGN) {
        if (lane < 8) *reinterpret_cast<uint32_t*>(a.codes + base * 32 + 4 * lane) = 0u;
        if (lane == 0) {
          a.idx[base] = 0;
          a.scale[base * 2] = 0; a.scale[base * 2 + 1] = 0;
          if (MODE == MODE_KEYS && a.cq != nullptr) {
            *reinterpret_cast<uint2*>(a.cq + base * R) = make_uint2(0u, 0u);
            a.cscale[base] = 0;
          }
          if (a.diag) atomicAdd((unsigned long long*)&a.diag->nonfinite_rows, 1ull);
        }
      } else if (lane == 0) {
        a.idx[base] = 0;
        // counted once per build: when its exclusion bit is first set
        const uint32_t bit = 1u << (tok & 31);
        const uint32_t was = a.excl ? atomicOr(a.excl + (int64_t)h * a.excl_words + (tok >> 5), bit) : 0u;
        if (a.diag && !(was & bit)) atomicAdd((unsigned long long*)&a.diag->nonfinite_rows, 1ull);
      }
      continue;
    }
    kx[wv][2 * lane] = x0;
    kx[wv][2 * lane + 1] = x1;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const bool wts = use_qsac && a.w != nullptr;
    wx[wv][2 * lane] = wts ? (double)a.w[h * D + 2 * lane] : 1.0;
    wx[wv][2 * lane + 1] = wts ? (double)a.w[h * D + 2 * lane + 1] : 1.0;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if constexpr (FULL) {
      // t = S k (S symmetric: lane r reads column entries S[c][r], conflict-free)
      double t0 = 0.0, t1 = 0.0;
      for (int c = 0; c < D; ++c) {
        const double kc = kx[wv][c];
        t0 = fma(sq[c * D + lane], kc, t0);
        t1 = fma(sq[c * D + lane + 64], kc, t1);
      }
      tq[wv][lane] = t0;
      tq[wv][lane + 64] = t1;
      const double kSk = wave_sum_d(kx[wv][lane] * t0 + kx[wv][lane + 64] * t1);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const u32x4* mrow = reinterpret_cast<const u32x4*>(a.mu + ((int64_t)h * NC + lane) * D);
      double s[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
      for (int c8 = 0; c8 < D / 8; ++c8) {
        double tt[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tt[e] = tq[wv][8 * c8 + e];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 v = mrow[q * 64 * (D / 8) + c8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t wd = v[e >> 1];
            const double m = (double)((e & 1) ? __uint_as_float(wd & 0xFFFF0000u) : __uint_as_float(wd << 16));
            s[q] = fma(tt[e], m, s[q]);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) dq[wv][lane + 64 * q] = kSk - 2.0 * s[q] + a.qB[h * NC + lane + 64 * q];
    } else {
    // d_Q for centroids lane + 64 q, direct form in fp64.  Channels outer (one
    // 8-channel slice of k and w at a time), the four centroids inner, so the
    // token never has to live in registers as a whole.
      const u32x4* mrow = reinterpret_cast<const u32x4*>(a.mu + ((int64_t)h * NC + lane) * D);
      double s[4] = {0.0, 0.0, 0.0, 0.0};
      // four channel slices per round trip: 16 table loads in flight
#pragma unroll 4
      for (int c8 = 0; c8 < D / 8; ++c8) {
        double kk[8], ww[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { kk[e] = kx[wv][8 * c8 + e]; ww[e] = wx[wv][8 * c8 + e]; }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 v = mrow[q * 64 * (D / 8) + c8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t wd = v[e >> 1];
            const double m = (double)((e & 1) ? __uint_as_float(wd & 0xFFFF0000u) : __uint_as_float(wd << 16));
            const double df = kk[e] - m;
            s[q] = fma(ww[e] * df, df, s[q]);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) dq[wv][lane + 64 * q] = s[q];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    int win = 0;
    double dwin = 0.0;   // the winner's exact squared distance (nearest-centroid choice)
    if (!use_qsac) {
      double bv = dq[wv][lane];
      int bj = lane;
      for (int q = 1; q < 4; ++q) {
        const double v = dq[wv][lane + 64 * q];
        if (v < bv) { bv = v; bj = lane + 64 * q; }
      }
      for (int o = 32; o > 0; o >>= 1) {
        const double ov = __shfl_xor(bv, o, 64);
        const int oj = __shfl_xor(bj, o, 64);
        if (ov < bv || (ov == bv && oj < bj)) { bv = ov; bj = oj; }
      }
      win = bj;
      dwin = bv;
    } else {
      const double Wa = a.Wg[2 * h], Wb = a.Wg[2 * h + 1];
      double bestS = __builtin_inf();
      int bestj = 0;
      // M rounds of (d_Q, j) selection (LDS and shuffles only); with M >= n_c
      // every centroid is a candidate and there is nothing to select ...
      int nc = 0;
      if (a.M >= NC) {
#pragma unroll
        for (int q = 0; q < 4; ++q) cand[wv][lane + 64 * q] = (uint8_t)(lane + 64 * q);
        nc = NC;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      }
      for (int m = 0; m < (a.M >= NC ? 0 : a.M); ++m) {
        double bv = __builtin_inf();
        int bj = NC;
        for (int q = 0; q < 4; ++q) {
          const int j = lane + 64 * q;
          const double v = dq[wv][j];
          if (v < bv || (v == bv && j < bj)) { bv = v; bj = j; }
        }
        for (int o = 32; o > 0; o >>= 1) {
          const double ov = __shfl_xor(bv, o, 64);
          const int oj = __shfl_xor(bj, o, 64);
          if (ov < bv || (ov == bv && oj < bj)) { bv = ov; bj = oj; }
        }
        if (bj >= NC) break;
        // remove it from the pool, record it
        if (lane == (bj & 63)) dq[wv][bj] = __builtin_inf();
        if (lane == 0) cand[wv][nc] = (uint8_t)bj;
        ++nc;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      }
      // ... then S for the candidates, eight at a time with their centroid rows
      // loaded together (the choice by (S, j) does not depend on the order);
      // lanes 0..31 group 0, 32..63 group 1
      for (int m0 = 0; m0 < nc; m0 += 8) {
        uint32_t mw[8];
        int jj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          jj[u] = cand[wv][m0 + u < nc ? m0 + u : m0];
          mw[u] = *reinterpret_cast<const uint32_t*>(a.mu + ((int64_t)h * NC + jj[u]) * D + 2 * lane);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (m0 + u >= nc) break;
          const float r0 = (float)x0 - __uint_as_float(mw[u] << 16);
          const float r1 = (float)x1 - __uint_as_float(mw[u] & 0xFFFF0000u);
          float rlo = fminf(fminf(r0, r1), 0.f), rhi = fmaxf(fmaxf(r0, r1), 0.f);
          for (int o = 16; o > 0; o >>= 1) {
            rlo = fminf(rlo, __shfl_xor(rlo, o, 64));
            rhi = fmaxf(rhi, __shfl_xor(rhi, o, 64));
          }
          const double Rg = (double)rhi - (double)rlo;
          const double Ra = __shfl(Rg, 0, 64), Rb = __shfl(Rg, 32, 64);
          const double S = Wa * Ra * Ra + Wb * Rb * Rb;
          if (S < bestS || (S == bestS && jj[u] < bestj)) { bestS = S; bestj = jj[u]; }
        }
      }
      win = bestj;
    }
    if (MODE == MODE_ASSIGN) {
      if (a.ub != nullptr) {
        // bounds for the later iterations: the winner's distance and the
        // second smallest (exact fp64 distances), rounded outward
        if (lane == (win & 63)) dq[wv][win] = __builtin_inf();
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        double b2 = dq[wv][lane];
        for (int q = 1; q < 4; ++q) b2 = fmin(b2, dq[wv][lane + 64 * q]);
        for (int o = 32; o > 0; o >>= 1) b2 = fmin(b2, __shfl_xor(b2, o, 64));
        if (lane == 0) {
          a.ub[base] = (float)sqrt(dwin) * (1.0f + 1.0f / 1048576.0f);
          a.lb[base] = (float)sqrt(b2) * (1.0f - 1.0f / 1048576.0f);
        }
      }
      if (lane == 0) {
        if (a.wl != nullptr) {
          const uint32_t old = a.idx[base];
          if (old != (uint32_t)win) {
            const int slot = atomicAdd(a.chg_cnt, 1);
            a.chg[slot] = make_uint2((uint32_t)base, old | ((uint32_t)win << 8));
          }
        }
        a.idx[base] = (uint8_t)win;
      }
      continue;
    }
    // codec for the winner
    const uint16_t* mw = a.mu + ((int64_t)h * NC + win) * D;
    const float m0 = bf16_bits_to_f32(mw[2 * lane]), m1 = bf16_bits_to_f32(mw[2 * lane + 1]);
    const float r0 = (float)x0 - m0, r1 = (float)x1 - m1;
    float rlo = fminf(fminf(r0, r1), 0.f), rhi = fmaxf(fmaxf(r0, r1), 0.f);
    for (int o = 16; o > 0; o >>= 1) {
      rlo = fminf(rlo, __shfl_xor(rlo, o, 64));
      rhi = fmaxf(rhi, __shfl_xor(rhi, o, 64));
    }
    bool sat = false;
    const GroupCodec g = make_codec(rlo, rhi, &sat);   // lanes 0..31: group 0, 32..63: group 1
    const uint32_t q0 = code_of(r0, g), q1 = code_of(r1, g);
    // byte b = channels 4b..4b+3 = lanes 2b, 2b+1
    const uint32_t pair = q0 | (q1 << 2);
    const uint32_t other = __shfl_xor(pair, 1, 64);
    if ((lane & 1) == 0) a.codes[base * 32 + (lane >> 1)] = (uint8_t)(pair | (other << 4));
    const uint32_t sb0 = __shfl(g.sbits, 0, 64), sb1 = __shfl(g.sbits, 32, 64);
    const int z0 = __shfl(g.z, 0, 64), z1 = __shfl(g.z, 32, 64);
    const int nsat = __popcll(__ballot(sat && ((lane & 31) == 0)));
    if (lane == 0) {
      a.idx[base] = (uint8_t)win;
      a.scale[base * 2] = (uint16_t)sb0;
      a.scale[base * 2 + 1] = (uint16_t)sb1;
      const uint32_t nib = (uint32_t)(z0 | (z1 << 2));
      uint8_t* zb = a.zeros + (int64_t)h * a.zstride + (tok >> 1);
      uint32_t* word = reinterpret_cast<uint32_t*>(reinterpret_cast<uintptr_t>(zb) & ~(uintptr_t)3);
      const int sh = 8 * (int)(reinterpret_cast<uintptr_t>(zb) & 3) + 4 * (int)(tok & 1);
      atomicOr(word, nib << sh);
      if (nsat && a.diag) atomicAdd((unsigned long long*)&a.diag->scale_saturations, (unsigned long long)nsat);
    }
    if (MODE == MODE_KEYS && a.cq != nullptr) {
      int8_t* cq = a.cq + base * R;
      if (use_psac) {
        // E = k - mu - r_hat in fp64 (exact), C = E U in fp64
        const double e0 = x0 - (double)m0 - (double)g.s * (double)((int)q0 - g.z);
        const double e1 = x1 - (double)m1 - (double)g.s * (double)((int)q1 - g.z);
        const uint16_t* Uh = a.U + (int64_t)h * D * R;
        double C[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          double v = e0 * (double)bf16_bits_to_f32(Uh[(2 * lane) * R + i]) +
                     e1 * (double)bf16_bits_to_f32(Uh[(2 * lane + 1) * R + i]);
          C[i] = wave_sum_d(v);
        }
        double m = 0.0;
#pragma unroll
        for (int i = 0; i < R; ++i) m = fmax(m, fabs(C[i]));
        bool s2 = false;
        const uint32_t csb = fp16_up_div(m, 127.0f, &s2);
        if (s2 && lane == 0 && a.diag) atomicAdd((unsigned long long*)&a.diag->scale_saturations, 1ull);
        const double cs = (double)f16_bits_to_f32(csb);
        // integer coefficients of every lane's view (all lanes need them for
        // the keep test)
        int cqi[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          int qi = 0;
          if (cs > 0.0) {
            // round half to even of C / cs, decided with exact products (n +- 1/2) cs
            const double Ci = C[i];
            double n = rint(Ci / cs);
            if (Ci > (n + 0.5) * cs) n += 1.0;
            if (Ci < (n - 0.5) * cs) n -= 1.0;
            int ni = (int)n;
            if (Ci == (n + 0.5) * cs && (ni & 1)) ni += 1;
            else if (Ci == (n - 0.5) * cs && (ni & 1)) ni -= 1;
            qi = ni < -127 ? -127 : (ni > 127 ? 127 : ni);
          }
          cqi[i] = qi;
        }
        bool keep = true;
        if (a.flags & QWM_PSAC_KEEP) {
          // Keep test (QuantWM method step (4)): the coefficients stay only if
          // the compensation D = (c_s C_q) U^T lowers the Query-weighted error
          // sum_c w_c e_c^2 (weights of the centroid choice), i.e. iff
          // sum_c w_c D_c (D_c - 2 e_c) < 0; here in fp64
          double D0 = 0.0, D1 = 0.0;
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const double ci = cs * (double)cqi[i];
            D0 += ci * (double)bf16_bits_to_f32(Uh[(2 * lane) * R + i]);
            D1 += ci * (double)bf16_bits_to_f32(Uh[(2 * lane + 1) * R + i]);
          }
          const double crit = wave_sum_d(wx[wv][2 * lane] * D0 * (D0 - 2.0 * e0) +
                                         wx[wv][2 * lane + 1] * D1 * (D1 - 2.0 * e1));
          keep = crit < 0.0;
        }
        if (lane < R) {
          int qi = cqi[0];
#pragma unroll
          for (int i = 1; i < R; ++i) if (lane == i) qi = cqi[i];
          cq[lane] = keep ? (int8_t)qi : (int8_t)0;
        }
        if (lane == 0) a.cscale[base] = keep ? (uint16_t)csb : (uint16_t)0;
      } else {
        if (lane < R) cq[lane] = 0;
        if (lane == 0) a.cscale[base] = 0;
      }
    }
  }
}

// PSAC coefficients for the rank ablation (r = 16, 32), exact in fp64, after
// the centroid choice and codes are stored (QuantWM Sec. 4.2, method step (4);
// App. C.2 rank study): E = k - (mu_idx + s (q - z)), C = E U, c_s = smallest
// fp16 with 127 c_s >= max|C|, C_q = clamp(rne(C / c_s), -127, 127); the keep
// test as in the exact path.  One wave per token (4 per block), lane l holds
// channels 2 l, 2 l + 1.  Rows with a non-finite channel store zeros.
struct PsacArgs {
  const void* x; int32_t dtype; int64_t T; int64_t st, sh; int32_t H;
  const uint16_t* mu; const float* w; const uint16_t* U; uint32_t flags;
  const uint8_t* idx; const uint8_t* codes; const uint16_t* scale; const uint8_t* zeros; int64_t zstride;
  int8_t* cq; uint16_t* cscale; qwm_diag* diag;
};

template <int RR>
__global__ __launch_bounds__(256) void psac_kernel(PsacArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (id >= (int64_t)a.H * a.T) return;
  const int h = (int)(id / a.T);
  const int64_t tok = id % a.T, base = id;
  int8_t* cq = a.cq + base * RR;
  const bool psac = (a.flags & QWM_PSAC) && a.U != nullptr;
  const int64_t rowoff = (int64_t)h * a.sh + tok * a.st + 2 * lane;
  double x0, x1;
  if (a.dtype == QWM_F32) {
    const float* xr = static_cast<const float*>(a.x) + rowoff;
    x0 = xr[0]; x1 = xr[1];
  } else {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.x) + rowoff);
    x0 = bf16_bits_to_f32(v & 0xFFFFu); x1 = bf16_bits_to_f32(v >> 16);
  }
  const bool bad = __any(!(__builtin_isfinite(x0) && __builtin_isfinite(x1)));
  if (!psac || bad) {
    if (lane < RR) cq[lane] = 0;
    if (lane == 0) a.cscale[base] = 0;
    return;
  }
  const int g = lane >> 5;
  const uint32_t mw = *reinterpret_cast<const uint32_t*>(a.mu + ((int64_t)h * NC + a.idx[base]) * D + 2 * lane);
  const double m0 = bf16_bits_to_f32(mw & 0xFFFFu), m1 = bf16_bits_to_f32(mw >> 16);
  const uint32_t cb = a.codes[base * 32 + (lane >> 1)] >> (4 * (lane & 1));
  const int q0 = (int)(cb & 3u), q1 = (int)((cb >> 2) & 3u);
  const double sg = (double)f16_bits_to_f32(a.scale[base * 2 + g]);
  const int z = (a.zeros[(int64_t)h * a.zstride + (tok >> 1)] >> (4 * (int)(tok & 1) + 2 * g)) & 3;
  const double e0 = x0 - (m0 + sg * (double)(q0 - z));
  const double e1 = x1 - (m1 + sg * (double)(q1 - z));
  const bool wts = (a.flags & QWM_QSAC) && a.w != nullptr;
  psac_token<RR>(e0, e1, lane, a.U + (int64_t)h * D * RR, (a.flags & QWM_PSAC_KEEP) != 0,
                 wts ? (double)a.w[h * D + 2 * lane] : 1.0, wts ? (double)a.w[h * D + 2 * lane + 1] : 1.0,
                 cq, a.cscale + base, a.diag);
}

// mu_j^T S mu_j in fp64 for the full-matrix candidate distance: grid (H, NC / 4),
// one wave per centroid; lane r forms (S mu)_r for r = lane, lane + 64 from
// the column entries S[c][r] (S symmetric; S = I while n = 0).
__global__ __launch_bounds__(256) void fullq_bj_kernel(const uint16_t* __restrict__ mu, const double* __restrict__ S,
                                                       const int64_t* __restrict__ n, double* __restrict__ B) {
  const int h = blockIdx.x, lane = threadIdx.x & 63, j = blockIdx.y * 4 + (threadIdx.x >> 6);
  __shared__ double m[4][D];
  const int wv = threadIdx.x >> 6;
  const uint16_t* row = mu + ((int64_t)h * NC + j) * D;
  const double m0 = bf16_bits_to_f32(row[lane]), m1 = bf16_bits_to_f32(row[lane + 64]);
  m[wv][lane] = m0;
  m[wv][lane + 64] = m1;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  double v;
  if (n[h] <= 0) {
    v = m0 * m0 + m1 * m1;
  } else {
    const double* Sh = S + (int64_t)h * D * D;
    double t0 = 0.0, t1 = 0.0;
    for (int c = 0; c < D; ++c) {
      const double mc = m[wv][c];
      t0 = fma(Sh[c * D + lane], mc, t0);
      t1 = fma(Sh[c * D + lane + 64], mc, t1);
    }
    v = m0 * t0 + m1 * t1;
  }
  const double b = wave_sum_d(v);
  if (lane == 0) B[h * NC + j] = b;
}

// Clears n bytes (the zero-point nibbles that the exact kernel ORs into place).
__global__ __launch_bounds__(256) void clear_bytes_kernel(uint8_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

// ---------------------------------------------------------------------------
// Lloyd: Forgy seeding and the deterministic mean update.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t splitmix_next(uint64_t& state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Whether row `row` of head h has only finite channels.
__device__ __forceinline__ bool row_finite(const void* x, int32_t dtype, int64_t st, int64_t sh, int h, int64_t row) {
  const int64_t off = (int64_t)h * sh + row * st;
  uint32_t bad = 0u;
  if (dtype == QWM_BF16) {
    const uint4* r = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const uint4 v = r[c];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {   // bf16 exponent all ones: Inf or NaN
        bad |= ((w4[k] & 0x7F80u) == 0x7F80u) | ((w4[k] & 0x7F800000u) == 0x7F800000u);
      }
    }
  } else {
    const float4* r = reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const float4 v = r[c];
      bad |= !(__builtin_isfinite(v.x) && __builtin_isfinite(v.y) && __builtin_isfinite(v.z) && __builtin_isfinite(v.w));
    }
  }
  return bad == 0u;
}

// Grid H, 256 threads.  The 256 picks of the partial Fisher-Yates shuffle
// (pick i swaps slot i with slot j_i = i + r_i mod (T - i), r_i the i-th
// SplitMix64 output) are found in parallel: thread i draws r_i directly (the
// generator's state after i + 1 steps is seed + (i + 1) * gamma), and the token
// in slot p just before swap i is p itself unless some earlier swap k < i had
// j_k = p, in which case it is the token slot k held just before swap k (the
// last such k; resolved by walking back).  Only when a pick lands on a row with
// a non-finite channel does thread 0 replay the shuffle sequentially in perm
// ([H][T] int32 workspace) and go on past slot 255 (checking each further
// pick), leaving zero rows for slots that no finite token fills.
__device__ __forceinline__ uint64_t splitmix_at(uint64_t seed, uint64_t k) {
  uint64_t state = seed + k * 0x9E3779B97F4A7C15ull;   // state after k steps
  state -= 0x9E3779B97F4A7C15ull;                      // splitmix_next adds it back
  return splitmix_next(state);
}

__global__ __launch_bounds__(256) void forgy_kernel(const void* x, int32_t dtype, int64_t T, int64_t st, int64_t sh,
                                                    uint64_t seed, int32_t* perm, uint16_t* out) {
  const int h = blockIdx.x, tid = threadIdx.x;
  __shared__ int32_t pick[NC];
  __shared__ int64_t js[NC];
  __shared__ uint8_t ok[NC];
  const uint64_t s0 = seed + ((uint64_t)h << 32);
  {
    const uint64_t r = splitmix_at(s0, (uint64_t)tid + 1);
    js[tid] = tid + (int64_t)(r % (uint64_t)(T - tid));
  }
  __syncthreads();
  {
    int64_t p = js[tid];
    int lim = tid;
    for (;;) {
      int k = -1;
      for (int q = lim - 1; q >= 0; --q)
        if (js[q] == p) { k = q; break; }
      if (k < 0) break;
      p = k;
      lim = k;
    }
    pick[tid] = (int32_t)p;
  }
  __syncthreads();
  ok[tid] = row_finite(x, dtype, st, sh, h, pick[tid]) ? 1 : 0;
  if (__syncthreads_count(ok[tid] == 0) > 0) {
    int32_t* p = perm + (int64_t)h * T;
    for (int64_t i = tid; i < T; i += 256) p[i] = (int32_t)i;
    __syncthreads();
    if (tid == 0) {
      uint64_t state = s0;
      int slot = 0;
      for (int64_t i = 0; slot < NC && i < T; ++i) {
        const uint64_t r = splitmix_next(state);
        const int64_t j = i + (int64_t)(r % (uint64_t)(T - i));
        const int32_t t = p[i]; p[i] = p[j]; p[j] = t;
        if (i < NC ? ok[i] != 0 : row_finite(x, dtype, st, sh, h, p[i])) pick[slot++] = p[i];
      }
      for (; slot < NC; ++slot) pick[slot] = -1;
    }
  }
  __syncthreads();
  for (int e = tid; e < NC * D; e += 256) {
    const int i = e / D, c = e % D;
    uint32_t b = 0u;
    if (pick[i] >= 0) {
      const int64_t off = (int64_t)h * sh + (int64_t)pick[i] * st + c;
      if (dtype == QWM_BF16) b = static_cast<const uint16_t*>(x)[off];
      else b = f32_to_bf16_bits(static_cast<const float*>(x)[off]);
    }
    out[((int64_t)h * NC + i) * D + c] = (uint16_t)b;
  }
}

// The mean update runs in two kernels.
//
// lloyd_sort_kernel (grid (H, nb), 1,024 threads): a stable counting sort of
// the head's assignment: ids[h][start_j .. start_j + n_j) lists the members of
// cluster j in token order, start[h][j] = start_j, start[h][256] = members in
// all.  Block (h, b) places the b-th of nb contiguous chunks; each block counts
// the whole head (one byte per token) for the cluster totals and the members
// of the chunks before its own.  Wave w owns the tokens of the w-th of 16
// ranges of the chunk; after a count and a scan over (cluster, range), it walks
// its range 64 tokens at a time, and each lane finds the lanes holding the same
// cluster from eight ballots, so its place is the range's running offset plus
// the number of such lanes below it.
//
// lloyd_sum_kernel (one wave per (head, cluster), 64 lanes x 2 channels): the
// member rows summed in token order in fp64, 32 rows in flight; the new
// centroid is bf16(sum / n); an empty cluster keeps its centroid.  Heads that
// hold their sums in fixed point (not flagged, isums given) store the exact
// integer sums and counts instead, for the mean update of lloyd.hip.
constexpr int LS_WAVES = 16;

__global__ __launch_bounds__(1024) void lloyd_sort_kernel(const int32_t* hflag, const uint8_t* assign, const uint32_t* excl,
                                                          int64_t excl_words, int64_t T, int32_t* ids,
                                                          int32_t* start) {
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (hflag != nullptr && hflag[h] == 0) return;   // the integer path handles this head
  __shared__ int32_t cnt[LS_WAVES][NC];     // counts, then running offsets
  __shared__ int32_t tot[NC];
  __shared__ int32_t pre[NC];               // members in the chunks before this block's
  for (int e = tid; e < LS_WAVES * NC; e += 1024) (&cnt[0][0])[e] = 0;
  if (tid < NC) { tot[tid] = 0; pre[tid] = 0; }
  __syncthreads();
  const uint8_t* ah = assign + (int64_t)h * T;
  const uint32_t* eh = excl + (int64_t)h * excl_words;
  // block (h, b) places chunk b of gridDim.y; wave w the w-th of 16 parts of it
  const int nb = gridDim.y, b = blockIdx.y;
  const int64_t c0 = T * b / nb, c1 = T * (b + 1) / nb;
  const int64_t r0 = c0 + (c1 - c0) * wv / LS_WAVES, r1 = c0 + (c1 - c0) * (wv + 1) / LS_WAVES;
  for (int64_t t = r0 + lane; t < r1; t += 64)
    if (!((eh[t >> 5] >> (t & 31)) & 1u)) atomicAdd(&cnt[wv][ah[t]], 1);
  // the other chunks: the members before this one, and the cluster totals
  for (int64_t t = tid; t < c0; t += 1024)
    if (!((eh[t >> 5] >> (t & 31)) & 1u)) atomicAdd(&pre[ah[t]], 1);
  for (int64_t t = c1 + tid; t < T; t += 1024)
    if (!((eh[t >> 5] >> (t & 31)) & 1u)) atomicAdd(&tot[ah[t]], 1);
  __syncthreads();
  if (tid < NC) {
    int32_t run = 0;
#pragma unroll
    for (int w = 0; w < LS_WAVES; ++w) { const int32_t c = cnt[w][tid]; cnt[w][tid] = run; run += c; }
    tot[tid] += run + pre[tid];
  }
  __syncthreads();
  // exclusive scan of the cluster totals (one wave, 4 clusters per lane)
  if (wv == 0) {
    int32_t v[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = tot[4 * lane + i]; sum += v[i]; }
    int32_t inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    int32_t run = inc - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) { tot[4 * lane + i] = run; run += v[i]; }
    // members in all: the end of the last cluster (excluded rows are not members)
    if (lane == 63 && b == 0) start[h * (NC + 1) + NC] = run;
  }
  __syncthreads();
  if (tid < NC) {
    if (b == 0) start[h * (NC + 1) + tid] = tot[tid];
    const int32_t base = tot[tid] + pre[tid];
#pragma unroll
    for (int w = 0; w < LS_WAVES; ++w) cnt[w][tid] += base;
  }
  __syncthreads();
  int32_t* idh = ids + (int64_t)h * T;
  for (int64_t t0 = r0; t0 < r1; t0 += 64) {
    const int64_t t = t0 + lane;
    const bool valid = t < r1 && !((eh[t >> 5] >> (t & 31)) & 1u);
    const uint32_t key = valid ? ah[t] : 0u;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (key >> bit) & 1u;
      const uint64_t bb = __ballot(on);
      m &= on ? bb : ~bb;
    }
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (valid) {
      const int32_t base = cnt[wv][key];
      idh[base + below] = (int32_t)t;
    }
    // the lowest lane of each cluster advances that cluster's offset (the
    // reads above come first: one wave's LDS operations complete in order)
    if (valid && below == 0) cnt[wv][key] += (int32_t)__popcll(m);
  }
}

__global__ __launch_bounds__(256) void lloyd_sum_kernel(const void* x, int32_t dtype, int64_t T, int64_t st,
                                                        int64_t sh, int32_t H, const int32_t* ids,
                                                        const int32_t* start, const uint16_t* cin, uint16_t* cout,
                                                        const int32_t* hflag, const int32_t* emax,
                                                        int64_t* isums, int32_t* icnt, int32_t P) {
  const int lane = threadIdx.x & 63;
  // wave-uniform unit: the member ids then come in through scalar loads
  const int unit = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (unit >= H * NC) return;
  const int h = unit / NC, j = unit % NC;
  const bool fixed = hflag != nullptr && hflag[h] == 0;
  if (fixed && isums == nullptr) return;   // lloyd.hip keeps this head's sums by changes
  const int32_t b = start[h * (NC + 1) + j], n = start[h * (NC + 1) + j + 1] - b;
  const int32_t* mem = ids + (int64_t)h * T + b;
  const int64_t rowbase = (int64_t)h * sh + 2 * lane;
  constexpr int U = 32;
  if (fixed) {
    // exact integer sums in units 2^(emax_c - P).  Every value of an unflagged
    // head is a whole number of units below 2^P (P <= 48), so the fp64 sum of
    // a batch of at most 32 rows is exact (below 2^53 units); each batch sum
    // is then scaled to units and added as an integer.
    const int32_t e0 = emax[h * D + 2 * lane], e1 = emax[h * D + 2 * lane + 1];
    const int sc0 = e0 == INT_MIN ? 0 : P - e0, sc1 = e1 == INT_MIN ? 0 : P - e1;
    int64_t s0 = 0, s1 = 0;
    auto flush = [&](double d0, double d1) __attribute__((always_inline)) {
      s0 += (int64_t)ldexp(d0, sc0);
      s1 += (int64_t)ldexp(d1, sc1);
    };
    int e = 0;
    if (dtype == QWM_BF16) {
      const uint16_t* xb = static_cast<const uint16_t*>(x) + rowbase;
      int32_t id[U];
      if (n >= U) {
#pragma unroll
        for (int u = 0; u < U; ++u) id[u] = mem[u];
      }
      for (; e + U <= n; e += U) {
        uint32_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const uint32_t*>(xb + (int64_t)id[u] * st);
        // the next batch's ids while these rows are in flight
        if (e + 2 * U <= n) {
#pragma unroll
          for (int u = 0; u < U; ++u) id[u] = mem[e + U + u];
        }
        double d0 = 0.0, d1 = 0.0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          d0 += (double)__uint_as_float(v[u] << 16);
          d1 += (double)__uint_as_float(v[u] & 0xFFFF0000u);
        }
        flush(d0, d1);
      }
      double d0 = 0.0, d1 = 0.0;
      for (; e < n; ++e) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(xb + (int64_t)mem[e] * st);
        d0 += (double)__uint_as_float(v << 16);
        d1 += (double)__uint_as_float(v & 0xFFFF0000u);
      }
      flush(d0, d1);
    } else {
      const float* xf = static_cast<const float*>(x) + rowbase;
      for (; e + U <= n; e += U) {
        float2 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const float2*>(xf + (int64_t)mem[e + u] * st);
        double d0 = 0.0, d1 = 0.0;
#pragma unroll
        for (int u = 0; u < U; ++u) { d0 += (double)v[u].x; d1 += (double)v[u].y; }
        flush(d0, d1);
      }
      double d0 = 0.0, d1 = 0.0;
      for (; e < n; ++e) {
        const float2 v = *reinterpret_cast<const float2*>(xf + (int64_t)mem[e] * st);
        d0 += (double)v.x;
        d1 += (double)v.y;
      }
      flush(d0, d1);
    }
    isums[(int64_t)unit * D + 2 * lane] = s0;
    isums[(int64_t)unit * D + 2 * lane + 1] = s1;
    if (lane == 0) icnt[unit] = n;
    return;
  }
  double s0 = 0.0, s1 = 0.0;
  int e = 0;
  if (dtype == QWM_BF16) {
    const uint16_t* xb = static_cast<const uint16_t*>(x) + rowbase;
    int32_t id[U];
    if (n >= U) {
#pragma unroll
      for (int u = 0; u < U; ++u) id[u] = mem[u];
    }
    for (; e + U <= n; e += U) {
      uint32_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const uint32_t*>(xb + (int64_t)id[u] * st);
      // the next batch's ids while these rows are in flight
      if (e + 2 * U <= n) {
#pragma unroll
        for (int u = 0; u < U; ++u) id[u] = mem[e + U + u];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s0 += (double)__uint_as_float(v[u] << 16);
        s1 += (double)__uint_as_float(v[u] & 0xFFFF0000u);
      }
    }
    for (; e < n; ++e) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(xb + (int64_t)mem[e] * st);
      s0 += (double)__uint_as_float(v << 16);
      s1 += (double)__uint_as_float(v & 0xFFFF0000u);
    }
  } else {
    const float* xf = static_cast<const float*>(x) + rowbase;
    for (; e + U <= n; e += U) {
      float2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const float2*>(xf + (int64_t)mem[e + u] * st);
#pragma unroll
      for (int u = 0; u < U; ++u) { s0 += (double)v[u].x; s1 += (double)v[u].y; }
    }
    for (; e < n; ++e) {
      const float2 v = *reinterpret_cast<const float2*>(xf + (int64_t)mem[e] * st);
      s0 += (double)v.x;
      s1 += (double)v.y;
    }
  }
  const uint16_t* src = cin + ((int64_t)h * NC + j) * D + 2 * lane;
  uint16_t* dst = cout + ((int64_t)h * NC + j) * D + 2 * lane;
  if (n > 0) {
    dst[0] = (uint16_t)f64_to_bf16_bits(s0 / (double)n);
    dst[1] = (uint16_t)f64_to_bf16_bits(s1 / (double)n);
  } else if (src != dst) {
    dst[0] = src[0];
    dst[1] = src[1];
  }
}

}  // namespace qwm

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
namespace qwm_host {
using namespace qwm;

struct SelWork {
  uint16_t* aug; float* Bj; float* Bmax; double* Wg; int32_t* counter; int32_t* worklist; double* qB;
  uint8_t* assign; int32_t* perm; int32_t* start; uint32_t* excl;
  LloydState ll;
};

static constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static constexpr int64_t excl_words(int64_t T) { return (T + 31) / 32; }

constexpr size_t select_ws_bytes_c(int64_t T, int32_t H, bool lloyd) {
  size_t b = 0;
  b += align256((size_t)H * NC * 4 * 2);
  b += align256((size_t)H * NC * 4);
  b += align256((size_t)H * PREP_PARTS * 4);
  b += align256((size_t)H * 2 * 8);
  b += align256(16 + (size_t)H * 4);
  b += align256((size_t)H * T * 4);
  b += align256((size_t)H * NC * 8);
  if (lloyd) {
    b += align256((size_t)H * T);
    b += align256((size_t)H * T * 4);
    b += align256((size_t)H * (NC + 1) * 4);
    b += align256((size_t)H * excl_words(T) * 4);
  }
  return b;
}

size_t select_ws_bytes(int64_t T, int32_t H, bool lloyd) {
  return select_ws_bytes_c(T, H, lloyd) + (lloyd ? lloyd_state_bytes(T, H) : 0);
}

// ---------------------------------------------------------------------------
// Scratch of qwm_quantize_keys_noalloc, for callers that cannot allocate: the
// workspace of one key call of at most NOALLOC_MAX_H heads and
// NOALLOC_MAX_TH token-heads, in a static device array (one per device, held
// until the process ends).  Host code reaches it only through the address
// hipGetSymbolAddress returns for the current device.
// ---------------------------------------------------------------------------
constexpr int32_t NOALLOC_MAX_H = QWM_NOALLOC_MAX_HEADS;
constexpr int64_t NOALLOC_MAX_TH = QWM_NOALLOC_MAX_TOKEN_HEADS;
constexpr size_t NOALLOC_BYTES = select_ws_bytes_c(NOALLOC_MAX_TH / NOALLOC_MAX_H, NOALLOC_MAX_H, false);
}  // namespace qwm_host

static __device__ __align__(256) uint8_t scratch[qwm_host::NOALLOC_BYTES];

namespace qwm_host {
constexpr int NOALLOC_MAX_DEVICES = 64;
static void* g_scratch_ptr[NOALLOC_MAX_DEVICES];
static hipError_t g_scratch_err[NOALLOC_MAX_DEVICES];
static std::once_flag g_scratch_once[NOALLOC_MAX_DEVICES];

// Device address of the current device's scratch (looked up once per device).
qwm_status noalloc_keys_scratch(void** ptr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QWM_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return fail(QWM_ERR_UNSUPPORTED, "device ordinal beyond 63");
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess)
    return fail(QWM_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(g_scratch_err[dev]));
  *ptr = g_scratch_ptr[dev];
  return QWM_OK;
}

static SelWork carve(void* ws, int64_t T, int32_t H, bool lloyd, int32_t dtype = QWM_BF16) {
  char* p = static_cast<char*>(ws);
  SelWork w{};
  auto take = [&](size_t n) { char* r = p; p += align256(n); return r; };
  w.aug = reinterpret_cast<uint16_t*>(take((size_t)H * NC * 4 * 2));
  w.Bj = reinterpret_cast<float*>(take((size_t)H * NC * 4));
  w.Bmax = reinterpret_cast<float*>(take((size_t)H * PREP_PARTS * 4));
  w.Wg = reinterpret_cast<double*>(take((size_t)H * 2 * 8));
  w.counter = reinterpret_cast<int32_t*>(take(16 + (size_t)H * 4));
  w.worklist = reinterpret_cast<int32_t*>(take((size_t)H * T * 4));
  w.qB = reinterpret_cast<double*>(take((size_t)H * NC * 8));
  if (lloyd) {
    w.assign = reinterpret_cast<uint8_t*>(take((size_t)H * T));
    w.perm = reinterpret_cast<int32_t*>(take((size_t)H * T * 4));
    w.start = reinterpret_cast<int32_t*>(take((size_t)H * (NC + 1) * 4));
    w.excl = reinterpret_cast<uint32_t*>(take((size_t)H * excl_words(T) * 4));
    w.ll = lloyd_state_carve(p, T, H, dtype);
  }
  return w;
}

// Compute units of the current device, looked up once per device.
static int device_cus() {
  static std::atomic<int> cache[NOALLOC_MAX_DEVICES];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Selection blocks per head: the grid fits in one wave of resident blocks (two
// per CU: 80 KiB of LDS each), and each block takes an equal contiguous share
// of its head's tiles, so no block is left running alone at the end.
static int blocks_per_head(int64_t T, int32_t H) {
  const int64_t ntile = (T + SEL_TOK - 1) / SEL_TOK;
  int64_t want = 2 * (int64_t)device_cus() / H;
  if (want < 1) want = 1;
  return (int)(ntile < want ? ntile : want);
}

template <int MODE>
static qwm_status run_select(const qwm_tokens* x, SelectArgs& a, hipStream_t stream, const char* what) {
  const int bph = blocks_per_head(x->T, x->H);
  const bool qs = (MODE == MODE_KEYS) && (a.flags & QWM_QSAC) && a.M > 1;
  const bool wt = (MODE == MODE_KEYS) && a.w != nullptr;
  // keys and values: one-dimensional, heads interleaved, tiles from the
  // per-head counters (SEL_HEAD_COUNTERS) when every wave has at least 16
  // tiles to draw (fewer, and the counters' atomics cost more than the
  // balance gains); the Lloyd assignment: (blocks per head, H)
  if ((MODE == MODE_KEYS || MODE == MODE_VALUES) && (x->T + 31) / 32 >= 64 * (int64_t)bph) a.flags |= SEL_HEAD_COUNTERS;
  // M in 9 .. 16: sixteen values tracked per lane, so that the shortlist can
  // still be certified without the exact path; M >= 256: every centroid
  const bool kq16 = qs && a.M > 8 && a.M <= 16;
  const bool flat_keys = MODE == MODE_KEYS || MODE == MODE_VALUES;
  const dim3 grid(flat_keys ? (unsigned)(bph * x->H) : (unsigned)bph, flat_keys ? 1u : (unsigned)x->H), block(256);
  const bool f32 = x->dtype != QWM_BF16;
  const bool exh = qs && a.M >= NC;
  if constexpr (MODE == MODE_KEYS) {
    if (exh) {
      if (f32 && wt) hipLaunchKernelGGL((select_kernel<MODE, true, true, true, NC>), grid, block, 0, stream, a);
      else if (f32) hipLaunchKernelGGL((select_kernel<MODE, true, true, false, NC>), grid, block, 0, stream, a);
      else if (wt) hipLaunchKernelGGL((select_kernel<MODE, false, true, true, NC>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((select_kernel<MODE, false, true, false, NC>), grid, block, 0, stream, a);
    } else if (f32) {
      if (kq16 && wt) hipLaunchKernelGGL((select_kernel<MODE, true, true, true, 16>), grid, block, 0, stream, a);
      else if (kq16) hipLaunchKernelGGL((select_kernel<MODE, true, true, false, 16>), grid, block, 0, stream, a);
      else if (qs && wt) hipLaunchKernelGGL((select_kernel<MODE, true, true, true>), grid, block, 0, stream, a);
      else if (qs) hipLaunchKernelGGL((select_kernel<MODE, true, true, false>), grid, block, 0, stream, a);
      else if (wt) hipLaunchKernelGGL((select_kernel<MODE, true, false, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((select_kernel<MODE, true, false, false>), grid, block, 0, stream, a);
    } else {
      if (kq16 && wt) hipLaunchKernelGGL((select_kernel<MODE, false, true, true, 16>), grid, block, 0, stream, a);
      else if (kq16) hipLaunchKernelGGL((select_kernel<MODE, false, true, false, 16>), grid, block, 0, stream, a);
      else if (qs && wt) hipLaunchKernelGGL((select_kernel<MODE, false, true, true>), grid, block, 0, stream, a);
      else if (qs) hipLaunchKernelGGL((select_kernel<MODE, false, true, false>), grid, block, 0, stream, a);
      else if (wt) hipLaunchKernelGGL((select_kernel<MODE, false, false, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((select_kernel<MODE, false, false, false>), grid, block, 0, stream, a);
    }
  } else if constexpr (MODE == MODE_ASSIGN) {
    if (a.wl != nullptr) {
      // one resident wave of blocks over all heads' listed tiles
      const int64_t tiles = (int64_t)x->H * ((x->T + SEL_TOK - 1) / SEL_TOK);
      const int64_t g = 2 * (int64_t)device_cus();
      const dim3 fgrid((unsigned)(tiles < g ? tiles : g));
      if (f32) hipLaunchKernelGGL((select_kernel<MODE, true, false, false, 8, true, true>), fgrid, block, 0, stream, a);
      else hipLaunchKernelGGL((select_kernel<MODE, false, false, false, 8, true, true>), fgrid, block, 0, stream, a);
    } else if (a.ub != nullptr) {
      if (f32) hipLaunchKernelGGL((select_kernel<MODE, true, false, false, 8, false, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((select_kernel<MODE, false, false, false, 8, false, true>), grid, block, 0, stream, a);
    } else {
      if (f32) hipLaunchKernelGGL((select_kernel<MODE, true, false, false>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((select_kernel<MODE, false, false, false>), grid, block, 0, stream, a);
    }
  } else {
    if (f32) hipLaunchKernelGGL((select_kernel<MODE, true, false, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((select_kernel<MODE, false, false, false>), grid, block, 0, stream, a);
  }
  qwm_status s = check_launch(what);
  if (s != QWM_OK) return s;
  // one wave per flagged token; the count is known only on the device, so the
  // grid covers the worst case (up to 4,096 tokens in one round, three blocks
  // per CU) and idle blocks exit at once
  // (a bounded Lloyd iteration sends few tokens: a quarter of the grid)
  const int64_t worst = ((int64_t)x->H * x->T + 3) / 4;
  const int64_t cap = a.wl != nullptr ? 256 : 1024;
  const int fb = (int)(worst < cap ? worst : cap);
  if (x->dtype == QWM_BF16)
    hipLaunchKernelGGL((fallback_kernel<MODE, false>), dim3(fb), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fallback_kernel<MODE, true>), dim3(fb), dim3(256), 0, stream, a);
  return check_launch(what);
}

static void fill_common(SelectArgs& a, const qwm_tokens* x, const SelWork& w, const uint16_t* mu) {
  a.x = x->ptr; a.T = x->T; a.st = x->stride_t; a.sh = x->stride_h; a.H = x->H;
  a.aug = w.aug; a.Bj = w.Bj; a.Bmax = w.Bmax; a.Wg = w.Wg;
  a.mu = mu; a.counter = w.counter; a.worklist = w.worklist;
}

static qwm_status prep(const SelWork& w, const uint16_t* mu, const float* wts, int32_t H, hipStream_t stream,
                       int32_t* zero = nullptr, int32_t nzero = 0) {
  TablePrepArgs p{mu, wts, w.aug, w.Bj, w.Bmax, w.Wg, w.counter, zero, nzero, H};
  hipLaunchKernelGGL(prep_table_kernel, dim3(H, PREP_PARTS), dim3(256), 0, stream, p);
  return check_launch("centroid table preparation");
}

// Certified bound c on |f_j - e_j| / (A + B_j), A = ||k||_w^2, for the GEMM
// values f_j = B_j + sum_c mu_jc t_c, t = -2 w (.) k (sum_c |mu_jc t_c| <= A + B_j):
//   fp32 accumulation of 131 exact bf16 products (t exact in bf16: unweighted
//   bf16 tokens): <= 131 u (2 (A + B)) ~ 1.6e-5; with the t_hi + t_lo pair, 259
//   products: ~3.1e-5
//   the pair's remainder |t - t_hi - t_lo| <= 2^-16 |t| (two RNE roundings):
//   <= 2^-16 (A + B) ~ 1.5e-5; fl32(w k): 2^-24 (A + B)
//   the 3-part bf16 split of B_j: 2^-24 B
//   the 8 index bits packed into each value: <= 2^-15 |f| <= 2^-14 (A + 2 B)
// i.e. ~7.7e-5 with an exact t and ~1.1e-4 with the pair; the constants below
// add margin.
static float error_coeff(bool split) {
  return split ? (1.0f / 8192.0f + 1.0f / 32768.0f) : (1.0f / 8192.0f);
}

// The rank ablation's coefficients: one exact pass after the codes are stored.
static qwm_status launch_psac(const qwm_tokens* k, const uint16_t* centroids, const float* w, const uint16_t* U,
                              uint32_t flags, const qwm_packed* out, qwm_diag* diag, hipStream_t stream) {
  PsacArgs p{};
  p.x = k->ptr; p.dtype = k->dtype; p.T = k->T; p.st = k->stride_t; p.sh = k->stride_h; p.H = k->H;
  p.mu = centroids; p.w = w; p.U = U; p.flags = flags;
  p.idx = out->idx; p.codes = out->codes; p.scale = out->scale; p.zeros = out->zeros; p.zstride = zeros_stride(k->T);
  p.cq = out->c; p.cscale = out->c_scale; p.diag = diag;
  const int64_t blocks = ((int64_t)k->H * k->T + 3) / 4;
  if (out->r == 16) hipLaunchKernelGGL(psac_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(psac_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return check_launch("PSAC coefficients");
}

qwm_status launch_keys(const qwm_tokens* k, const uint16_t* centroids, const float* w, const uint16_t* U,
                       int32_t M, uint32_t flags, const qwm_packed* out, qwm_diag* diag, void* ws,
                       hipStream_t stream) {
  SelWork wk = carve(ws, k->T, k->H, false);
  const bool qsac = flags & QWM_QSAC;
  const float* wts = qsac ? w : nullptr;
  const bool fused_psac = out->r == R;   // rank 8: coefficients inside the selection kernels
  qwm_status s = prep(wk, centroids, wts, k->H, stream);
  if (s != QWM_OK) return s;
  SelectArgs a{};
  fill_common(a, k, wk, centroids);
  a.w = wts; a.U = (fused_psac && (flags & QWM_PSAC)) ? U : nullptr; a.M = M; a.flags = flags;
  a.cb = error_coeff(wts != nullptr || k->dtype != QWM_BF16);
  a.idx = out->idx; a.codes = out->codes; a.scale = out->scale; a.zeros = out->zeros;
  a.zstride = zeros_stride(k->T); a.diag = diag;
  a.cq = fused_psac ? out->c : nullptr; a.cscale = fused_psac ? out->c_scale : nullptr;
  s = run_select<MODE_KEYS>(k, a, stream, "key quantization");
  if (s != QWM_OK || fused_psac) return s;
  return launch_psac(k, centroids, wts, U, flags, out, diag, stream);
}

// The full-matrix ablation: S-weighted candidates for every token on the
// exact fp64 path (one wave per token, 4 per block, one head per grid row).
qwm_status launch_keys_full(const qwm_tokens* k, const uint16_t* centroids, const double* S, const int64_t* n,
                            const float* w, const uint16_t* U, int32_t M, uint32_t flags, const qwm_packed* out,
                            qwm_diag* diag, void* ws, hipStream_t stream) {
  SelWork wk = carve(ws, k->T, k->H, false);
  qwm_status s = prep(wk, centroids, w, k->H, stream);
  if (s != QWM_OK) return s;
  hipLaunchKernelGGL(fullq_bj_kernel, dim3(k->H, NC / 4), dim3(256), 0, stream, centroids, S, n, wk.qB);
  s = check_launch("full-matrix centroid terms");
  if (s != QWM_OK) return s;
  const int64_t zb = (int64_t)k->H * zeros_stride(k->T);
  const int64_t zblocks = (zb + 255) / 256;
  hipLaunchKernelGGL(clear_bytes_kernel, dim3((unsigned)(zblocks < 1024 ? (zblocks > 0 ? zblocks : 1) : 1024)),
                     dim3(256), 0, stream, out->zeros, zb);
  s = check_launch("zero-point clear");
  if (s != QWM_OK) return s;
  const bool fused_psac = out->r == R;
  SelectArgs a{};
  fill_common(a, k, wk, centroids);
  a.w = w; a.U = (fused_psac && (flags & QWM_PSAC)) ? U : nullptr; a.M = M; a.flags = flags;
  a.idx = out->idx; a.codes = out->codes; a.scale = out->scale; a.zeros = out->zeros;
  a.zstride = zeros_stride(k->T); a.diag = diag;
  a.cq = fused_psac ? out->c : nullptr; a.cscale = fused_psac ? out->c_scale : nullptr;
  a.qS = S; a.qn = n; a.qB = wk.qB;
  const int64_t per = (k->T + 3) / 4;
  const dim3 grid((unsigned)(per < 64 ? (per > 0 ? per : 1) : 64), (unsigned)k->H);
  if (k->dtype == QWM_BF16)
    hipLaunchKernelGGL((fallback_kernel<MODE_KEYS, false, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fallback_kernel<MODE_KEYS, true, true>), grid, dim3(256), 0, stream, a);
  s = check_launch("full-matrix key quantization");
  if (s != QWM_OK || fused_psac) return s;
  return launch_psac(k, centroids, w, U, flags, out, diag, stream);
}

qwm_status launch_values(const qwm_tokens* v, const uint16_t* centroids, const qwm_packed* out, qwm_diag* diag,
                         void* ws, hipStream_t stream) {
  SelWork wk = carve(ws, v->T, v->H, false);
  qwm_status s = prep(wk, centroids, nullptr, v->H, stream);
  if (s != QWM_OK) return s;
  SelectArgs a{};
  fill_common(a, v, wk, centroids);
  a.w = nullptr; a.U = nullptr; a.M = 1; a.flags = 0; a.cb = error_coeff(v->dtype != QWM_BF16);
  a.idx = out->idx; a.codes = out->codes; a.scale = out->scale; a.zeros = out->zeros;
  a.zstride = zeros_stride(v->T); a.cq = nullptr; a.cscale = nullptr; a.diag = diag;
  return run_select<MODE_VALUES>(v, a, stream, "value quantization");
}

qwm_status launch_lloyd(const qwm_tokens* x, int32_t iters, uint64_t seed, const uint16_t* init, uint16_t* centroids,
                        qwm_diag* diag, void* ws, hipStream_t stream) {
  SelWork wk = carve(ws, x->T, x->H, true, x->dtype);
  const LloydState& ll = wk.ll;
  const uint16_t* cur = init;
  if (init == nullptr) {
    hipLaunchKernelGGL(forgy_kernel, dim3(x->H), dim3(256), 0, stream, x->ptr, x->dtype, x->T, x->stride_t,
                       x->stride_h, seed, wk.perm, centroids);
    qwm_status s = check_launch("centroid seeding");
    if (s != QWM_OK) return s;
    cur = centroids;
  }
  if (iters == 0 && init != nullptr && init != centroids) {
    if (hipMemcpyAsync(centroids, init, (size_t)x->H * NC * D * 2, hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return check_launch("centroid copy");
    return QWM_OK;
  }
  // Builds of at most three iterations (at most one could skip tokens, and the
  // scan and bound kernels would cost more than it saves) take the plain form:
  // every iteration assigns every token and every head's members are summed
  // in fp64 in token order (no flags: no scan).
  const bool with_bounds = iters >= 4;
  if (iters > 0) {   // no row excluded yet: the exact path marks non-finite rows
    const int64_t eb = (int64_t)x->H * excl_words(x->T) * 4;
    const int64_t eblocks = (eb + 255) / 256;
    hipLaunchKernelGGL(clear_bytes_kernel, dim3((unsigned)(eblocks < 1024 ? eblocks : 1024)), dim3(256), 0, stream,
                       reinterpret_cast<uint8_t*>(wk.excl), eb);
    qwm_status s = check_launch("Lloyd exclusion clear");
    if (s != QWM_OK) return s;
    // the fixed-point units of the member sums; heads with values finer than
    // their unit are flagged and take the fp64 member sums every iteration
    if (with_bounds) {
      s = lloyd_scan(x, ll, stream);
      if (s != QWM_OK) return s;
    }
  }
  for (int it = 0; it < iters; ++it) {
    // every iteration: the table terms of the GEMM, cleared list counters
    qwm_status s = prep(wk, cur, nullptr, x->H, stream, ll.wl_cnt, x->H + 1);
    if (s != QWM_OK) return s;
    SelectArgs a{};
    fill_common(a, x, wk, cur);
    a.M = 1; a.flags = 0; a.cb = error_coeff(x->dtype != QWM_BF16);
    a.idx = wk.assign; a.diag = diag; a.excl = wk.excl; a.excl_words = excl_words(x->T);
    // (the bounds that the third iteration starts from are the second's)
    if (with_bounds && it >= 1) { a.ub = ll.ub; a.lb = ll.lb; }
    // The first two iterations assign every token (the means still move far)
    // and sum the members from scratch; later ones assign again only the
    // tokens whose bounds no longer settle their centroid (every token of a
    // flagged head) and apply the recorded changes to the integer sums.
    const bool bounded = with_bounds && it >= 2;
    if (bounded) {
      s = lloyd_bounds(x, wk.assign, wk.excl, excl_words(x->T), ll, stream);
      if (s != QWM_OK) return s;
      a.wl = ll.wl; a.wl_cnt = ll.wl_cnt; a.chg = ll.chg; a.chg_cnt = ll.chg_cnt;
    }
    s = run_select<MODE_ASSIGN>(x, a, stream, "Lloyd assignment");
    if (s != QWM_OK) return s;
    // members sorted by centroid (the Forgy permutation is dead by now: its
    // buffer holds them), summed in fp64 for flagged heads, in fixed point for
    // the others while they are summed from scratch
    // (every head when all are sorted: chunks over the resident grid, two
    // 1,024-thread blocks per CU; bounded: only flagged heads, one block each)
    int nb = bounded ? 1 : 2 * device_cus() / x->H;
    nb = nb < 1 ? 1 : (nb > 8 ? 8 : nb);
    if ((int64_t)nb * 64 > x->T) nb = 1;
    hipLaunchKernelGGL(lloyd_sort_kernel, dim3(x->H, nb), dim3(1024), 0, stream, bounded ? ll.hflag : nullptr, wk.assign,
                       wk.excl, excl_words(x->T), x->T, wk.perm, wk.start);
    s = check_launch("Lloyd member sort");
    if (s != QWM_OK) return s;
    const int64_t units = (int64_t)x->H * NC;
    hipLaunchKernelGGL(lloyd_sum_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, x->ptr, x->dtype,
                       x->T, x->stride_t, x->stride_h, x->H, wk.perm, wk.start, cur, centroids,
                       with_bounds ? ll.hflag : nullptr, ll.emax,
                       bounded ? nullptr : ll.sums, ll.cnt, ll.P);
    s = check_launch("Lloyd update");
    if (s != QWM_OK) return s;
    if (bounded) {
      s = lloyd_apply_changes(x, ll, stream);
      if (s != QWM_OK) return s;
    }
    if (with_bounds) {   // (without flags every mean comes from the fp64 member sums)
      s = lloyd_finalize(x, ll, cur, centroids, stream);
      if (s != QWM_OK) return s;
    }
    cur = centroids;
  }
  return QWM_OK;
}

}  // namespace qwm_host
