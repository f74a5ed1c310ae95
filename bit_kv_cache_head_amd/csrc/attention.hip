// Attention over the compressed cache (QuantWM method section ¶1: logits
// Q K0_hat^T + (Q U_r) C^T; Sec. 3.3 logits Q K^T / sqrt(d); App. D.1 / Fig. 9
// on-demand reconstruction of keys and values, here fused into the kernel).
//
// Work unit: one head, 256 queries (8 waves x 32), one share of every
// segment's 64-key tiles.  Tiles flow through a two-stage pipeline: the packed
// bytes and centroid rows of tile t+2 are fetched into registers, tile t+1 is
// dequantized from registers into the second LDS buffer (fp16: K0_hat rows,
// the PSAC coefficients c_scale * c as 8 extra contraction channels, V_hat
// transposed), while tile t runs
//   S^T = [K0_hat | C_hat] [Q | Q U]^T     (MFMA 32x32x16 f16, contraction 128 + 16)
//   online softmax in fp32 (exp2 domain, lazy rescaling)
//   O^T += V_hat^T P                       (MFMA 32x32x16 f16)
// Split-key partial results are merged by a second kernel.  Work units are
// mapped to blocks so that one head's units share an XCD (and its L2).
#include "common.hpp"

namespace qwm {

constexpr int AT_W = 8;              // waves per block (two per SIMD)
constexpr int AT_QW = 32;            // queries per wave (one 32-query MFMA column tile)
constexpr int AT_Q = AT_W * AT_QW;   // queries per block
constexpr int AT_K = 64;             // keys per tile
constexpr int AT_T = 64 * AT_W;      // threads per block
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_SLACK = 8.0f;   // running max may lag the true max by 2^8
constexpr int TAB_ELEMS = NC * D;       // one fp16 centroid table

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Address-space views.  Segment descriptors are read through the constant
// address space (scalar loads: uniform, cached, counted apart from vector
// memory); packed data through the global one (global_load, never flat, so
// the register prefetch does not hold up LDS waits).
typedef const __attribute__((address_space(4))) qwm_segment cseg;
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gmem(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}

struct AttnArgs {
  const void* q; int32_t qdtype; int64_t Tq; int64_t qst; int64_t qsh;
  const qwm_segment* segs; int32_t n_segs; int32_t nsplit;   // segs: device array
  int32_t nqb; int32_t units;
  float scale;
  const uint16_t* tabs;   // fp16 centroid tables [seg][H][2][256][128]: K (channel-permuted), V
  // final outputs (nsplit == 1)
  float* out; float* lse; int32_t* top1; int32_t H;
  // partial outputs (nsplit > 1): [split][H][Tq][D], [split][H][Tq] x (m, l), top value / index
  float* po; float* pm; float* pl; float* ptv; int32_t* pti;
};

// K0_hat rows use a channel order in which the 32-bit word m of every
// 16-channel block holds channels (m, m + 8): the INT2 codes of those two
// channels sit 16 bits apart in the packed code word, so one shift and one
// mask put both into the two fp16 halves.  Q uses the same order (the
// contraction does not care); V_hat keeps the natural order.
struct AttnBuf {
  _Float16 khat[AT_K * D];     // [key][128 permuted], 16-byte chunk c of row k at (c ^ (k & 15))
  _Float16 chat[AT_K][16];     // PSAC channels: c_scale * c (8) + zero padding (8)
  _Float16 vt[D * AT_K];       // [channel][slot], chunk c of row ch at (c ^ ((ch >> 1) & 7))
};

// slot of a key in the transposed V tile: bits 2 and 3 swapped (matches the
// register order of the probabilities produced by the S^T MFMA)
__device__ __forceinline__ int vslot(int key) {
  return (key & ~0xC) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const uint16_t x = __builtin_bit_cast(uint16_t, (_Float16)a);
  const uint16_t y = __builtin_bit_cast(uint16_t, (_Float16)b);
  return (uint32_t)x | ((uint32_t)y << 16);
}
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
// two INT2 codes 16 bits apart (at bit `sh` and `sh + 16`) -> fp16 pair (1024 + q0, 1024 + q1)
__device__ __forceinline__ h2 code_pair(uint32_t w, int sh) {
  return as_h2(((w >> sh) & 0x00030003u) | 0x64006400u);
}

// ---------------------------------------------------------------------------
// fp16 copies of every segment's centroid tables (exact for bf16 values in
// fp16's normal range).  Grid (n_segs * H), 256 threads, thread = centroid.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attention_tables_kernel(const qwm_segment* __restrict__ segs, int32_t H,
                                                               uint16_t* __restrict__ tabs) {
  const int sh = blockIdx.x, seg = sh / H, h = sh % H, j = threadIdx.x;
  const qwm_segment& sg = segs[seg];
  const u32x4* kr = reinterpret_cast<const u32x4*>(sg.k_centroids + ((int64_t)h * NC + j) * D);
  const u32x4* vr = reinterpret_cast<const u32x4*>(sg.v_centroids + ((int64_t)h * NC + j) * D);
  u32x4* kt = reinterpret_cast<u32x4*>(tabs + ((int64_t)sh * 2 + 0) * TAB_ELEMS + (int64_t)j * D);
  u32x4* vtb = reinterpret_cast<u32x4*>(tabs + ((int64_t)sh * 2 + 1) * TAB_ELEMS + (int64_t)j * D);
#pragma unroll
  for (int blk = 0; blk < D / 16; ++blk) {
    const u32x4 a = kr[2 * blk], b = kr[2 * blk + 1];   // channels 16 blk + 0..7, + 8..15
    u32x4 o0, o1;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      // word m = (channel m, channel m + 8)
      const uint32_t lo = (m < 8) ? ((m & 1) ? (a[m >> 1] >> 16) : (a[m >> 1] & 0xFFFFu)) : 0u;
      const uint32_t hi = (m & 1) ? (b[m >> 1] >> 16) : (b[m >> 1] & 0xFFFFu);
      const uint32_t w = pack_f16x2(__uint_as_float(lo << 16), __uint_as_float(hi << 16));
      if (m < 4) o0[m] = w; else o1[m - 4] = w;
    }
    kt[2 * blk] = o0;
    kt[2 * blk + 1] = o1;
    const u32x4 c = vr[2 * blk], d = vr[2 * blk + 1];
    u32x4 p0, p1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p0[e] = pack_f16x2(__uint_as_float(c[e] << 16), __uint_as_float(c[e] & 0xFFFF0000u));
      p1[e] = pack_f16x2(__uint_as_float(d[e] << 16), __uint_as_float(d[e] & 0xFFFF0000u));
    }
    vtb[2 * blk] = p0;
    vtb[2 * blk + 1] = p1;
  }
}

__device__ __forceinline__ cseg& seg_at(const AttnArgs& a, int i) { return ((cseg*)a.segs)[i]; }

// Position in the flattened (segment, tile) sequence of one split.
struct TileIt {
  int seg;          // segment index, n_segs when done
  int64_t tile;     // tile index within the segment
  int64_t t_hi;     // end of this split's tile range in the segment
  int64_t kbase;    // global index of the segment's first key
};

__device__ __forceinline__ void seg_range(const AttnArgs& a, int seg, int split, int64_t& lo, int64_t& hi) {
  const int64_t T = seg_at(a, seg).T;
  const int64_t nt = (T + AT_K - 1) / AT_K;
  lo = nt * split / a.nsplit;
  hi = nt * (split + 1) / a.nsplit;
}

// first tile at or after segment `seg` (kbase = first key of `seg`)
__device__ __forceinline__ TileIt first_tile(const AttnArgs& a, int seg, int64_t kbase, int split) {
  TileIt it;
  while (seg < a.n_segs) {
    int64_t lo, hi;
    seg_range(a, seg, split, lo, hi);
    if (lo < hi) { it.seg = seg; it.tile = lo; it.t_hi = hi; it.kbase = kbase; return it; }
    kbase += seg_at(a, seg).T;
    ++seg;
  }
  it.seg = a.n_segs; it.tile = 0; it.t_hi = 0; it.kbase = kbase;
  return it;
}

// The tile iterator is wave-uniform; saying so keeps it in scalar registers, so
// descriptor reads stay scalar loads.
__device__ __forceinline__ int64_t sfl64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ TileIt uni(const TileIt& t) {
  TileIt u;
  u.seg = __builtin_amdgcn_readfirstlane(t.seg);
  u.tile = sfl64(t.tile);
  u.t_hi = sfl64(t.t_hi);
  u.kbase = sfl64(t.kbase);
  return u;
}

__device__ __forceinline__ TileIt next_tile(const AttnArgs& a, const TileIt& it, int split) {
  if (it.tile + 1 < it.t_hi) { TileIt n = it; n.tile += 1; return n; }
  return first_tile(a, it.seg + 1, it.kbase + seg_at(a, it.seg).T, split);
}

// Per-thread share of one tile, loaded in three stages so that no load waits
// for another inside the loop:
//   idx  (issued three tiles ahead): the centroid index bytes;
//   raw  (two tiles ahead): codes, scales, zero-point bytes, PSAC bytes, plus
//        the centroid rows (their idx arrived one iteration earlier);
//   all arithmetic on these bytes happens in dequant_tile.
// Loads never branch: keys past the segment end read the segment's last key
// and are zeroed in dequant_tile.
//  K:    key tid / 8, channels 16 (tid % 8) .. +16 (one code word)
//  PSAC: key tid / 8, coefficients 2 (tid % 8), +1 for tid % 8 < 4
//  V:    keys 2 (tid % 32), +1, channels 8 (tid / 32) .. +8
struct TileIdx {
  uint32_t k, v0, v1;
};
struct TileRegs {
  uint32_t kcode, kscale, kzb, c2, cs;   // raw bytes / halves
  uint32_t vcode[2], vscale[2], vzb[2];
  u32x4 kmu[2];                           // 16 permuted fp16 centroid channels
  u32x4 vmu[2];                           // 8 fp16 centroid channels of each key
};

__device__ __forceinline__ int64_t clamp_key(int64_t gk, int64_t T) { return gk < T ? gk : T - 1; }

__device__ __forceinline__ void load_idx(const AttnArgs& a, const TileIt& it, int h, int tid, TileIdx& x) {
  cseg& sg = seg_at(a, it.seg);
  const int64_t T = sg.T, k0 = it.tile * AT_K, hb = (int64_t)h * T;
  x.k = gmem(sg.k_idx)[hb + clamp_key(k0 + (tid >> 3), T)];
  const int64_t g0 = k0 + 2 * (tid & 31);
  x.v0 = gmem(sg.v_idx)[hb + clamp_key(g0, T)];
  x.v1 = gmem(sg.v_idx)[hb + clamp_key(g0 + 1, T)];
}

__device__ __forceinline__ void load_raw(const AttnArgs& a, const TileIt& it, int h, int tid, bool psac,
                                         const TileIdx& x, TileRegs& r) {
  cseg& sg = seg_at(a, it.seg);
  const int64_t T = sg.T, k0 = it.tile * AT_K, hb = (int64_t)h * T;
  const int64_t zb = (int64_t)h * zeros_stride(T);
  const uint16_t* ktab = a.tabs + ((int64_t)(it.seg * a.H + h) * 2 + 0) * TAB_ELEMS;
  const uint16_t* vtab = ktab + TAB_ELEMS;
  {
    const int blk = tid & 7, g = blk >> 2;
    const int64_t gk = clamp_key(k0 + (tid >> 3), T);
    const int64_t row = hb + gk;
    r.kcode = *gmem(reinterpret_cast<const uint32_t*>(sg.k_codes + row * 32 + 4 * blk));
    r.kscale = gmem(sg.k_scale)[row * 2 + g];
    r.kzb = gmem(sg.k_zeros)[zb + (gk >> 1)];
    const u32x4* mu = reinterpret_cast<const u32x4*>(ktab + (int64_t)x.k * D + 16 * blk);
    r.kmu[0] = gmem(mu)[0];
    r.kmu[1] = gmem(mu)[1];
    // PSAC bytes; without PSAC any in-bounds bytes do (the term is skipped)
    const uint16_t* c2p = psac ? reinterpret_cast<const uint16_t*>(sg.k_c + row * R + 2 * (blk & 3))
                               : reinterpret_cast<const uint16_t*>(sg.k_codes + row * 32);
    const uint16_t* csp = psac ? sg.k_c_scale + row : sg.k_scale + row * 2;
    r.c2 = *gmem(c2p);
    r.cs = *gmem(csp);
  }
  {
    const int oct = tid >> 5, g = oct >> 3;
    const int64_t g0 = k0 + 2 * (tid & 31);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t gk = clamp_key(g0 + u, T);
      const int64_t row = hb + gk;
      r.vcode[u] = *gmem(reinterpret_cast<const uint16_t*>(sg.v_codes + row * 32 + 2 * oct));
      r.vscale[u] = gmem(sg.v_scale)[row * 2 + g];
      r.vzb[u] = gmem(sg.v_zeros)[zb + (gk >> 1)];
      r.vmu[u] = *gmem(reinterpret_cast<const u32x4*>(vtab + (int64_t)(u ? x.v1 : x.v0) * D + 8 * oct));
    }
  }
}

// fp16 step | fp16 (-1024 - z) << 16 for key gk, group g, from the raw bytes
__device__ __forceinline__ uint32_t sz_pair(uint32_t sbits, uint32_t zbyte, int64_t gk, int g) {
  const uint32_t z = (zbyte >> (4 * (uint32_t)(gk & 1) + 2 * g)) & 3u;
  const uint16_t nz = __builtin_bit_cast(uint16_t, (_Float16)(-1024.0f - (float)z));
  return sbits | ((uint32_t)nz << 16);
}

// nvalid = keys of this tile inside its segment; k0 = first key's index in it
__device__ __forceinline__ void dequant_tile(const TileRegs& r, int tid, int nvalid, int64_t k0, AttnBuf& b) {
  {
    const int key = tid >> 3, blk = tid & 7;
    const bool ok = key < nvalid;
    const uint32_t ksz = sz_pair(r.kscale, r.kzb, k0 + key, blk >> 2);
    const h2 s2 = as_h2((ksz & 0xFFFFu) * 0x10001u);
    const h2 nz2 = as_h2((ksz >> 16) * 0x10001u);
    u32x4 o[2];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const h2 d = code_pair(r.kcode, 2 * m) + nz2;
      const h2 v = __builtin_elementwise_fma(s2, d, as_h2(r.kmu[m >> 2][m & 3]));
      o[m >> 2][m & 3] = ok ? as_u32(v) : 0u;
    }
    u32x4* kr = reinterpret_cast<u32x4*>(b.khat) + key * 16;
    kr[(2 * blk) ^ (key & 15)] = o[0];
    kr[(2 * blk + 1) ^ (key & 15)] = o[1];
    if (blk < 4) {
      // PSAC coefficients c_scale * c of this key, two of the eight
      const float cs = f16_bits_to_f32(r.cs);
      const int8_t c0 = (int8_t)(r.c2 & 0xFFu), c1 = (int8_t)((r.c2 >> 8) & 0xFFu);
      *reinterpret_cast<uint32_t*>(&b.chat[key][2 * blk]) = ok ? pack_f16x2(cs * (float)c0, cs * (float)c1) : 0u;
    }
  }
  {
    // keys 2p (low half) and 2p + 1 (high half) of channel 8 oct + c; a key past
    // the segment end gets s = 0, mu = 0 and a zero (-1024 - z) word: value 0
    const int p = tid & 31, oct = tid >> 5, g = oct >> 3;
    const bool v0 = 2 * p < nvalid, v1 = 2 * p + 1 < nvalid;
    const uint32_t cw = (v0 ? r.vcode[0] : 0u) | ((v1 ? r.vcode[1] : 0u) << 16);
    const uint32_t sz0 = v0 ? sz_pair(r.vscale[0], r.vzb[0], k0 + 2 * p, g) : 0u;
    const uint32_t sz1 = v1 ? sz_pair(r.vscale[1], r.vzb[1], k0 + 2 * p + 1, g) : 0u;
    const h2 s2 = as_h2((sz0 & 0xFFFFu) | (sz1 << 16));
    const h2 nz2 = as_h2((sz0 >> 16) | (sz1 & 0xFFFF0000u));
    const int slot = vslot(2 * p);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t w0 = v0 ? r.vmu[0][c >> 1] : 0u, w1 = v1 ? r.vmu[1][c >> 1] : 0u;
      const uint32_t mu2 = __builtin_amdgcn_perm(w1, w0, (c & 1) ? 0x07060302u : 0x05040100u);
      const h2 d = code_pair(cw, 2 * c) + nz2;
      const uint32_t v = as_u32(__builtin_elementwise_fma(s2, d, as_h2(mu2)));
      const int ch = 8 * oct + c;
      const int ck = (slot >> 3) ^ ((ch >> 1) & 7);
      *reinterpret_cast<uint32_t*>(&b.vt[ch * AT_K + ck * 8 + (slot & 7)]) = v;
    }
  }
}

__device__ __forceinline__ int tile_nvalid(const AttnArgs& a, const TileIt& it) {
  const int64_t rest = seg_at(a, it.seg).T - it.tile * AT_K;
  return (int)(rest < AT_K ? rest : AT_K);
}

template <bool TOP1>
__global__ __launch_bounds__(AT_T, 1) void attention_kernel(AttnArgs a) {
  __shared__ AttnBuf sb[2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hh = lane >> 5, ln = lane & 31;
  // XCD-aware unit mapping: consecutive units (same head) go to the same XCD
  const int nb = (int)gridDim.x;
  const int per = (nb + 7) / 8;
  const int unit = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (unit >= a.units) return;
  const int qb = unit % a.nqb;
  const int split = (unit / a.nqb) % a.nsplit;
  const int h = unit / (a.nqb * a.nsplit);
  const int64_t qw0 = (int64_t)qb * AT_Q + wv * AT_QW;
  const bool wave_active = qw0 < a.Tq;
  const int64_t qi = qw0 + ln;
  const bool qvalid = qi < a.Tq;
  const int64_t qoff = (int64_t)h * a.qsh + (qvalid ? qi : 0) * a.qst;

  // Q fragments (B operand of S^T), fp16, in the permuted channel order of the
  // K0_hat rows: k-step s, half hh holds channels 16 s + 4 hh + e and
  // 16 s + 8 + 4 hh + e (e = 0..3) in word e.
  f16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    u32x4 o;
    const int c_lo = 16 * s + 4 * hh, c_hi = c_lo + 8;
    if (a.qdtype == QWM_BF16) {
      const uint16_t* src = static_cast<const uint16_t*>(a.q) + qoff;
      const uint2 lo = qvalid ? *reinterpret_cast<const uint2*>(src + c_lo) : make_uint2(0u, 0u);
      const uint2 hi = qvalid ? *reinterpret_cast<const uint2*>(src + c_hi) : make_uint2(0u, 0u);
      const uint32_t lw[4] = {lo.x << 16, lo.x & 0xFFFF0000u, lo.y << 16, lo.y & 0xFFFF0000u};
      const uint32_t hw[4] = {hi.x << 16, hi.x & 0xFFFF0000u, hi.y << 16, hi.y & 0xFFFF0000u};
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_f16x2(__uint_as_float(lw[e]), __uint_as_float(hw[e]));
    } else {
      const float* src = static_cast<const float*>(a.q) + qoff;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = qvalid ? pack_f16x2(src[c_lo + e], src[c_hi + e]) : 0u;
    }
    qf[s] = __builtin_bit_cast(f16x8, o);
  }

  const float sc2 = a.scale * LOG2E;
  float m_run = -__builtin_inff();     // running max (may lag the true max by RESCALE_SLACK)
  float l_run = 0.f;
  float best_v = -__builtin_inff();
  int32_t best_i = 0x7FFFFFFF;
  f32x16 o_acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) o_acc[c] = f32x16{};

  TileIt it = first_tile(a, 0, 0, split);
  if (it.seg >= a.n_segs) {
    // nothing to do for this split: publish an empty partial
    if (qvalid && a.nsplit > 1 && hh == 0) {
      const int64_t pidx = ((int64_t)split * a.H + h) * a.Tq + qi;
      a.pm[pidx] = -__builtin_inff(); a.pl[pidx] = 0.f;
      if (TOP1) { a.ptv[pidx] = best_v; a.pti[pidx] = best_i; }
    }
    return;
  }
  // the zero padding of the PSAC channels never changes
  if (tid < 2 * AT_K)
    *reinterpret_cast<u32x4*>(&sb[tid / AT_K].chat[tid % AT_K][8]) = u32x4{0u, 0u, 0u, 0u};
  // pipeline fill: tile 0 dequantized, tile 1 in registers, tile 2's indices in flight
  TileRegs regs;
  TileIdx tix;
  load_idx(a, it, h, tid, tix);
  load_raw(a, it, h, tid, seg_at(a, it.seg).U != nullptr, tix, regs);
  dequant_tile(regs, tid, tile_nvalid(a, it), it.tile * AT_K, sb[0]);
  TileIt nt = next_tile(a, it, split);
  TileIt nn = (nt.seg < a.n_segs) ? next_tile(a, nt, split) : nt;
  {
    // loads never sit behind a branch (a branch would turn the loaded registers
    // into phi copies that wait for the data): stages past the end of the split
    // reload a tile that exists, and nobody reads what they produce
    const TileIt l1 = uni((nt.seg < a.n_segs) ? nt : it);
    load_idx(a, l1, h, tid, tix);
    load_raw(a, l1, h, tid, seg_at(a, l1.seg).U != nullptr, tix, regs);
    const TileIt l2 = uni((nn.seg < a.n_segs) ? nn : l1);
    load_idx(a, l2, h, tid, tix);
  }
  __syncthreads();

  int cur = 0;
  int qp_seg = -1;
  f16x8 qpf = __builtin_bit_cast(f16x8, u32x4{0, 0, 0, 0});
  bool psac = false;
  const h2 ones = as_h2(0x3C003C00u);
  while (true) {
    cseg& sg = seg_at(a, it.seg);
    if (it.seg != qp_seg) {
      // Q U for this segment: (U^T) (Q^T) on MFMA with bf16 operands
      qp_seg = it.seg;
      psac = sg.U != nullptr;
      qpf = __builtin_bit_cast(f16x8, u32x4{0, 0, 0, 0});
      if (psac && wave_active) {
        const __attribute__((address_space(1))) uint16_t* Uh = gmem(sg.U) + (int64_t)h * D * R;
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          u32x4 uv = {0, 0, 0, 0};
          if (ln < R) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              uv[e] = (uint32_t)Uh[(16 * s + 8 * hh + 2 * e) * R + ln] |
                      ((uint32_t)Uh[(16 * s + 8 * hh + 2 * e + 1) * R + ln] << 16);
          }
          u32x4 qv;
          if (a.qdtype == QWM_BF16) {
            qv = qvalid ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + qoff + 16 * s + 8 * hh)
                        : u32x4{0, 0, 0, 0};
          } else {
            const float* src = static_cast<const float*>(a.q) + qoff + 16 * s + 8 * hh;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              qv[e] = qvalid ? (f32_to_bf16_bits(src[2 * e]) | (f32_to_bf16_bits(src[2 * e + 1]) << 16)) : 0u;
          }
          acc = mfma_bf16(__builtin_bit_cast(bf16x8, uv), __builtin_bit_cast(bf16x8, qv), acc);
        }
        // lane (query, hh) holds (QU)[4 hh + 0..3]; hh = 0 needs all 8
        const float o0 = swap32_f(acc[0]), o1 = swap32_f(acc[1]), o2 = swap32_f(acc[2]), o3 = swap32_f(acc[3]);
        u32x4 pv = {0, 0, 0, 0};
        if (hh == 0) {
          pv[0] = pack_f16x2(acc[0], acc[1]);
          pv[1] = pack_f16x2(acc[2], acc[3]);
          pv[2] = pack_f16x2(o0, o1);
          pv[3] = pack_f16x2(o2, o3);
        }
        qpf = __builtin_bit_cast(f16x8, pv);
      }
    }
    const AttnBuf& B = sb[cur];
    const int64_t k0 = it.tile * AT_K;
    const int nvalid = (int)((sg.T - k0) < AT_K ? (sg.T - k0) : AT_K);
    const TileIt n3 = uni((nn.seg < a.n_segs) ? next_tile(a, nn, split) : nn);

    // The tile is processed as two 32-key halves; the next tile is dequantized
    // between them.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (wave_active && 32 * kt < nvalid) {
        // ---- S^T = K_ext Q_ext^T for 32 keys x 32 queries ----
        f32x16 sacc = {};
        const int key = 32 * kt + ln;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int c = 2 * s + hh;
          const f16x8 kf = reinterpret_cast<const f16x8*>(B.khat)[key * 16 + (c ^ (key & 15))];
          sacc = mfma_f16(kf, qf[s], sacc);
        }
        if (psac) {
          const f16x8 cf = *reinterpret_cast<const f16x8*>(&B.chat[key][8 * hh]);
          sacc = mfma_f16(cf, qpf, sacc);
        }
        // ---- online softmax (exp2 domain) ----
        if (32 * kt + 32 > nvalid) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + c_row(i, hh) >= nvalid) sacc[i] = -__builtin_inff();
        }
        float mt = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 16; i += 2) mt = fmaxf(mt, fmaxf(sacc[i], sacc[i + 1]));
        if (TOP1) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (sacc[i] > best_v) { best_v = sacc[i]; best_i = (int32_t)(it.kbase + k0 + 32 * kt + c_row(i, hh)); }
        }
        mt = fmaxf(mt, swap32_f(mt)) * sc2;
        if (mt > m_run + RESCALE_SLACK || m_run == -__builtin_inff()) {
          // raise the running max (to this max) and rescale what was accumulated
          const float alpha = (m_run == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m_run - mt);
          m_run = mt;
          l_run *= alpha;
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) o_acc[c][i] *= alpha;
        }
        u32x4 pw[2];
        float lsum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[i], sc2, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[i + 1], sc2, -m_run));
          const h2 pk = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(p0, p1));
          // the denominator sums exactly the fp16 probabilities the P V product uses
          lsum = __builtin_amdgcn_fdot2(pk, ones, lsum, false);
          // PV k-step 2 kt + i / 8, element (i % 8)
          pw[i >> 3][(i & 7) >> 1] = as_u32(pk);
        }
        l_run += lsum;
        // ---- O^T += V^T P over these 32 keys ----
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int ch = 32 * c + ln;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int chunk = (2 * (2 * kt + s2) + hh) ^ ((ch >> 1) & 7);
            const f16x8 vf = *reinterpret_cast<const f16x8*>(&B.vt[ch * AT_K + chunk * 8]);
            o_acc[c] = mfma_f16(vf, __builtin_bit_cast(f16x8, pw[s2]), o_acc[c]);
          }
        }
      }
      if (kt == 0) {
        // ---- next tile: dequantize from registers into the other buffer; fetch the
        //      bytes of the tile after it and the indices of the one after that.
        //      Past the end of the split these stages repeat a tile that exists
        //      (into a buffer nobody reads), so that no load is conditional. ----
        const TileIt d1 = uni((nt.seg < a.n_segs) ? nt : it);
        dequant_tile(regs, tid, tile_nvalid(a, d1), d1.tile * AT_K, sb[cur ^ 1]);
        const TileIt l2 = uni((nn.seg < a.n_segs) ? nn : d1);
        load_raw(a, l2, h, tid, seg_at(a, l2.seg).U != nullptr, tix, regs);
        const TileIt l3 = uni((n3.seg < a.n_segs) ? n3 : l2);
        load_idx(a, l3, h, tid, tix);
      }
    }
    __syncthreads();
    if (nt.seg >= a.n_segs) break;
    it = nt;
    nt = nn;
    nn = n3;
    cur ^= 1;
  }

  // ---- epilogue ----
  const float l_tot = l_run + swap32_f(l_run);
  if (TOP1) {
    const float ov = swap32_f(best_v);
    const int32_t oi = (int32_t)swap32_u((uint32_t)best_i);
    if (ov > best_v || (ov == best_v && oi < best_i)) { best_v = ov; best_i = oi; }
  }
  if (!qvalid) return;
  if (a.nsplit == 1) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    float* orow = a.out + (qi * a.H + h) * D;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int ch = 32 * c + 8 * m + 4 * hh;
        *reinterpret_cast<f32x4*>(orow + ch) =
            f32x4{o_acc[c][4 * m] * inv, o_acc[c][4 * m + 1] * inv, o_acc[c][4 * m + 2] * inv, o_acc[c][4 * m + 3] * inv};
      }
    if (hh == 0) {
      if (a.lse) a.lse[(int64_t)h * a.Tq + qi] = (m_run + log2f(l_tot)) / LOG2E;
      if (TOP1 && a.top1) a.top1[(int64_t)h * a.Tq + qi] = best_i;
    }
  } else {
    const int64_t pidx = ((int64_t)split * a.H + h) * a.Tq + qi;
    float* orow = a.po + pidx * D;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int ch = 32 * c + 8 * m + 4 * hh;
        *reinterpret_cast<f32x4*>(orow + ch) = f32x4{o_acc[c][4 * m], o_acc[c][4 * m + 1], o_acc[c][4 * m + 2], o_acc[c][4 * m + 3]};
      }
    if (hh == 0) {
      a.pm[pidx] = m_run;
      a.pl[pidx] = l_tot;
      if (TOP1) { a.ptv[pidx] = best_v; a.pti[pidx] = best_i; }
    }
  }
}

// Merge split partials.  Grid (ceil(Tq/2), H), 256 threads: two queries per block.
template <bool TOP1>
__global__ __launch_bounds__(256) void attention_combine_kernel(AttnArgs a) {
  const int h = blockIdx.y, c = threadIdx.x & 127;
  const int64_t qi = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  if (qi >= a.Tq) return;
  float mx = -__builtin_inff();
  for (int p = 0; p < a.nsplit; ++p) mx = fmaxf(mx, a.pm[((int64_t)p * a.H + h) * a.Tq + qi]);
  float l = 0.f, o = 0.f;
  float bv = -__builtin_inff();
  int32_t bi = 0x7FFFFFFF;
  for (int p = 0; p < a.nsplit; ++p) {
    const int64_t pidx = ((int64_t)p * a.H + h) * a.Tq + qi;
    const float pm = a.pm[pidx];
    const float wgt = (pm == -__builtin_inff()) ? 0.f : exp2f(pm - mx);
    l += a.pl[pidx] * wgt;
    o += a.po[pidx * D + c] * wgt;
    if (TOP1) {
      const float v = a.ptv[pidx];
      const int32_t i = a.pti[pidx];
      if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
    }
  }
  a.out[(qi * a.H + h) * D + c] = l > 0.f ? o / l : 0.f;
  if (c == 0) {
    if (a.lse) a.lse[(int64_t)h * a.Tq + qi] = (mx + log2f(l)) / LOG2E;
    if (TOP1 && a.top1) a.top1[(int64_t)h * a.Tq + qi] = bi;
  }
}

}  // namespace qwm

namespace qwm_host {
using namespace qwm;

// Number of key splits: fill the 256 CUs (one block per CU) in whole rounds.
static int attention_splits(int64_t Tq, int32_t H, int64_t total_keys) {
  const int64_t units = ((Tq + AT_Q - 1) / AT_Q) * H;
  const int64_t tiles = (total_keys + AT_K - 1) / AT_K;
  int best = 1;
  double best_score = -1.0;
  for (int s = 1; s <= 32; ++s) {
    if (s > 1 && tiles / s < 8) break;                 // keep splits meaningfully long
    const int64_t n = units * s;
    const int64_t rounds = (n + 255) / 256;
    // CU occupancy over whole rounds, minus a small cost per extra split (merge work)
    const double score = (double)n / (double)(rounds * 256) - 0.02 * s;
    if (score > best_score + 1e-9) { best_score = score; best = s; }
  }
  return best;
}

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t attention_ws_bytes(int64_t total_keys, int32_t H, int64_t Tq, int32_t n_segs) {
  size_t bytes = al256((size_t)n_segs * H * 2 * TAB_ELEMS * sizeof(uint16_t));
  const int ns = attention_splits(Tq, H, total_keys);
  if (ns > 1) {
    const size_t n = (size_t)ns * H * Tq;
    bytes += al256(n * D * 4) + 4 * al256(n * 4);
  }
  return bytes;
}

qwm_status launch_attention(const qwm_tokens* q, const qwm_segment* segs, int32_t n_segs, int64_t total_keys,
                            float scale, float* out, float* lse, int32_t* top1, void* ws, hipStream_t stream) {
  AttnArgs a{};
  a.q = q->ptr; a.qdtype = q->dtype; a.Tq = q->T; a.qst = q->stride_t; a.qsh = q->stride_h;
  a.segs = segs; a.n_segs = n_segs; a.scale = scale; a.out = out; a.lse = lse; a.top1 = top1; a.H = q->H;
  a.nsplit = attention_splits(q->T, q->H, total_keys);
  a.nqb = (int32_t)((q->T + AT_Q - 1) / AT_Q);
  a.units = a.nqb * a.nsplit * q->H;
  char* p = static_cast<char*>(ws);
  a.tabs = reinterpret_cast<uint16_t*>(p);
  p += al256((size_t)n_segs * q->H * 2 * TAB_ELEMS * sizeof(uint16_t));
  if (a.nsplit > 1) {
    const size_t n = (size_t)a.nsplit * q->H * q->T;
    a.po = reinterpret_cast<float*>(p); p += al256(n * D * 4);
    a.pm = reinterpret_cast<float*>(p); p += al256(n * 4);
    a.pl = reinterpret_cast<float*>(p); p += al256(n * 4);
    a.ptv = reinterpret_cast<float*>(p); p += al256(n * 4);
    a.pti = reinterpret_cast<int32_t*>(p);
  }
  hipLaunchKernelGGL(attention_tables_kernel, dim3((unsigned)(n_segs * q->H)), dim3(NC), 0, stream, segs, q->H,
                     const_cast<uint16_t*>(a.tabs));
  qwm_status s = check_launch("attention tables");
  if (s != QWM_OK) return s;
  const int per = (a.units + 7) / 8;
  const dim3 grid((unsigned)(per * 8));
  if (top1) hipLaunchKernelGGL(attention_kernel<true>, grid, dim3(AT_T), 0, stream, a);
  else hipLaunchKernelGGL(attention_kernel<false>, grid, dim3(AT_T), 0, stream, a);
  s = check_launch("attention");
  if (s != QWM_OK || a.nsplit == 1) return s;
  const dim3 g2((unsigned)((q->T + 1) / 2), (unsigned)q->H);
  if (top1) hipLaunchKernelGGL(attention_combine_kernel<true>, g2, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(attention_combine_kernel<false>, g2, dim3(256), 0, stream, a);
  return check_launch("attention merge");
}

}  // namespace qwm_host
