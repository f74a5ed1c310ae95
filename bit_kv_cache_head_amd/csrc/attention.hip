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

constexpr int AT_W = 8;            // waves per block
constexpr int AT_Q = 32 * AT_W;    // queries per block
constexpr int AT_K = 64;           // keys per tile
constexpr int AT_T = 64 * AT_W;    // threads per block
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_SLACK = 8.0f;   // running max may lag the true max by 2^8

struct AttnArgs {
  const void* q; int32_t qdtype; int64_t Tq; int64_t qst; int64_t qsh;
  const qwm_segment* segs; int32_t n_segs; int32_t nsplit;
  int32_t nqb; int32_t units;
  float scale;
  // final outputs (nsplit == 1)
  float* out; float* lse; int32_t* top1; int32_t H;
  // partial outputs (nsplit > 1): [split][H][Tq][D], [split][H][Tq] x (m, l), top value / index
  float* po; float* pm; float* pl; float* ptv; int32_t* pti;
};

struct AttnBuf {
  _Float16 khat[AT_K * D];     // [key][128], 16-byte chunk c of row k at (c ^ (k & 15))
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

// Position in the flattened (segment, tile) sequence of one split.
struct TileIt {
  int seg;          // segment index, n_segs when done
  int64_t tile;     // tile index within the segment
  int64_t t_hi;     // end of this split's tile range in the segment
  int64_t kbase;    // global index of the segment's first key
};

__device__ __forceinline__ void seg_range(const AttnArgs& a, int seg, int split, int64_t& lo, int64_t& hi) {
  const int64_t T = a.segs[seg].T;
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
    kbase += a.segs[seg].T;
    ++seg;
  }
  it.seg = a.n_segs; it.tile = 0; it.t_hi = 0; it.kbase = kbase;
  return it;
}

__device__ __forceinline__ TileIt next_tile(const AttnArgs& a, const TileIt& it, int split) {
  if (it.tile + 1 < it.t_hi) { TileIt n = it; n.tile += 1; return n; }
  return first_tile(a, it.seg + 1, it.kbase + a.segs[it.seg].T, split);
}

// Packed bytes and centroid rows of one tile held in registers by one thread.
// Keys: thread -> (key = tid / 8, 16 channels 16 * (tid % 8) ...).
// Values: thread -> (keys 2 p, 2 p + 1 with p = tid / 16, 8 channels 8 * (tid % 16) ...).
struct TileRegs {
  uint32_t kcode;       // 16 codes
  u32x4 kmu0, kmu1;     // 16 bf16 centroid channels
  float ks, kz;         // step and zero-point of the key's group
  uint2 c8;             // PSAC coefficients (chunk 0 threads)
  float cs;
  uint32_t vcode[2];    // 8 codes of each key (16 bits used)
  u32x4 vmu[2];         // 8 bf16 centroid channels of each key
  float vs[2], vz[2];
  bool kvalid, vvalid[2];
};

__device__ __forceinline__ void load_tile(const AttnArgs& a, const TileIt& it, int h, int tid, TileRegs& r) {
  const qwm_segment& sg = a.segs[it.seg];
  const int64_t T = sg.T;
  const int64_t zstride = zeros_stride(T);
  const int64_t k0 = it.tile * AT_K;
  {
    const int key = tid >> 3, chunk = tid & 7, g = chunk >> 2;
    const int64_t gk = k0 + key;
    r.kvalid = gk < T;
    if (r.kvalid) {
      const int64_t row = (int64_t)h * T + gk;
      const uint32_t j = sg.k_idx[row];
      r.kcode = *reinterpret_cast<const uint32_t*>(sg.k_codes + row * 32 + 4 * chunk);
      r.ks = f16_bits_to_f32(sg.k_scale[row * 2 + g]);
      const uint32_t nib = (sg.k_zeros[(int64_t)h * zstride + (gk >> 1)] >> (4 * (gk & 1))) & 0xFu;
      r.kz = (float)((nib >> (2 * g)) & 3u);
      const u32x4* mu = reinterpret_cast<const u32x4*>(sg.k_centroids + ((int64_t)h * NC + j) * D + 16 * chunk);
      r.kmu0 = mu[0];
      r.kmu1 = mu[1];
      if (chunk == 0 && sg.U != nullptr) {
        r.c8 = *reinterpret_cast<const uint2*>(sg.k_c + row * R);
        r.cs = f16_bits_to_f32(sg.k_c_scale[row]);
      } else {
        r.c8 = make_uint2(0u, 0u);
        r.cs = 0.f;
      }
    }
  }
  {
    const int p = tid >> 4, chunk = tid & 15, g = chunk >> 3;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t gk = k0 + 2 * p + u;
      r.vvalid[u] = gk < T;
      if (r.vvalid[u]) {
        const int64_t row = (int64_t)h * T + gk;
        const uint32_t j = sg.v_idx[row];
        r.vcode[u] = *reinterpret_cast<const uint16_t*>(sg.v_codes + row * 32 + 2 * chunk);
        r.vs[u] = f16_bits_to_f32(sg.v_scale[row * 2 + g]);
        const uint32_t nib = (sg.v_zeros[(int64_t)h * zstride + (gk >> 1)] >> (4 * (gk & 1))) & 0xFu;
        r.vz[u] = (float)((nib >> (2 * g)) & 3u);
        r.vmu[u] = *reinterpret_cast<const u32x4*>(sg.v_centroids + ((int64_t)h * NC + j) * D + 8 * chunk);
      }
    }
  }
}

__device__ __forceinline__ void dequant_tile(const TileRegs& r, int tid, AttnBuf& b) {
  {
    const int key = tid >> 3, chunk = tid & 7;
    u32x4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
    if (r.kvalid) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w0 = r.kmu0[e], w1 = r.kmu1[e];
        const float q0 = (float)((r.kcode >> (4 * e)) & 3u), q1 = (float)((r.kcode >> (4 * e + 2)) & 3u);
        const float q2 = (float)((r.kcode >> (16 + 4 * e)) & 3u), q3 = (float)((r.kcode >> (16 + 4 * e + 2)) & 3u);
        o0[e] = pack_f16x2(fmaf(r.ks, q0 - r.kz, __uint_as_float(w0 << 16)),
                           fmaf(r.ks, q1 - r.kz, __uint_as_float(w0 & 0xFFFF0000u)));
        o1[e] = pack_f16x2(fmaf(r.ks, q2 - r.kz, __uint_as_float(w1 << 16)),
                           fmaf(r.ks, q3 - r.kz, __uint_as_float(w1 & 0xFFFF0000u)));
      }
    }
    u32x4* kr = reinterpret_cast<u32x4*>(b.khat) + key * 16;
    kr[(2 * chunk) ^ (key & 15)] = o0;
    kr[(2 * chunk + 1) ^ (key & 15)] = o1;
    if (chunk == 0) {
      u32x4 cv = {0, 0, 0, 0};
      if (r.kvalid) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wd = e < 2 ? r.c8.x : r.c8.y;
          const int8_t c0 = (int8_t)((wd >> (16 * (e & 1))) & 0xFF);
          const int8_t c1 = (int8_t)((wd >> (16 * (e & 1) + 8)) & 0xFF);
          cv[e] = pack_f16x2(r.cs * (float)c0, r.cs * (float)c1);
        }
      }
      *reinterpret_cast<u32x4*>(&b.chat[key][0]) = cv;
      *reinterpret_cast<u32x4*>(&b.chat[key][8]) = u32x4{0, 0, 0, 0};
    }
  }
  {
    const int p = tid >> 4, chunk = tid & 15;
    float vv[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = r.vmu[u][e];
        const float q0 = (float)((r.vcode[u] >> (4 * e)) & 3u), q1 = (float)((r.vcode[u] >> (4 * e + 2)) & 3u);
        vv[u][2 * e] = r.vvalid[u] ? fmaf(r.vs[u], q0 - r.vz[u], __uint_as_float(w << 16)) : 0.f;
        vv[u][2 * e + 1] = r.vvalid[u] ? fmaf(r.vs[u], q1 - r.vz[u], __uint_as_float(w & 0xFFFF0000u)) : 0.f;
      }
    const int slot = vslot(2 * p);     // slot of key 2p; key 2p + 1 takes the next slot
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int ch = 8 * chunk + c;
      const int ck = (slot >> 3) ^ ((ch >> 1) & 7);
      *reinterpret_cast<uint32_t*>(&b.vt[ch * AT_K + ck * 8 + (slot & 7)]) = pack_f16x2(vv[0][c], vv[1][c]);
    }
  }
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
  const int64_t qi = (int64_t)qb * AT_Q + wv * 32 + ln;
  const bool qvalid = qi < a.Tq;
  const int64_t qoff = (int64_t)h * a.qsh + (qvalid ? qi : 0) * a.qst;

  // Q fragments (B operand of S^T): channels 16 s + 8 hh + j, fp16
  f16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    u32x4 o;
    if (a.qdtype == QWM_BF16) {
      const u32x4 v = qvalid ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + qoff + 16 * s + 8 * hh)
                             : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = pack_f16x2(__uint_as_float(v[e] << 16), __uint_as_float(v[e] & 0xFFFF0000u));
    } else {
      const float* src = static_cast<const float*>(a.q) + qoff + 16 * s + 8 * hh;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = qvalid ? pack_f16x2(src[2 * e], src[2 * e + 1]) : 0u;
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
    if (qvalid && a.nsplit > 1) {
      const int64_t pidx = ((int64_t)split * a.H + h) * a.Tq + qi;
      if (hh == 0) { a.pm[pidx] = -__builtin_inff(); a.pl[pidx] = 0.f; if (TOP1) { a.ptv[pidx] = best_v; a.pti[pidx] = best_i; } }
    }
    return;
  }
  TileRegs regs;
  load_tile(a, it, h, tid, regs);
  dequant_tile(regs, tid, sb[0]);
  TileIt nt = next_tile(a, it, split);
  if (nt.seg < a.n_segs) load_tile(a, nt, h, tid, regs);
  __syncthreads();

  int cur = 0;
  int qp_seg = -1;
  f16x8 qpf = __builtin_bit_cast(f16x8, u32x4{0, 0, 0, 0});
  bool psac = false;
  while (true) {
    const qwm_segment& sg = a.segs[it.seg];
    if (it.seg != qp_seg) {
      // Q U for this segment: (U^T) (Q^T) on MFMA with bf16 operands
      qp_seg = it.seg;
      psac = sg.U != nullptr;
      qpf = __builtin_bit_cast(f16x8, u32x4{0, 0, 0, 0});
      if (psac) {
        const uint16_t* Uh = sg.U + (int64_t)h * D * R;
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

    // ---- S^T = K_ext Q_ext^T : two 32-key tiles ----
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 acc = {};
      const int key = 32 * kt + ln;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int c = 2 * s + hh;
        const f16x8 kf = reinterpret_cast<const f16x8*>(B.khat)[key * 16 + (c ^ (key & 15))];
        acc = mfma_f16(kf, qf[s], acc);
      }
      if (psac) {
        const f16x8 cf = *reinterpret_cast<const f16x8*>(&B.chat[key][8 * hh]);
        acc = mfma_f16(cf, qpf, acc);
      }
      sacc[kt] = acc;
    }

    // ---- next tile: dequantize from registers into the other buffer, fetch the one after ----
    const TileIt nn = (nt.seg < a.n_segs) ? next_tile(a, nt, split) : nt;
    if (nt.seg < a.n_segs) {
      dequant_tile(regs, tid, sb[cur ^ 1]);
      if (nn.seg < a.n_segs) load_tile(a, nn, h, tid, regs);
    }

    // ---- online softmax (exp2 domain) ----
    float mt = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * kt + c_row(i, hh);
        if (key >= nvalid) sacc[kt][i] = -__builtin_inff();
        mt = fmaxf(mt, sacc[kt][i]);
        if (TOP1) {
          if (sacc[kt][i] > best_v) { best_v = sacc[kt][i]; best_i = (int32_t)(it.kbase + k0 + key); }
        }
      }
    mt = fmaxf(mt, swap32_f(mt)) * sc2;
    if (mt > m_run + RESCALE_SLACK || m_run == -__builtin_inff()) {
      // raise the running max (to the tile max) and rescale what was accumulated
      const float alpha = (m_run == -__builtin_inff()) ? 0.f : exp2f(m_run - mt);
      m_run = mt;
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) o_acc[c][i] *= alpha;
    }
    u32x4 pw[4];
    float lsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = exp2f(fmaf(sacc[kt][i], sc2, -m_run));
        const float p1 = exp2f(fmaf(sacc[kt][i + 1], sc2, -m_run));
        lsum += p0 + p1;
        // PV k-step s = 2 kt + i / 8, element (i % 8)
        pw[2 * kt + (i >> 3)][(i & 7) >> 1] = pack_f16x2(p0, p1);
      }
    l_run += lsum;

    // ---- O^T += V^T P ----
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ch = 32 * c + ln;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int chunk = (2 * s + hh) ^ ((ch >> 1) & 7);
        const f16x8 vf = *reinterpret_cast<const f16x8*>(&B.vt[ch * AT_K + chunk * 8]);
        o_acc[c] = mfma_f16(vf, __builtin_bit_cast(f16x8, pw[s]), o_acc[c]);
      }
    }
    __syncthreads();
    if (nt.seg >= a.n_segs) break;
    it = nt;
    nt = nn;
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

size_t attention_ws_bytes(int64_t total_keys, int32_t H, int64_t Tq) {
  const int ns = attention_splits(Tq, H, total_keys);
  if (ns == 1) return 0;
  const size_t n = (size_t)ns * H * Tq;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(n * D * 4) + 4 * al(n * 4);
}

qwm_status launch_attention(const qwm_tokens* q, const qwm_segment* segs, int32_t n_segs, int64_t total_keys,
                            float scale, float* out, float* lse, int32_t* top1, void* ws, hipStream_t stream) {
  AttnArgs a{};
  a.q = q->ptr; a.qdtype = q->dtype; a.Tq = q->T; a.qst = q->stride_t; a.qsh = q->stride_h;
  a.segs = segs; a.n_segs = n_segs; a.scale = scale; a.out = out; a.lse = lse; a.top1 = top1; a.H = q->H;
  a.nsplit = attention_splits(q->T, q->H, total_keys);
  a.nqb = (int32_t)((q->T + AT_Q - 1) / AT_Q);
  a.units = a.nqb * a.nsplit * q->H;
  if (a.nsplit > 1) {
    const size_t n = (size_t)a.nsplit * q->H * q->T;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    char* p = static_cast<char*>(ws);
    a.po = reinterpret_cast<float*>(p); p += al(n * D * 4);
    a.pm = reinterpret_cast<float*>(p); p += al(n * 4);
    a.pl = reinterpret_cast<float*>(p); p += al(n * 4);
    a.ptv = reinterpret_cast<float*>(p); p += al(n * 4);
    a.pti = reinterpret_cast<int32_t*>(p);
  }
  const int per = (a.units + 7) / 8;
  const dim3 grid((unsigned)(per * 8));
  if (top1) hipLaunchKernelGGL(attention_kernel<true>, grid, dim3(AT_T), 0, stream, a);
  else hipLaunchKernelGGL(attention_kernel<false>, grid, dim3(AT_T), 0, stream, a);
  qwm_status s = check_launch("attention");
  if (s != QWM_OK || a.nsplit == 1) return s;
  const dim3 g2((unsigned)((q->T + 1) / 2), (unsigned)q->H);
  if (top1) hipLaunchKernelGGL(attention_combine_kernel<true>, g2, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(attention_combine_kernel<false>, g2, dim3(256), 0, stream, a);
  return check_launch("attention merge");
}

}  // namespace qwm_host
