// Attention over the compressed cache (QuantWM method section ¶1: logits
// Q K0_hat^T + (Q U_r) C^T; Sec. 3.3 logits Q K^T / sqrt(d); App. D.1 / Fig. 9
// on-demand reconstruction of keys and values, here fused into the kernel).
//
// Per block: one head, 128 queries (4 waves x 32), a share of every segment's
// 64-key tiles.  Each tile is dequantized into LDS as fp16 (K0_hat rows, the
// PSAC coefficients c_scale * c as 8 extra contraction channels, V_hat
// transposed), then
//   S^T = [K0_hat | C_hat] [Q | Q U]^T     (MFMA 32x32x16 f16, contraction 128 + 16)
//   online softmax in fp32 (exp2 domain)
//   O^T += V_hat^T P                       (MFMA 32x32x16 f16)
// Split-key partial results are merged by a second kernel.
#include "common.hpp"

namespace qwm {

constexpr int AT_Q = 128;        // queries per block
constexpr int AT_K = 64;         // keys per tile
constexpr float LOG2E = 1.4426950408889634f;

struct AttnArgs {
  const void* q; int32_t qdtype; int64_t Tq; int64_t qst; int64_t qsh;
  const qwm_segment* segs; int32_t n_segs; int32_t nsplit;
  float scale;
  // final outputs (nsplit == 1)
  float* out; float* lse; int32_t* top1; int32_t H;
  // partial outputs (nsplit > 1): [split][H][Tq][D], [split][H][Tq] x (m, l), top value / index
  float* po; float* pm; float* pl; float* ptv; int32_t* pti;
};

struct AttnShared {
  _Float16 khat[AT_K * D];     // [key][128], 16-byte chunk c of row k at (c ^ (k & 15))
  _Float16 chat[AT_K][16];     // PSAC channels: c_scale * c (8) + zero padding (8)
  _Float16 vt[D * AT_K];       // [channel][slot], chunk c of row ch at (c ^ ((ch >> 1) & 7))
  uint16_t ut[R][D];           // U^T of the current segment (bf16)
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

template <bool TOP1>
__global__ __launch_bounds__(256, 2) void attention_kernel(AttnArgs a) {
  __shared__ AttnShared sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hh = lane >> 5, ln = lane & 31;
  const int qb = blockIdx.x, h = blockIdx.y, split = blockIdx.z;
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
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  float best_v = -__builtin_inff();
  int32_t best_i = 0x7FFFFFFF;
  f32x16 o_acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) o_acc[c] = f32x16{};

  int64_t key_base = 0;
  for (int sg = 0; sg < a.n_segs; ++sg) {
    const qwm_segment seg = a.segs[sg];
    const int64_t T = seg.T;
    const int64_t ntiles = (T + AT_K - 1) / AT_K;
    const int64_t t_lo = ntiles * split / a.nsplit, t_hi = ntiles * (split + 1) / a.nsplit;
    const bool psac = seg.U != nullptr;
    const int64_t zstride = zeros_stride(T);
    f16x8 qpf = __builtin_bit_cast(f16x8, u32x4{0, 0, 0, 0});
    if (t_lo < t_hi && psac) {
      // Q U for this segment: (U^T) (Q^T) on MFMA, bf16 operands
      __syncthreads();
      for (int e = tid; e < D * R; e += 256) sm.ut[e % R][e / R] = seg.U[(int64_t)h * D * R + e];
      __syncthreads();
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x8 uf;
        if (ln < R) uf = *reinterpret_cast<const bf16x8*>(&sm.ut[ln][16 * s + 8 * hh]);
        else uf = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
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
        acc = mfma_bf16(uf, __builtin_bit_cast(bf16x8, qv), acc);
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

    for (int64_t tile = t_lo; tile < t_hi; ++tile) {
      const int64_t k0 = tile * AT_K;
      __syncthreads();
      // ---- dequantize keys: thread -> (key, 32 channels) ----
      {
        const int key = tid >> 2, quarter = tid & 3, g = quarter >> 1;
        const int64_t gk = k0 + key;
        u32x4 outv[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
        if (gk < T) {
          const int64_t row = (int64_t)h * T + gk;
          const uint32_t j = seg.k_idx[row];
          const uint2 cw = *reinterpret_cast<const uint2*>(seg.k_codes + row * 32 + 8 * quarter);
          const float s = f16_bits_to_f32(seg.k_scale[row * 2 + g]);
          const uint32_t nib = (seg.k_zeros[(int64_t)h * zstride + (gk >> 1)] >> (4 * (gk & 1))) & 0xFu;
          const float z = (float)((nib >> (2 * g)) & 3u);
          const u32x4* mu = reinterpret_cast<const u32x4*>(seg.k_centroids + ((int64_t)h * NC + j) * D + 32 * quarter);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x4 mv = mu[m];
            const uint32_t cb = (m < 2 ? cw.x : cw.y) >> (16 * (m & 1));   // 8 codes
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float m0 = __uint_as_float(mv[e] << 16), m1 = __uint_as_float(mv[e] & 0xFFFF0000u);
              const float q0 = (float)((cb >> (4 * e)) & 3u), q1 = (float)((cb >> (4 * e + 2)) & 3u);
              outv[m][e] = pack_f16x2(fmaf(s, q0 - z, m0), fmaf(s, q1 - z, m1));
            }
          }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int c = 4 * quarter + m;
          reinterpret_cast<u32x4*>(sm.khat)[key * 16 + (c ^ (key & 15))] = outv[m];
        }
        if (quarter == 0) {
          u32x4 cv = {0, 0, 0, 0};
          if (psac && gk < T) {
            const int64_t row = (int64_t)h * T + gk;
            const float cs = f16_bits_to_f32(seg.k_c_scale[row]);
            const uint2 c8 = *reinterpret_cast<const uint2*>(seg.k_c + row * R);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t wd = e < 2 ? c8.x : c8.y;
              const int8_t c0 = (int8_t)((wd >> (16 * (e & 1))) & 0xFF);
              const int8_t c1 = (int8_t)((wd >> (16 * (e & 1) + 8)) & 0xFF);
              cv[e] = pack_f16x2(cs * (float)c0, cs * (float)c1);
            }
          }
          *reinterpret_cast<u32x4*>(&sm.chat[key][0]) = cv;
          *reinterpret_cast<u32x4*>(&sm.chat[key][8]) = u32x4{0, 0, 0, 0};
        }
      }
      // ---- dequantize values: thread -> (key pair, 16 channels), written transposed ----
      {
        const int kp = tid >> 3, cg = tid & 7, g = cg >> 2;
        float vv[2][16];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int64_t gk = k0 + 2 * kp + u;
#pragma unroll
          for (int c = 0; c < 16; ++c) vv[u][c] = 0.f;
          if (gk < T) {
            const int64_t row = (int64_t)h * T + gk;
            const uint32_t j = seg.v_idx[row];
            const uint32_t cw = *reinterpret_cast<const uint32_t*>(seg.v_codes + row * 32 + 4 * cg);
            const float s = f16_bits_to_f32(seg.v_scale[row * 2 + g]);
            const uint32_t nib = (seg.v_zeros[(int64_t)h * zstride + (gk >> 1)] >> (4 * (gk & 1))) & 0xFu;
            const float z = (float)((nib >> (2 * g)) & 3u);
            const u32x4* mu = reinterpret_cast<const u32x4*>(seg.v_centroids + ((int64_t)h * NC + j) * D + 16 * cg);
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const u32x4 mv = mu[m];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int c = 8 * m + 2 * e;
                const float q0 = (float)((cw >> (2 * c)) & 3u), q1 = (float)((cw >> (2 * c + 2)) & 3u);
                vv[u][c] = fmaf(s, q0 - z, __uint_as_float(mv[e] << 16));
                vv[u][c + 1] = fmaf(s, q1 - z, __uint_as_float(mv[e] & 0xFFFF0000u));
              }
            }
          }
        }
        const int slot = vslot(2 * kp);     // slot of key 2kp; 2kp + 1 is the next slot
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const int ch = 16 * cg + c;
          const int chunk = (slot >> 3) ^ ((ch >> 1) & 7);
          *reinterpret_cast<uint32_t*>(&sm.vt[ch * AT_K + chunk * 8 + (slot & 7)]) = pack_f16x2(vv[0][c], vv[1][c]);
        }
      }
      __syncthreads();

      // ---- S^T = K_ext Q_ext^T : two 32-key tiles ----
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 acc = {};
        const int key = 32 * kt + ln;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int c = 2 * s + hh;
          const f16x8 kf = reinterpret_cast<const f16x8*>(sm.khat)[key * 16 + (c ^ (key & 15))];
          acc = mfma_f16(kf, qf[s], acc);
        }
        if (psac) {
          const f16x8 cf = *reinterpret_cast<const f16x8*>(&sm.chat[key][8 * hh]);
          acc = mfma_f16(cf, qpf, acc);
        }
        sacc[kt] = acc;
      }
      // ---- online softmax (exp2 domain) ----
      const int nvalid = (int)((T - k0) < AT_K ? (T - k0) : AT_K);
      float mt = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kt + c_row(i, hh);
          if (key >= nvalid) sacc[kt][i] = -__builtin_inff();
          mt = fmaxf(mt, sacc[kt][i]);
          if (TOP1) {
            if (sacc[kt][i] > best_v) { best_v = sacc[kt][i]; best_i = (int32_t)(key_base + k0 + key); }
          }
        }
      mt = fmaxf(mt, swap32_f(mt));
      const float m_new = fmaxf(m_run, mt * sc2);
      float alpha = 1.f;
      if (m_new != -__builtin_inff()) alpha = exp2f(m_run - m_new);
      u32x4 pw[4];
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          float p0 = 0.f, p1 = 0.f;
          if (m_new != -__builtin_inff()) {
            p0 = exp2f(fmaf(sacc[kt][i], sc2, -m_new));
            p1 = exp2f(fmaf(sacc[kt][i + 1], sc2, -m_new));
          }
          lsum += p0 + p1;
          // PV k-step s = 2 kt + i / 8, element (i % 8)
          pw[2 * kt + (i >> 3)][(i & 7) >> 1] = pack_f16x2(p0, p1);
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) o_acc[c][i] *= alpha;
      // ---- O^T += V^T P ----
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int ch = 32 * c + ln;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int chunk = (2 * s + hh) ^ ((ch >> 1) & 7);
          const f16x8 vf = *reinterpret_cast<const f16x8*>(&sm.vt[ch * AT_K + chunk * 8]);
          o_acc[c] = mfma_f16(vf, __builtin_bit_cast(f16x8, pw[s]), o_acc[c]);
        }
      }
    }
    key_base += T;
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

static int attention_splits(int64_t Tq, int32_t H, int64_t total_keys) {
  const int64_t blocks = ((Tq + AT_Q - 1) / AT_Q) * H;
  int64_t want = (1024 + blocks - 1) / blocks;        // about two waves of blocks per CU
  const int64_t tiles = (total_keys + AT_K - 1) / AT_K;
  if (want > tiles / 4) want = tiles / 4;              // keep splits meaningfully long
  if (want > 32) want = 32;
  if (want < 1) want = 1;
  return (int)want;
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
  const dim3 grid((unsigned)((q->T + AT_Q - 1) / AT_Q), (unsigned)q->H, (unsigned)a.nsplit);
  if (top1) hipLaunchKernelGGL(attention_kernel<true>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(attention_kernel<false>, grid, dim3(256), 0, stream, a);
  qwm_status s = check_launch("attention");
  if (s != QWM_OK || a.nsplit == 1) return s;
  const dim3 g2((unsigned)((q->T + 1) / 2), (unsigned)q->H);
  if (top1) hipLaunchKernelGGL(attention_combine_kernel<true>, g2, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(attention_combine_kernel<false>, g2, dim3(256), 0, stream, a);
  return check_launch("attention merge");
}

}  // namespace qwm_host
