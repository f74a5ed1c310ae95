// Reconstruction of a packed chunk in BF16: the decoder of QuantWM App. D.1
// and Fig. 9 (residual unpacking, parameter reconstruction, centroid gather
// and PSAC accumulation into temporary BF16 keys and values that a dense
// attention then reads).  The fused attention kernel never forms these rows;
// this path exists to compare the two designs.  The same file holds the
// centroid residual used by the multi-stage (progressive) codec.
//
// Each element is computed exactly in fp64 and rounded once to bf16 (RNE):
//   K_hat[t][c] = mu_k[idx][c] + s_g (q - z_g) + sum_r (c_s C_r) U[c][r]
//   V_hat[t][c] = mu_v[idx][c] + s_g (q - z_g)
// (mu bf16, s fp16, q and z 2-bit, c_s fp16, C int8, U bf16: every product is
// exact in fp64, and so are the sums for values of sane dynamic range).
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "quantwm.h"

namespace qwm {

struct DecodeArgs {
  qwm_segment seg;      // device pointers of the packed chunk
  int32_t H;
  uint16_t* kout; uint16_t* vout;
  int64_t ost, osh;     // output element strides (token, head); channel stride 1
};

constexpr int DEC_TOK = 32;   // tokens per block: 8 threads per token, 16 channels each

// Grid (ceil(T / 32), H), 256 threads.  Thread (token tid / 8, channels
// 16 (tid % 8) .. +16): the 16 channels' codes are one 32-bit word of the
// token's code row (channel 16 b + j at bits 2 j).
template <int RK>   // PSAC rank of the chunk: 8, 16 or 32
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  const int h = blockIdx.y, tid = threadIdx.x, tk = tid >> 3, cb = tid & 7;
  const qwm_segment& g = a.seg;
  const int64_t T = g.T;
  __shared__ double U[D][RK];
  const bool psac = g.U != nullptr;
  if (psac)
    for (int e = tid; e < D * RK; e += 256) U[e / RK][e % RK] = (double)bf16_bits_to_f32(g.U[(int64_t)h * D * RK + e]);
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * DEC_TOK + tk;
  if (t >= T) return;
  const int64_t ht = (int64_t)h * T + t;
  const int grp = cb >> 2;   // 64-channel group of this thread's channels
  const int zsh = 4 * (int)(t & 1) + 2 * grp;
  const int64_t zrow = (int64_t)h * zeros_stride(T) + (t >> 1);
  uint16_t ko[16], vo[16];
  {
    const uint32_t code = *reinterpret_cast<const uint32_t*>(g.k_codes + ht * 32 + 4 * cb);
    // group step: fp16, or a two-level step code times its power-of-two second level
    const double s = g.k_scale2 ? (double)reinterpret_cast<const uint8_t*>(g.k_scale)[ht * 2 + grp] *
                                      (double)f16_bits_to_f32(g.k_scale2[h * 2 + grp])
                                : (double)f16_bits_to_f32(g.k_scale[ht * 2 + grp]);
    const int z = (g.k_zeros[zrow] >> zsh) & 3;
    const uint16_t* mu = g.k_centroids + ((int64_t)h * NC + g.k_idx[ht]) * D + 16 * cb;
    const u32x4 m0 = *reinterpret_cast<const u32x4*>(mu), m1 = *reinterpret_cast<const u32x4*>(mu + 8);
    double cc[RK];
    if (psac) {
      // the key's coefficients: dense rows, or from the compacted layout
      const int8_t* crow = g.k_c + ht * RK;
      const uint16_t* csp = g.k_c_scale + ht;
      bool have = true;
      if (g.k_cdir) {
        const qwm_cdir e = g.k_cdir[h];
        const uint8_t* base = g.k_carena + e.offset;
        if (e.layout == QWM_LAYOUT_DENSE) {
          crow = reinterpret_cast<const int8_t*>(base) + t * RK;
          csp = reinterpret_cast<const uint16_t*>(base + ((T * RK + 15) & ~(int64_t)15)) + t;
        } else if (e.layout == QWM_LAYOUT_SPARSE) {
          const int64_t nw = (T + 63) / 64;
          const uint64_t word = reinterpret_cast<const uint64_t*>(base)[t >> 6];
          const uint32_t pre = reinterpret_cast<const uint32_t*>(base + ((nw * 8 + 15) & ~(int64_t)15))[t >> 6];
          const int b = (int)(t & 63);
          have = (word >> b) & 1ull;
          const int64_t ent = (int64_t)pre + __popcll(word & ((1ull << b) - 1ull));
          const uint8_t* cbase = base + ((nw * 8 + 15) & ~(int64_t)15) + ((nw * 4 + 15) & ~(int64_t)15);
          crow = reinterpret_cast<const int8_t*>(cbase) + ent * RK;
          csp = reinterpret_cast<const uint16_t*>(cbase + (((int64_t)e.count * RK + 15) & ~(int64_t)15)) + ent;
        } else {
          have = false;
        }
      }
      const double cs = have ? (double)f16_bits_to_f32(*csp) : 0.0;
#pragma unroll
      for (int r = 0; r < RK; ++r) cc[r] = have ? cs * (double)crow[r] : 0.0;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t w = j < 8 ? m0[j >> 1] : m1[(j - 8) >> 1];
      const double m = (double)((j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16));
      const int q = (int)((code >> (2 * j)) & 3u);
      double v = m + s * (double)(q - z);
      if (psac) {
#pragma unroll
        for (int r = 0; r < RK; ++r) v += cc[r] * U[16 * cb + j][r];
      }
      ko[j] = (uint16_t)f64_to_bf16_bits(v);
    }
  }
  {
    const uint32_t code = *reinterpret_cast<const uint32_t*>(g.v_codes + ht * 32 + 4 * cb);
    const double s = g.v_scale2 ? (double)reinterpret_cast<const uint8_t*>(g.v_scale)[ht * 2 + grp] *
                                      (double)f16_bits_to_f32(g.v_scale2[h * 2 + grp])
                                : (double)f16_bits_to_f32(g.v_scale[ht * 2 + grp]);
    const int z = (g.v_zeros[zrow] >> zsh) & 3;
    const uint16_t* mu = g.v_centroids + ((int64_t)h * NC + g.v_idx[ht]) * D + 16 * cb;
    const u32x4 m0 = *reinterpret_cast<const u32x4*>(mu), m1 = *reinterpret_cast<const u32x4*>(mu + 8);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t w = j < 8 ? m0[j >> 1] : m1[(j - 8) >> 1];
      const double m = (double)((j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16));
      const int q = (int)((code >> (2 * j)) & 3u);
      vo[j] = (uint16_t)f64_to_bf16_bits(m + s * (double)(q - z));
    }
  }
  u32x4 kw[2], vw[2];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kw[e >> 2][e & 3] = (uint32_t)ko[2 * e] | ((uint32_t)ko[2 * e + 1] << 16);
    vw[e >> 2][e & 3] = (uint32_t)vo[2 * e] | ((uint32_t)vo[2 * e + 1] << 16);
  }
  const int64_t o = t * a.ost + (int64_t)h * a.osh + 16 * cb;
  *reinterpret_cast<u32x4*>(a.kout + o) = kw[0];
  *reinterpret_cast<u32x4*>(a.kout + o + 8) = kw[1];
  *reinterpret_cast<u32x4*>(a.vout + o) = vw[0];
  *reinterpret_cast<u32x4*>(a.vout + o + 8) = vw[1];
}

// The residual of every token against its assigned centroid, fp32:
// out[t][h][c] = fl32(x[t][h][c] - C[h][idx[h][t]][c]) -- the centroid
// subtraction of QVG's smoothing step (QVG summary Sec. 2A), which its
// progressive residual quantization repeats stage by stage (Sec. 2B).
// Grid (ceil(T / 32), H), 256 threads: token tid / 8, channels 16 (tid % 8) .. +16.
struct ResidArgs {
  const void* x; int32_t dtype; int64_t T; int64_t st, sh;
  const uint16_t* C; const uint8_t* idx;
  float* out; int64_t ost, osh;
};

__global__ __launch_bounds__(256) void centroid_residual_kernel(ResidArgs a) {
  const int h = blockIdx.y, tk = threadIdx.x >> 3, cb = threadIdx.x & 7;
  const int64_t t = (int64_t)blockIdx.x * DEC_TOK + tk;
  if (t >= a.T) return;
  const uint16_t* mu = a.C + ((int64_t)h * NC + a.idx[(int64_t)h * a.T + t]) * D + 16 * cb;
  const u32x4 m0 = *reinterpret_cast<const u32x4*>(mu), m1 = *reinterpret_cast<const u32x4*>(mu + 8);
  float x[16];
  const int64_t xo = t * a.st + (int64_t)h * a.sh + 16 * cb;
  if (a.dtype == QWM_BF16) {
    const uint16_t* xp = static_cast<const uint16_t*>(a.x) + xo;
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(xp), v1 = *reinterpret_cast<const u32x4*>(xp + 8);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t w = j < 8 ? v0[j >> 1] : v1[(j - 8) >> 1];
      x[j] = (j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    }
  } else {
    const float* xp = static_cast<const float*>(a.x) + xo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(xp + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q + e] = v[e];
    }
  }
  f32x4 o[4];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t w = j < 8 ? m0[j >> 1] : m1[(j - 8) >> 1];
    const float m = (j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    o[j >> 2][j & 3] = x[j] - m;
  }
  float* op = a.out + t * a.ost + (int64_t)h * a.osh + 16 * cb;
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<f32x4*>(op + 4 * q) = o[q];
}

}  // namespace qwm

namespace qwm_host {
using namespace qwm;

qwm_status launch_decode(const qwm_segment* seg, int32_t H, uint16_t* k_out, uint16_t* v_out, int64_t ost,
                         int64_t osh, hipStream_t stream) {
  DecodeArgs a{};
  a.seg = *seg;
  a.H = H; a.kout = k_out; a.vout = v_out; a.ost = ost; a.osh = osh;
  const dim3 grid((unsigned)((seg->T + DEC_TOK - 1) / DEC_TOK), (unsigned)H);
  if (seg->r == 32) hipLaunchKernelGGL(decode_kernel<32>, grid, dim3(256), 0, stream, a);
  else if (seg->r == 16) hipLaunchKernelGGL(decode_kernel<16>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(decode_kernel<8>, grid, dim3(256), 0, stream, a);
  return check_launch("chunk decode");
}

qwm_status launch_centroid_residual(const qwm_tokens* x, const uint16_t* centroids, const uint8_t* idx, float* out,
                                   int64_t ost, int64_t osh, hipStream_t stream) {
  ResidArgs a{};
  a.x = x->ptr; a.dtype = x->dtype; a.T = x->T; a.st = x->stride_t; a.sh = x->stride_h;
  a.C = centroids; a.idx = idx; a.out = out; a.ost = ost; a.osh = osh;
  const dim3 grid((unsigned)((x->T + DEC_TOK - 1) / DEC_TOK), (unsigned)x->H);
  hipLaunchKernelGGL(centroid_residual_kernel, grid, dim3(256), 0, stream, a);
  return check_launch("centroid residual");
}

}  // namespace qwm_host
