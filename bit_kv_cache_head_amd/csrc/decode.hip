// Reconstruction of a packed chunk in BF16: the decoder of QuantWM App. D.1
// and Fig. 9 (residual unpacking, parameter reconstruction, centroid gather
// and PSAC accumulation into temporary BF16 keys and values that a dense
// attention then reads).  The fused attention kernel never forms these rows;
// this path exists to compare the two designs.
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
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  const int h = blockIdx.y, tid = threadIdx.x, tk = tid >> 3, cb = tid & 7;
  const qwm_segment& g = a.seg;
  const int64_t T = g.T;
  __shared__ double U[D][R];
  const bool psac = g.U != nullptr;
  if (psac)
    for (int e = tid; e < D * R; e += 256) U[e / R][e % R] = (double)bf16_bits_to_f32(g.U[(int64_t)h * D * R + e]);
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
    const double s = (double)f16_bits_to_f32(g.k_scale[ht * 2 + grp]);
    const int z = (g.k_zeros[zrow] >> zsh) & 3;
    const uint16_t* mu = g.k_centroids + ((int64_t)h * NC + g.k_idx[ht]) * D + 16 * cb;
    const u32x4 m0 = *reinterpret_cast<const u32x4*>(mu), m1 = *reinterpret_cast<const u32x4*>(mu + 8);
    double cc[R];
    if (psac) {
      const double cs = (double)f16_bits_to_f32(g.k_c_scale[ht]);
#pragma unroll
      for (int r = 0; r < R; ++r) cc[r] = cs * (double)g.k_c[ht * R + r];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t w = j < 8 ? m0[j >> 1] : m1[(j - 8) >> 1];
      const double m = (double)((j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16));
      const int q = (int)((code >> (2 * j)) & 3u);
      double v = m + s * (double)(q - z);
      if (psac) {
#pragma unroll
        for (int r = 0; r < R; ++r) v += cc[r] * U[16 * cb + j][r];
      }
      ko[j] = (uint16_t)f64_to_bf16_bits(v);
    }
  }
  {
    const uint32_t code = *reinterpret_cast<const uint32_t*>(g.v_codes + ht * 32 + 4 * cb);
    const double s = (double)f16_bits_to_f32(g.v_scale[ht * 2 + grp]);
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

}  // namespace qwm

namespace qwm_host {
using namespace qwm;

qwm_status launch_decode(const qwm_segment* seg, int32_t H, uint16_t* k_out, uint16_t* v_out, int64_t ost,
                         int64_t osh, hipStream_t stream) {
  DecodeArgs a{};
  a.seg = *seg;
  a.H = H; a.kout = k_out; a.vout = v_out; a.ost = ost; a.osh = osh;
  const dim3 grid((unsigned)((seg->T + DEC_TOK - 1) / DEC_TOK), (unsigned)H);
  hipLaunchKernelGGL(decode_kernel, grid, dim3(256), 0, stream, a);
  return check_launch("chunk decode");
}

}  // namespace qwm_host
