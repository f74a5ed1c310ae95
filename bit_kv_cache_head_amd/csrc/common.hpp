// Shared device helpers for libquantwm (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "quantwm.h"

namespace qwm {

constexpr int D = 128;          // head dim
constexpr int G = 2;            // 64-channel groups per token
constexpr int NC = 256;         // centroids
constexpr int R = 8;            // PSAC rank
constexpr int WAVE = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// ---------------------------------------------------------------------------
// MFMA 32x32x16 (bf16 / fp16 inputs, fp32 accumulate).  Operand layouts
// (lane l, h = l / 32):  A[m][k]: m = l % 32, k = 8h + j (j = 0..7);
// B[k][n]: n = l % 32, k = 8h + j;  C[m][n]: n = l % 32, register i holds
// m = 8 (i / 4) + 4h + (i % 4).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int c_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// ---------------------------------------------------------------------------
// Number formats.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp64 -> bf16 bits, round to nearest even directly from double (no double rounding).
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  if (x == 0.0) return (__double_as_longlong(x) < 0) ? 0x8000u : 0u;
  int e;
  (void)frexp(x, &e);                       // x = m 2^e, 0.5 <= |m| < 1
  int q = e - 8;
  if (q < -133) q = -133;
  double y = rint(ldexp(x, -q));            // exact scaling, half-to-even
  float f = (float)ldexp(y, q);             // <= 8 significant bits: exact in fp32
  return __float_as_uint(f) >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)b);
  return (float)h;
}

// Smallest binary16 h >= 0 with m * h >= x (x >= 0, m a small positive integer).
// Returns bits; *sat set when x > m * 65504 (then h = 65504).
__device__ __forceinline__ uint32_t fp16_up_div(double x, float m, bool* sat) {
  *sat = false;
  if (!(x > 0.0)) return 0u;
  if (x > (double)m * 65504.0) { *sat = true; return 0x7BFFu; }
  float y = (float)(x / (double)m);
  uint32_t hb = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y);
  if (hb > 0x7BFFu) hb = 0x7BFFu;
  // exact fix-up: (double)m * h is exact (11-bit h times a small integer)
  for (int it = 0; it < 2; ++it) {
    if ((double)m * (double)f16_bits_to_f32(hb) < x) hb += 1u;
    if (hb > 0u && (double)m * (double)f16_bits_to_f32(hb - 1u) >= x) hb -= 1u;
  }
  return hb;
}

// Round-half-to-even of the exact quotient a / b, b > 0 a binary16 value held
// in fp32, |a / b| <= 4096.  (n +- 1/2) * b is exact in fp32.
__device__ __forceinline__ int rne_quot(float a, float b) {
  float n = rintf(a / b);
  if (a > (n + 0.5f) * b) n += 1.0f;
  if (a < (n - 0.5f) * b) n -= 1.0f;
  int ni = (int)n;
  if (a == (n + 0.5f) * b && (ni & 1)) ni += 1;
  else if (a == (n - 0.5f) * b && (ni & 1)) ni -= 1;
  return ni;
}

__device__ __forceinline__ bool is_finite_f(float x) { return __builtin_isfinite(x); }

// Largest float below a finite x.
__device__ __forceinline__ float prev_float(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) == 0u) return __uint_as_float(0x80000001u);
  return __uint_as_float((u & 0x80000000u) ? u + 1u : u - 1u);
}

// Row stride of a chunk's zeros array: ceil(T/2) bytes rounded up to 4.
__host__ __device__ __forceinline__ int64_t zeros_stride(int64_t T) { return (((T + 1) / 2) + 3) & ~(int64_t)3; }

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float swap32_f(float v) { return __shfl_xor(v, 32, 64); }
__device__ __forceinline__ uint32_t swap32_u(uint32_t v) { return __shfl_xor(v, 32, 64); }
__device__ __forceinline__ double swap32_d(double v) { return __shfl_xor(v, 32, 64); }

// Lanes l and l ^ 32 (v_permlane32_swap, no LDS round trip).  The swap of a
// value with itself returns s[0] = lane l % 32's value and s[1] = lane
// (l % 32) + 32's value on both lanes, so the pair reductions below compute the
// same result, in the same order, on both lanes.
__device__ __forceinline__ float lanepair_sum(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float lanepair_min(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fminf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float lanepair_max(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
// the value held by lane l ^ 32 (hh = l / 32)
__device__ __forceinline__ float lanepair_other(float v, int hh) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(hh ? s[0] : s[1]);
}

__device__ __forceinline__ float wave_max_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace qwm

// ---------------------------------------------------------------------------
// Host-side status plumbing.
// ---------------------------------------------------------------------------
namespace qwm_host {
void set_error(const std::string& msg);
qwm_status fail(qwm_status s, const std::string& msg);
qwm_status check_launch(const char* what);
}  // namespace qwm_host
