// Top-1 key of every Query over unquantized BF16 keys: the reference side of
// the token-shift metric (QuantWM v2 Sec. 5.3 and the rainbus digest's token
// shift analysis: how often the key a Query attends to most changes when the
// cache is quantized).
//
//   top1[h][i] = argmax_j  q_i . k_j      (lowest j on ties)
//
// Logits are MFMA 32x32x16 bf16 products (exact) accumulated in fp32.  One
// block = one head x 128 Queries (4 waves x 32); every wave walks all keys in
// 32-key tiles, the next tile's fragments loaded while the current one is
// multiplied.
#include "common.hpp"

namespace qwm {

constexpr int RT_W = 4;
constexpr int RT_Q = 32 * RT_W;

struct RefArgs {
  const uint16_t* q; int64_t Tq; int64_t qst; int64_t qsh;
  const uint16_t* k; int64_t Tk; int64_t kst; int64_t ksh;
  int32_t* top1;
};

__global__ __launch_bounds__(64 * RT_W) void reference_top1_kernel(RefArgs a) {
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hh = lane >> 5, ln = lane & 31;
  const int64_t qi = (int64_t)blockIdx.x * RT_Q + wv * 32 + ln;
  const bool qvalid = qi < a.Tq;
  const uint16_t* qrow = a.q + (int64_t)h * a.qsh + (qvalid ? qi : 0) * a.qst;
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const u32x4 v = qvalid ? *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
    qf[s] = __builtin_bit_cast(bf16x8, v);
  }
  const uint16_t* kh = a.k + (int64_t)h * a.ksh;
  const int64_t ntiles = (a.Tk + 31) / 32;
  // key fragments of one tile: lane (key ln, half hh) holds channels 16 s + 8 hh .. +8
  auto load = [&](int64_t t, bf16x8 (&f)[8]) {
    int64_t key = t * 32 + ln;
    key = key < a.Tk ? key : a.Tk - 1;           // clamped; masked below
    const uint16_t* krow = kh + key * a.kst;
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 16 * s + 8 * hh));
  };
  float best_v = -__builtin_inff();
  int32_t best_i = 0x7FFFFFFF;
  bf16x8 cur[8], nxt[8];
  load(0, cur);
  for (int64_t t = 0; t < ntiles; ++t) {
    load(t + 1 < ntiles ? t + 1 : t, nxt);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma_bf16(cur[s], qf[s], acc);
    // lane (query ln, half hh) holds keys t*32 + c_row(i, hh), increasing in i
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t key = t * 32 + c_row(i, hh);
      if (key < a.Tk && acc[i] > best_v) { best_v = acc[i]; best_i = (int32_t)key; }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) cur[s] = nxt[s];
  }
  const float ov = swap32_f(best_v);
  const int32_t oi = (int32_t)swap32_u((uint32_t)best_i);
  if (ov > best_v || (ov == best_v && oi < best_i)) { best_v = ov; best_i = oi; }
  if (qvalid && hh == 0) a.top1[(int64_t)h * a.Tq + qi] = best_i;
}

}  // namespace qwm

namespace qwm_host {
using namespace qwm;

qwm_status launch_reference_top1(const qwm_tokens* q, const qwm_tokens* k, int32_t* top1, hipStream_t stream) {
  RefArgs a{};
  a.q = static_cast<const uint16_t*>(q->ptr); a.Tq = q->T; a.qst = q->stride_t; a.qsh = q->stride_h;
  a.k = static_cast<const uint16_t*>(k->ptr); a.Tk = k->T; a.kst = k->stride_t; a.ksh = k->stride_h;
  a.top1 = top1;
  const dim3 grid((unsigned)((q->T + RT_Q - 1) / RT_Q), (unsigned)q->H);
  hipLaunchKernelGGL(reference_top1_kernel, grid, dim3(64 * RT_W), 0, stream, a);
  return check_launch("reference top-1");
}

}  // namespace qwm_host
