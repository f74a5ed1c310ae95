// Exact fp64 PSAC coefficients of one token, one wave per token (lane l holds
// channels 2 l and 2 l + 1): C = E U over the stored bf16 basis, c_s = the
// smallest fp16 with 127 c_s >= max|C|, C_q = clamp(rne(C / c_s), -127, 127)
// decided with exact products, and the keep test (QuantWM method step (4)) in
// its diagonal form sum_c w_c D_c (D_c - 2 e_c) < 0, D = (c_s C_q) U^T.
#pragma once

#include "common.hpp"

namespace qwm {

template <int RR>
__device__ __forceinline__ void psac_token(double e0, double e1, int lane, const uint16_t* __restrict__ Uh,
                                           bool keep_test, double w0, double w1, int8_t* __restrict__ cq,
                                           uint16_t* __restrict__ cs_out, qwm_diag* diag) {
  double u0[RR], u1[RR];
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    u0[i] = (double)bf16_bits_to_f32(Uh[(2 * lane) * RR + i]);
    u1[i] = (double)bf16_bits_to_f32(Uh[(2 * lane + 1) * RR + i]);
  }
  double C[RR];
#pragma unroll
  for (int i = 0; i < RR; ++i) C[i] = wave_sum_d(e0 * u0[i] + e1 * u1[i]);
  double m = 0.0;
#pragma unroll
  for (int i = 0; i < RR; ++i) m = fmax(m, fabs(C[i]));
  bool sat = false;
  const uint32_t csb = fp16_up_div(m, 127.0f, &sat);
  if (sat && lane == 0 && diag) atomicAdd((unsigned long long*)&diag->scale_saturations, 1ull);
  const double cs = (double)f16_bits_to_f32(csb);
  int cqi[RR];
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    int qi = 0;
    if (cs > 0.0) {
      const double Ci = C[i];
      double nq = rint(Ci / cs);
      if (Ci > (nq + 0.5) * cs) nq += 1.0;
      if (Ci < (nq - 0.5) * cs) nq -= 1.0;
      int ni = (int)nq;
      if (Ci == (nq + 0.5) * cs && (ni & 1)) ni += 1;
      else if (Ci == (nq - 0.5) * cs && (ni & 1)) ni -= 1;
      qi = ni < -127 ? -127 : (ni > 127 ? 127 : ni);
    }
    cqi[i] = qi;
  }
  bool keep = true;
  if (keep_test) {
    double D0 = 0.0, D1 = 0.0;
#pragma unroll
    for (int i = 0; i < RR; ++i) {
      const double ci = cs * (double)cqi[i];
      D0 += ci * u0[i];
      D1 += ci * u1[i];
    }
    keep = wave_sum_d(w0 * D0 * (D0 - 2.0 * e0) + w1 * D1 * (D1 - 2.0 * e1)) < 0.0;
  }
  if (lane < RR) {
    int qi = cqi[0];
#pragma unroll
    for (int i = 1; i < RR; ++i) if (lane == i) qi = cqi[i];
    cq[lane] = keep ? (int8_t)qi : (int8_t)0;
  }
  if (lane == 0) *cs_out = keep ? (uint16_t)csb : (uint16_t)0;
}

}  // namespace qwm
