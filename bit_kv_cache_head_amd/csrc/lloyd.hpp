// Lloyd iterations with distance bounds and exact integer member sums: the
// pieces the centroid build in quantize.hip drives (kernels in lloyd.hip).
#pragma once

#include "common.hpp"

namespace qwm {

// A bf16 (MB = 8) or fp32 (MB = 24) value, given by its bits, as a whole
// number of units 2^(emax - P); sc = P - emax.  The value is k 2^(e' - bias)
// with k its integer significand; the shift is in [0, P - MB] for every
// nonzero value of a head that is not flagged (clamped, to stay defined).
template <int MB>
__device__ __forceinline__ int64_t to_fixed(uint32_t b, int sc) {
  constexpr int EB = MB == 8 ? 7 : 23;            // stored significand bits
  constexpr int SB = MB == 8 ? 15 : 31;           // sign bit
  const uint32_t ef = (b >> EB) & 0xFFu;
  const uint32_t k = (b & ((1u << EB) - 1u)) | ((uint32_t)(ef != 0u) << EB);   // 0 for a zero
  int shift = (int)(ef > 1u ? ef : 1u) - (127 + EB) + sc;
  shift = shift < 0 ? 0 : (shift > 62 ? 62 : shift);
  const int64_t m = (int64_t)((uint64_t)k << shift);
  const int64_t neg = -(int64_t)((b >> SB) & 1u);   // 0 or -1
  return (m ^ neg) - neg;
}

}  // namespace qwm

namespace qwm_host {

// Per-build state of the bounded Lloyd iteration, carved from the centroid
// workspace.
struct LloydState {
  // per (head, channel): the largest and smallest binary exponent (frexp
  // convention, x = m 2^e with 1/2 <= |m| < 1) over the nonzero channel values
  // of the head's finite rows; per head: 1 when some value is not a whole
  // multiple of the fixed-point unit, so the head takes the fp64 path
  int32_t* emax;    // [H][128]
  int32_t* emin;    // [H][128]
  int32_t* hflag;   // [H]
  // per (head, centroid, channel): member sums in units of 2^(emax - P); counts
  int64_t* sums;    // [H][256][128]
  int32_t* cnt;     // [H][256]
  // per (head, centroid): an upper bound on how far the last mean update moved it
  float* delta;     // [H][256]
  // per token-head: upper bound on the distance to its centroid, lower bound on
  // the distance to every other centroid
  float* ub;        // [H][T]
  float* lb;        // [H][T]
  // per head: tokens whose bounds no longer settle their centroid
  int32_t* wl;      // [H][T]
  int32_t* wl_cnt;  // [H]
  // changed assignments of an iteration: (h T + t, old | new << 8)
  uint2* chg;       // [H T]
  int32_t* chg_cnt; // [1]
  int32_t P;        // fixed-point unit 2^(emax - P), P = min(62 - bit length of T, 48): no sum of
                    // T values leaves 63 bits, and a sum of 32 is exact in fp64
  int32_t MB;       // significant bits of a token value (8 bf16, 24 fp32)
};

size_t lloyd_state_bytes(int64_t T, int32_t H);
LloydState lloyd_state_carve(char*& p, int64_t T, int32_t H, int32_t dtype);

// Once per build: exponent ranges of every (head, channel) and the per-head flag.
qwm_status lloyd_scan(const qwm_tokens* x, const LloydState& s, hipStream_t stream);
// Later iterations: the tokens whose bounds no longer hold go to the per-head
// lists (every token of a flagged head); the rest get their updated bounds.
qwm_status lloyd_bounds(const qwm_tokens* x, const uint8_t* assign, const uint32_t* excl, int64_t excl_words,
                        const LloydState& s, hipStream_t stream);
// Later iterations: the recorded changes applied to the sums and counts.
qwm_status lloyd_apply_changes(const qwm_tokens* x, const LloydState& s, hipStream_t stream);
// New means of the heads not flagged (an empty cluster keeps its centroid) and
// how far each moved.
qwm_status lloyd_finalize(const qwm_tokens* x, const LloydState& s, const uint16_t* cur, uint16_t* out,
                          hipStream_t stream);

}  // namespace qwm_host
