// Attention over the compressed cache (QuantWM method section ¶1: logits
// Q K0_hat^T + (Q U_r) C^T; Sec. 3.3 logits Q K^T / sqrt(d); App. D.1 / Fig. 9
// on-demand reconstruction of keys and values, here fused into the kernel).
//
// Work unit: one head, 256 queries (8 waves x 32), one share of every
// segment's 64-key tiles.  Tiles flow through a register pipeline: the index
// bytes and packed bytes of tile t+3 and the centroid rows of tile t+2 are in
// flight, tile t+1 is dequantized from registers into the second LDS buffer
// (fp16: K0_hat rows, the PSAC coefficients c_scale * c as 8 extra
// contraction channels, V_hat transposed), while tile t runs
//   S^T = [K0_hat | C_hat] [Q | Q U]^T     (MFMA 32x32x16 f16, contraction 128 + 16)
//   online softmax in fp32 (exp2 domain, lazy rescaling)
//   O^T += V_hat^T P                       (MFMA 32x32x16 f16)
// Split-key partial results are merged by a second kernel.  Work units are
// mapped to blocks so that one head's units share an XCD (and its L2).
#include <algorithm>

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
  const qwm_segment* segs; int32_t n_segs; int32_t nsplit;   // segs: the workspace copy of the descriptors; nsplit: splits of its keys
  int32_t nqb; int32_t units;
  // The active BF16 chunk, attended by the dense units: key t of head h is
  // ka[t * kast + h * kash] (va alike), global key index kbase_a + t.  Units
  // [0, units_p) are packed units, [units_p, units) dense ones (nsplit_a splits).
  const uint16_t* ka; const uint16_t* va; int64_t kast, kash, vast, vash; int64_t Ta; int64_t kbase_a;
  int32_t units_p; int32_t nsplit_a;
  int32_t nparts;         // partial sets: nsplit (+ nsplit_a); one set means no partials
  float scale;
  const uint16_t* tabs;   // fp16 centroid tables [seg][H][2][256][128]: K (channel-permuted), V
  const uint16_t* ut;     // fp16 basis fragments [seg][H][UT_ROWS][8][2][8] (rows < the rank written), see attention_tables_kernel
  // final outputs (nparts == 1)
  float* out; float* lse; int32_t* top1; int32_t H;
  // partial outputs (nparts > 1): [part][H][Tq][D], [part][H][Tq] x (m, l), top value / index
  float* po; float* pm; float* pl; float* ptv; int32_t* pti;
};

// K0_hat rows use a channel order in which the 32-bit word m of every
// 16-channel block holds channels (m, m + 8): the INT2 codes of those two
// channels sit 16 bits apart in the packed code word, so one shift and one
// mask put both into the two fp16 halves.  Q uses the same order (the
// contraction does not care); V_hat keeps the natural order.
// Rows are padded by 16 bytes: 16 lanes reading the same 16-byte column of 16
// consecutive rows then cover all 64 banks once, and every LDS address is a
// per-thread base plus a compile-time offset.
constexpr int KSTR = 2 * D + 16;      // bytes per K0_hat row
constexpr int VSTR = 2 * AT_K + 16;   // bytes per V_hat^T row
// NPK: PSAC k-steps of 16 coefficients (1: ranks 8 and 16; 2: rank 32)
// PSAC coefficients sit in 2 NPK planes of 8 per key (16 bytes), planes
// padded by 128 bytes: the 16 lanes of an operand read cover 256 contiguous
// bytes, and the coefficient stores of a wave (8 keys x 8 threads) fall in 64
// different banks.
constexpr int CPL = AT_K * 16 + 128;   // bytes per coefficient plane
template <int NPK>
struct AttnBuf {
  uint8_t khat[AT_K * KSTR];       // [key][128 permuted channels] fp16
  uint8_t vt[D * VSTR];            // [channel][64 keys in vslot order] fp16
  uint8_t chat[2 * NPK * CPL];     // [plane q][key][8] fp16: c_scale * c for coefficients 8 q .. 8 q + 7 (zeros past the rank)
};
constexpr int UT_ROWS = QWM_MAX_RANK;   // basis rows per (segment, head) in the fragment buffer

// slot of a key in the transposed V tile: bits 2 and 3 swapped (matches the
// register order of the probabilities produced by the S^T MFMA)
__device__ __forceinline__ int vslot(int key) {
  return (key & ~0xC) | ((key & 4) << 1) | ((key & 8) >> 1);
}
// Byte offset of (channel ch, slot) in the V_hat^T tile: the 16-byte chunks of
// row ch are XOR-swizzled by (ch / 16) % 8, so the dequantizing threads (16
// channel groups x 8 keys per wave) spread their 32-bit stores over the banks,
// while the MFMA operand reads (16 consecutive rows, one chunk) stay
// conflict-free and keep a per-lane base plus compile-time offsets.
__device__ __forceinline__ int vt_offset(int ch, int slot) {
  return ch * VSTR + 16 * ((slot >> 3) ^ ((ch >> 4) & 7)) + 2 * (slot & 7);
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
// The same with both masks in registers (one v_and_or_b32 instead of an AND
// and an OR: a VOP3 instruction encodes only one literal).
struct CodeMasks {
  uint32_t q, e;   // 0x00030003, 0x64006400
};
__device__ __forceinline__ CodeMasks code_masks() {
  CodeMasks m;
  asm("v_mov_b32 %0, 0x30003" : "=v"(m.q));
  asm("v_mov_b32 %0, 0x64006400" : "=v"(m.e));
  return m;
}
__device__ __forceinline__ h2 code_pair(uint32_t w, int sh, const CodeMasks& m) {
  return as_h2(((w >> sh) & m.q) | m.e);
}

// ---------------------------------------------------------------------------
// Per-call set-up of the segments, from a batch of host descriptors passed by
// value (kernel arguments, so the caller's array may die when the call
// returns): the descriptors go to the device array the attention kernel reads;
// every segment's centroid tables become fp16 copies (exact for bf16 values in
// fp16's normal range), and its basis becomes the A operand of (U^T)(Q^T): for
// basis vector n, k-step s and lane half hh, the 8 values U[c][n] at the
// channels c = 16 s + 4 hh + j / 2 + 8 (j % 2) (j = 0..7) that the Query
// fragments hold in that position.  Zeros for a segment without a basis.
// Grid (count * H, 8): block (sh, y) converts centroids 32 y .. +32 of local
// segment sh / H, head sh % H, thread (centroid 32 y + tid / 8, channels
// 16 (tid % 8) .. +16), so a wave reads 8 whole rows; blocks y = 0 also write
// the basis fragments, and block (local segment, head 0, y = 0) its descriptor.
// ---------------------------------------------------------------------------
constexpr int SEG_BATCH = 20;   // descriptors per launch (3 KiB of kernel arguments)
struct SegBatch {
  qwm_segment s[SEG_BATCH];
  int32_t first, count;
};

__global__ __launch_bounds__(256) void attention_tables_kernel(SegBatch b, int32_t H, qwm_segment* __restrict__ dsegs,
                                                               uint16_t* __restrict__ tabs, uint16_t* __restrict__ ut) {
  const int local = (int)blockIdx.x / H, h = (int)blockIdx.x % H, tid = threadIdx.x;
  const int seg = b.first + local, sh = seg * H + h;
  const int j = 32 * (int)blockIdx.y + (tid >> 3), blk = tid & 7;
  const qwm_segment& sg = b.s[local];
  if (blockIdx.y == 0 && h == 0 && tid < (int)(sizeof(qwm_segment) / 8))
    reinterpret_cast<uint64_t*>(dsegs + seg)[tid] = reinterpret_cast<const uint64_t*>(&sg)[tid];
  if (blockIdx.y == 0) {
    // basis rows n < r: four consecutive fragment values per thread and pass
    // (same n, s, hh; j' = 4 (i % 2) .. +4); rows past the rank are never read
    const int rk = sg.r;
    for (int i = 4 * tid; i < rk * D; i += 4 * 256) {
      const int n = i >> 7, s = (i >> 4) & 7, hf = (i >> 3) & 1;
      uint32_t w[2] = {0u, 0u};
      if (sg.U != nullptr) {
        const uint16_t* Uh = sg.U + (int64_t)h * D * rk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = (i & 7) + e;
          const int c = 16 * s + 4 * hf + (jj >> 1) + 8 * (jj & 1);
          const uint16_t v = __builtin_bit_cast(uint16_t, (_Float16)__uint_as_float((uint32_t)Uh[c * rk + n] << 16));
          w[e >> 1] |= (uint32_t)v << (16 * (e & 1));
        }
      }
      *reinterpret_cast<uint2*>(ut + (int64_t)sh * UT_ROWS * D + i) = make_uint2(w[0], w[1]);
    }
  }
  const u32x4* kr = reinterpret_cast<const u32x4*>(sg.k_centroids + ((int64_t)h * NC + j) * D);
  const u32x4* vr = reinterpret_cast<const u32x4*>(sg.v_centroids + ((int64_t)h * NC + j) * D);
  u32x4* kt = reinterpret_cast<u32x4*>(tabs + ((int64_t)sh * 2 + 0) * TAB_ELEMS + (int64_t)j * D);
  u32x4* vtb = reinterpret_cast<u32x4*>(tabs + ((int64_t)sh * 2 + 1) * TAB_ELEMS + (int64_t)j * D);
  {
    const u32x4 a = kr[2 * blk], b = kr[2 * blk + 1];   // channels 16 blk + 0..7, + 8..15
    u32x4 o0, o1;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      // word m = (channel m, channel m + 8)
      const uint32_t lo = (m & 1) ? (a[m >> 1] >> 16) : (a[m >> 1] & 0xFFFFu);
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

__device__ __forceinline__ int ntiles(int64_t T) { return (int)((T + AT_K - 1) / AT_K); }

// ---------------------------------------------------------------------------
// Tile positions.  The tiles of all segments, in segment order, form one
// sequence; split p of nsplit owns a contiguous share of it.  A position is
// wave-uniform (scalar registers).
// ---------------------------------------------------------------------------
struct Pos {
  int seg;          // segment index
  int tile;         // tile index within the segment
  int64_t kbase;    // global index of the segment's first key
};

__device__ __forceinline__ int64_t sfl64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Number of tiles over all segments (every lane gets the total).
__device__ int count_tiles(const AttnArgs& a, int lane) {
  int tot = 0;
  for (int base = 0; base < a.n_segs; base += 64) {
    const int s = base + lane;
    int nt = s < a.n_segs ? ntiles(a.segs[s].T) : 0;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) nt += __shfl_xor(nt, d, 64);
    tot += nt;
  }
  return __builtin_amdgcn_readfirstlane(tot);
}

// Position of tile g of the sequence (0 <= g < total): a prefix scan of the
// per-segment tile counts, 64 segments at a time.
__device__ Pos locate(const AttnArgs& a, int g, int lane) {
  int carry = 0;
  int64_t kcarry = 0;
  for (int base = 0; base < a.n_segs; base += 64) {
    const int s = base + lane;
    const int64_t T = s < a.n_segs ? a.segs[s].T : 0;
    const int nt = ntiles(T);
    int inc = nt;
    int64_t kinc = T;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(inc, d, 64);
      const int64_t ko = __shfl_up(kinc, d, 64);
      if (lane >= d) { inc += o; kinc += ko; }
    }
    const uint64_t hit = __ballot(carry + inc > g);
    if (hit != 0) {
      const int l = __ffsll((unsigned long long)hit) - 1;
      Pos p;
      p.seg = base + l;
      p.tile = g - carry - __shfl(inc - nt, l, 64);
      p.kbase = kcarry + __shfl(kinc - T, l, 64);
      p.seg = __builtin_amdgcn_readfirstlane(p.seg);
      p.tile = __builtin_amdgcn_readfirstlane(p.tile);
      p.kbase = sfl64(p.kbase);
      return p;
    }
    carry += __shfl(inc, 63, 64);
    kcarry += __shfl(kinc, 63, 64);
  }
  Pos p;
  p.seg = a.n_segs - 1; p.tile = 0; p.kbase = 0;   // not reached for g < total
  return p;
}

// Keys of segment s; a dense unit's only segment is the active chunk.
template <bool DENSE>
__device__ __forceinline__ int64_t seg_T(const AttnArgs& a, int s) {
  if constexpr (DENSE) return a.Ta;
  else return seg_at(a, s).T;
}

// The next tile (the caller knows one exists); T = keys of p's segment.
template <bool DENSE>
__device__ __forceinline__ Pos advance(const AttnArgs& a, Pos p, int64_t T) {
  if constexpr (DENSE) {
    p.tile += 1;
    return p;
  }
  p.tile += 1;
  while ((int64_t)p.tile * AT_K >= T && p.seg + 1 < a.n_segs) {
    p.kbase += T;
    p.seg += 1;
    p.tile = 0;
    T = seg_at(a, p.seg).T;
  }
  return p;
}

// ---------------------------------------------------------------------------
// Loads.  Every packed array is read through a buffer descriptor whose base
// is the tile's first row and whose size covers only the rows that exist, so
// rows past the segment end read as zeros (no clamping or masking in the
// loop) and each thread's byte offsets are the same for every tile.
// Keys past the end thus dequantize to centroid 0 of their table (finite);
// their logits are masked before the softmax.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_CFG = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ rsrc_t buf(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, RSRC_CFG);
}
// off: per-thread byte offset; so: wave-uniform byte offset.  The range check
// covers off + so, so a descriptor can span a whole segment-head while the
// tile's offset travels in so.
__device__ __forceinline__ uint32_t ld8(rsrc_t r, int off, int so = 0) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, so, 0);
}
__device__ __forceinline__ uint8_t ld8b(rsrc_t r, int off, int so = 0) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, so, 0);
}
__device__ __forceinline__ uint32_t ld16(rsrc_t r, int off, int so = 0) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, so, 0);
}
__device__ __forceinline__ uint32_t ld32(rsrc_t r, int off, int so = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, so, 0);
}
__device__ __forceinline__ u32x4 ld128(rsrc_t r, int off, int so = 0) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, so, 0));
}

// Per-thread share of one tile (fixed for the whole kernel):
//  K:    key tid / 8, channels 16 (tid % 8) .. +16 (one code word)
//  PSAC: key tid / 8, coefficients 2 (tid % 8), +1 for tid % 8 < 4
//  V:    keys 2 (tid / 16), +1, channels 8 (tid % 16) .. +8 (a wave: 8 keys, all channels,
//        so its centroid-row loads touch 8 table rows, not 64)
struct Lane {
  int key, blk, p, oct;
  uint32_t zsh_k, zsh_v;   // bit offset of this thread's zero-point in its byte
  int c_off;               // byte offset of this thread's PSAC coefficients in a tile buffer
};
template <int NPK>
__device__ __forceinline__ Lane lane_share(int tid) {
  Lane L;
  L.key = tid >> 3;
  L.blk = tid & 7;
  // key pair p (keys 2p, 2p + 1) of the V_hat tile: a wave's four pairs fill
  // all four 32-bit words of their 16-byte chunks of a V_hat^T row, so that
  // the wave's 64 stores per channel hit 64 different banks
  const int w = tid >> 6, j = (tid >> 4) & 3;
  L.p = 8 * (w >> 1) + 2 * (w & 1) + (j & 1) + 4 * (j >> 1);
  L.oct = tid & 15;
  L.zsh_k = 4u * (uint32_t)(L.key & 1) + 2u * (uint32_t)(L.blk >> 2);
  L.zsh_v = 2u * (uint32_t)(L.oct >> 3);
  // thread blk owns coefficients 2 NPK blk .. +2 NPK of its key
  const int c0 = 2 * NPK * L.blk;
  L.c_off = (int)offsetof(AttnBuf<NPK>, chat) + (c0 >> 3) * CPL + L.key * 16 + 2 * (c0 & 7);
  return L;
}

// Three load stages, so that no load waits for another inside the loop:
//   idx (issued three tiles ahead): the centroid index bytes;
//   raw (two tiles ahead): codes, scales, zero-point bytes, PSAC bytes, and
//        the fp16 centroid rows (their idx arrived one iteration earlier);
//   all arithmetic on these bytes happens in dequant_tile.
// Kept as bytes: the zero-extension then happens where the table offsets are
// formed, not on the loop-carried value (which would make the top of every
// iteration wait for these loads).
struct TileIdx {
  uint8_t k, v0, v1;
};
struct TileRegs {
  uint32_t kcode, kscale, kzb, c2, cs;
  uint32_t bmhi;   // sparse coefficients: the tile's bitmap word is (bmhi, c2), its prefix count cs
  uint32_t vcode0, vcode1, vscale0, vscale1, vzb;
  u32x4 kmu[2];   // 16 permuted fp16 centroid channels
  u32x4 vmu[2];   // 8 fp16 centroid channels of each of the two keys
};

// One segment-head's packed arrays as seen by the bytes/index stage: the
// head's base addresses, carried in scalar registers from the moment the
// stage enters the segment.  Each load builds a buffer descriptor spanning
// the head's rows (num_records = their bytes), so rows past the segment end
// read as zeros, and reaches the tile's rows through the scalar offset
// (the range check covers it).  Offsets are 32-bit: a segment holds fewer
// than 2^26 keys.
struct SegDesc {
  const uint8_t *kc, *ks, *kz, *c, *cs, *vc, *vs, *vz, *ki, *vi;
  int T;
  int cT;     // rows of PSAC coefficients: T (dense), the kept count (sparse), or 0 without PSAC
  int r;      // PSAC rank (bytes per coefficient row)
  // compacted coefficients in the sparse layout: bitmap words and prefix counts
  const uint8_t *cbm, *cpre;
  int csparse, nw;
  // two-level group scales: INT8 step codes under fp16 second-level scales
  // (group 0 in the low half, group 1 in the high half)
  int ktwo, vtwo;
  uint32_t ks2, vs2;
};
__device__ __forceinline__ int64_t al16(int64_t n) { return (n + 15) & ~(int64_t)15; }

template <bool EXT>
__device__ __forceinline__ SegDesc seg_desc(const AttnArgs& a, int s, int h) {
  cseg& g = seg_at(a, s);
  const int64_t T = g.T;
  const int64_t hb = (int64_t)h * T;
  const int64_t zb = (int64_t)h * zeros_stride(T);
  SegDesc d;
  const bool psac = g.U != nullptr;
  d.kc = g.k_codes + hb * 32;
  d.ks = reinterpret_cast<const uint8_t*>(g.k_scale + hb * 2);
  d.kz = g.k_zeros + zb;
  // without PSAC the descriptors are empty: the loads return zeros and touch no memory
  d.r = __builtin_amdgcn_readfirstlane(g.r);
  d.c = psac ? reinterpret_cast<const uint8_t*>(g.k_c + hb * d.r) : g.k_codes;
  d.cs = psac ? reinterpret_cast<const uint8_t*>(g.k_c_scale + hb) : g.k_codes;
  d.vc = g.v_codes + hb * 32;
  d.vs = reinterpret_cast<const uint8_t*>(g.v_scale + hb * 2);
  d.vz = g.v_zeros + zb;
  d.ki = g.k_idx + hb;
  d.vi = g.v_idx + hb;
  d.T = (int)T;
  // wave-uniform by construction; saying so keeps the descriptors scalar
  d.cT = __builtin_amdgcn_readfirstlane(psac ? (int)T : 0);
  d.cbm = d.cpre = nullptr;
  d.csparse = 0; d.nw = 0; d.ktwo = 0; d.vtwo = 0; d.ks2 = 0u; d.vs2 = 0u;
  if constexpr (EXT) {
    if (psac && g.k_cdir != nullptr) {
      const __attribute__((address_space(4))) qwm_cdir* dir = (const __attribute__((address_space(4))) qwm_cdir*)g.k_cdir;
      const int layout = dir[h].layout, count = dir[h].count;
      const uint8_t* base = g.k_carena + dir[h].offset;
      if (layout == QWM_LAYOUT_DENSE) {
        d.c = base;
        d.cs = base + al16(T * d.r);
      } else if (layout == QWM_LAYOUT_SPARSE) {
        const int64_t nw = (T + 63) / 64;
        d.cbm = base;
        d.cpre = base + al16(nw * 8);
        d.c = d.cpre + al16(nw * 4);
        d.cs = d.c + al16((int64_t)count * d.r);
        d.csparse = 1;
        d.nw = (int)nw;
        d.cT = __builtin_amdgcn_readfirstlane(count);
      } else {
        d.cT = 0;   // the arena could not hold this head: no compensation
      }
    }
    if (g.k_scale2 != nullptr) {
      d.ktwo = 1;
      d.ks = reinterpret_cast<const uint8_t*>(g.k_scale) + hb * 2;   // INT8 step codes: [H][T][G] bytes
      d.ks2 = __builtin_amdgcn_readfirstlane(*(const __attribute__((address_space(4))) uint32_t*)(g.k_scale2 + 2 * h));
    }
    if (g.v_scale2 != nullptr) {
      d.vtwo = 1;
      d.vs = reinterpret_cast<const uint8_t*>(g.v_scale) + hb * 2;
      d.vs2 = __builtin_amdgcn_readfirstlane(*(const __attribute__((address_space(4))) uint32_t*)(g.v_scale2 + 2 * h));
    }
  }
  return d;
}

// A dense unit's descriptor: no packed arrays (every load of them reads 0).
__device__ __forceinline__ SegDesc dense_desc(const AttnArgs& a) {
  SegDesc d{};
  d.T = (int)a.Ta;
  d.cT = 0;
  d.r = 8;
  return d;
}
template <bool DENSE, bool EXT>
__device__ __forceinline__ SegDesc desc_for(const AttnArgs& a, int s, int h) {
  if constexpr (DENSE) return dense_desc(a);
  else return seg_desc<EXT>(a, s, h);
}

template <bool DENSE>
__device__ __forceinline__ void load_idx(const SegDesc& d, const Pos& P, const Lane& L, TileIdx& x) {
  const int k0 = P.tile * AT_K;
  const int pT = DENSE ? 0 : d.T;
  const rsrc_t ki = buf(d.ki, pT), vi = buf(d.vi, pT);
  x.k = ld8b(ki, L.key, k0);
  x.v0 = ld8b(vi, 2 * L.p, k0);
  x.v1 = ld8b(vi, 2 * L.p + 1, k0);
}

// The packed bytes of a tile (codes, scales, zero-points, PSAC bytes); for
// a dense unit all zeros, so its tiles dequantize to the rows themselves.
template <bool DENSE, int NPK, bool EXT>
__device__ __forceinline__ void load_bytes(const SegDesc& d, const Pos& P, const Lane& L, TileRegs& r) {
  const int k0 = P.tile * AT_K, T = DENSE ? 0 : d.T;
  {
    const int g = L.blk >> 2;
    r.kcode = ld32(buf(d.kc, T * 32), L.key * 32 + 4 * L.blk, k0 * 32);
    if (EXT && d.ktwo) r.kscale = ld8(buf(d.ks, T * 2), L.key * 2 + g, k0 * 2);   // step code, scaled in load_mu
    else r.kscale = ld16(buf(d.ks, T * 4), L.key * 4 + 2 * g, k0 * 4);
    r.kzb = ld8(buf(d.kz, (T + 1) >> 1), L.key >> 1, k0 >> 1);
    if (EXT && d.csparse) {
      // the tile's bitmap word and prefix count; load_mu gathers the kept rows
      const rsrc_t bm = buf(d.cbm, d.nw * 8);
      r.c2 = ld32(bm, 0, P.tile * 8);
      r.bmhi = ld32(bm, 4, P.tile * 8);
      r.cs = ld32(buf(d.cpre, d.nw * 4), 0, P.tile * 4);
    } else {
      const rsrc_t cr = buf(d.c, d.cT * d.r);
      const uint32_t cv = NPK == 1 ? ld16(cr, L.key * d.r + 2 * L.blk, k0 * d.r)
                                   : ld32(cr, L.key * d.r + 4 * L.blk, k0 * d.r);
      r.c2 = (2 * NPK * L.blk < d.r) ? cv : 0u;
      r.cs = ld16(buf(d.cs, d.cT * 2), L.key * 2, k0 * 2);
    }
  }
  {
    const int g = L.oct >> 3;
    const rsrc_t vc = buf(d.vc, T * 32);
    r.vcode0 = ld16(vc, (2 * L.p) * 32 + 2 * L.oct, k0 * 32);
    r.vcode1 = ld16(vc, (2 * L.p + 1) * 32 + 2 * L.oct, k0 * 32);
    if (EXT && d.vtwo) {
      const rsrc_t vs = buf(d.vs, T * 2);
      r.vscale0 = ld8(vs, (2 * L.p) * 2 + g, k0 * 2);
      r.vscale1 = ld8(vs, (2 * L.p + 1) * 2 + g, k0 * 2);
    } else {
      const rsrc_t vs = buf(d.vs, T * 4);
      r.vscale0 = ld16(vs, (2 * L.p) * 4 + 2 * g, k0 * 4);
      r.vscale1 = ld16(vs, (2 * L.p + 1) * 4 + 2 * g, k0 * 4);
    }
    r.vzb = ld8(buf(d.vz, (T + 1) >> 1), L.p, k0 >> 1);
  }
}

// The stored-format conversions of a tile whose bytes have arrived (segment
// descriptor d): a sparse head's kept rows are gathered by the tile's bitmap
// word and prefix count; two-level step codes become fp16 steps (code times
// the power-of-two second-level scale: exact).
template <int NPK>
__device__ __forceinline__ void ext_convert(const SegDesc& d, const Lane& L, TileRegs& r) {
  if (d.csparse) {
    const uint32_t lo = r.c2, hi = r.bmhi, pre = r.cs;
    const int key = L.key;
    const uint32_t word = key < 32 ? lo : hi;
    const bool kept = (word >> (key & 31)) & 1u;
    const uint32_t below = key < 32 ? __popc(lo & ((1u << key) - 1u))
                                    : __popc(lo) + __popc(hi & ((1u << (key - 32)) - 1u));
    const int e = (int)(pre + below);
    const rsrc_t cr = buf(d.c, d.cT * d.r);
    const uint32_t cv = NPK == 1 ? ld16(cr, e * d.r + 2 * L.blk) : ld32(cr, e * d.r + 4 * L.blk);
    const uint32_t sv = ld16(buf(d.cs, d.cT * 2), e * 2);
    r.c2 = (kept && 2 * NPK * L.blk < d.r) ? cv : 0u;
    r.cs = kept ? sv : 0u;
  }
  if (d.ktwo) {
    const uint32_t s2 = (L.blk >> 2) ? (d.ks2 >> 16) : (d.ks2 & 0xFFFFu);
    const _Float16 st = (_Float16)(float)r.kscale * __builtin_bit_cast(_Float16, (uint16_t)s2);
    r.kscale = (uint32_t)__builtin_bit_cast(uint16_t, st);
  }
  if (d.vtwo) {
    const _Float16 s2 = __builtin_bit_cast(_Float16, (uint16_t)((L.oct >> 3) ? (d.vs2 >> 16) : (d.vs2 & 0xFFFFu)));
    r.vscale0 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)((_Float16)(float)r.vscale0 * s2));
    r.vscale1 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)((_Float16)(float)r.vscale1 * s2));
  }
}

// The fp16 centroid rows of a tile's keys (segment seg), from its indices;
// for a dense unit the keys' own bf16 rows (rows_to_f16 converts them once
// they have arrived).  Rows past the end read as zeros.
template <bool DENSE>
__device__ __forceinline__ void load_mu(const AttnArgs& a, int seg, int tile, int h, const Lane& L,
                                        const TileIdx& x, TileRegs& r) {
  if constexpr (DENSE) {
    const int k0 = tile * AT_K, T = (int)a.Ta;
    const int kst = (int)a.kast * 2, vst = (int)a.vast * 2;   // bytes
    const rsrc_t kb = buf(a.ka + h * a.kash, T * kst);
    const rsrc_t vb = buf(a.va + h * a.vash, T * vst);
    r.kmu[0] = ld128(kb, L.key * kst + 32 * L.blk, k0 * kst);
    r.kmu[1] = ld128(kb, L.key * kst + 32 * L.blk + 16, k0 * kst);
    r.vmu[0] = ld128(vb, (2 * L.p) * vst + 16 * L.oct, k0 * vst);
    r.vmu[1] = ld128(vb, (2 * L.p + 1) * vst + 16 * L.oct, k0 * vst);
    return;
  }
  const uint16_t* ktab = a.tabs + ((int64_t)(seg * a.H + h) * 2) * TAB_ELEMS;
  const rsrc_t kt = buf(ktab, TAB_ELEMS * 2);
  const int mo = (int)(x.k * (D * 2)) + 32 * L.blk;
  r.kmu[0] = ld128(kt, mo);
  r.kmu[1] = ld128(kt, mo + 16);
  const rsrc_t vt = buf(ktab + TAB_ELEMS, TAB_ELEMS * 2);
  r.vmu[0] = ld128(vt, (int)(x.v0 * (D * 2)) + 16 * L.oct);
  r.vmu[1] = ld128(vt, (int)(x.v1 * (D * 2)) + 16 * L.oct);
}

// Dense rows, as load_mu leaves them, into the fp16 layout of the centroid
// rows: K channels 16 blk + m and 16 blk + m + 8 in word m (the K tables'
// permuted order), V channels in order.  bf16 -> fp16 is exact within fp16's
// range.
__device__ __forceinline__ void rows_to_f16(TileRegs& r) {
  const u32x4 a = r.kmu[0], b = r.kmu[1];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const uint32_t lo = (m & 1) ? (a[m >> 1] & 0xFFFF0000u) : (a[m >> 1] << 16);
    const uint32_t hi = (m & 1) ? (b[m >> 1] & 0xFFFF0000u) : (b[m >> 1] << 16);
    r.kmu[m >> 2][m & 3] = pack_f16x2(__uint_as_float(lo), __uint_as_float(hi));
  }
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r.vmu[k][e] = pack_f16x2(__uint_as_float(r.vmu[k][e] << 16), __uint_as_float(r.vmu[k][e] & 0xFFFF0000u));
}

// Copy the packed-byte fields (the centroid rows are loaded separately).
__device__ __forceinline__ void take_bytes(TileRegs& d, const TileRegs& s) {
  d.kcode = s.kcode; d.kscale = s.kscale; d.kzb = s.kzb; d.c2 = s.c2; d.cs = s.cs; d.bmhi = s.bmhi;
  d.vcode0 = s.vcode0; d.vcode1 = s.vcode1; d.vscale0 = s.vscale0; d.vscale1 = s.vscale1; d.vzb = s.vzb;
}

// PSAC coefficients c_scale * c of the thread's share of its key: each int8
// pair becomes the exact fp16 pair (1024 + c + 128) - 1152, then one rounded
// fp16 product.
template <int NPK>
__device__ __forceinline__ void store_coeffs(const TileRegs& r, const Lane& L, uint8_t* buf_base) {
  const _Float16 cs = __builtin_bit_cast(_Float16, (uint16_t)r.cs);
  const h2 bias = h2{(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t sp0 = __builtin_amdgcn_perm(0u, r.c2, 0x0C010C00u) ^ 0x64806480u;
  const uint32_t v0 = as_u32((as_h2(sp0) - bias) * h2{cs, cs});
  if constexpr (NPK == 1) {
    *reinterpret_cast<uint32_t*>(buf_base + L.c_off) = v0;
  } else {
    const uint32_t sp1 = __builtin_amdgcn_perm(0u, r.c2, 0x0C030C02u) ^ 0x64806480u;
    const uint32_t v1 = as_u32((as_h2(sp1) - bias) * h2{cs, cs});
    *reinterpret_cast<uint2*>(buf_base + L.c_off) = make_uint2(v0, v1);
  }
}

// fp16 pair (-1024 - z0, -1024 - z1) from two 2-bit zero-points: 0xE400 + z
__device__ __forceinline__ h2 neg_zero_pair(uint32_t z01) { return as_h2(z01 | 0xE400E400u); }

template <int NPK>
__device__ __forceinline__ void dequant_tile(const TileRegs& r, const Lane& L, const CodeMasks& cm, AttnBuf<NPK>& b) {
  {
    // K0_hat: s (c - z) + mu in packed fp16 (c - z is exact; one rounding in the fma)
    const uint32_t z = __builtin_amdgcn_ubfe(r.kzb, L.zsh_k, 2);
    const h2 nz2 = neg_zero_pair(z * 0x10001u);
    const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)r.kscale);
    const h2 s2 = {s, s};
    u32x4 o[2];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const h2 d = code_pair(r.kcode, 2 * m, cm) + nz2;
      o[m >> 2][m & 3] = as_u32(__builtin_elementwise_fma(s2, d, as_h2(r.kmu[m >> 2][m & 3])));
    }
    u32x4* kr = reinterpret_cast<u32x4*>(b.khat + L.key * KSTR + 32 * L.blk);
    kr[0] = o[0];
    kr[1] = o[1];
    store_coeffs<NPK>(r, L, reinterpret_cast<uint8_t*>(&b));
  }
  {
    // V_hat, keys 2p (low half) and 2p + 1 (high half) of channel 8 oct + c
    const uint32_t cw = r.vcode0 | (r.vcode1 << 16);
    const h2 s2 = as_h2(r.vscale0 | (r.vscale1 << 16));
    const uint32_t t = r.vzb >> L.zsh_v;    // bits 0-1: key 2p, bits 4-5: key 2p + 1
    const h2 nz2 = neg_zero_pair((t | (t << 12)) & 0x00030003u);
    uint8_t* vrow = b.vt + vt_offset(8 * L.oct, vslot(2 * L.p));
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t mu2 = __builtin_amdgcn_perm(r.vmu[1][c >> 1], r.vmu[0][c >> 1], (c & 1) ? 0x07060302u : 0x05040100u);
      const h2 d = code_pair(cw, 2 * c, cm) + nz2;
      *reinterpret_cast<uint32_t*>(vrow + c * VSTR) = as_u32(__builtin_elementwise_fma(s2, d, as_h2(mu2)));
    }
  }
}

// Phase 1 of a tile: S^T for its 64 keys as two 32-key MFMA tiles (A: keys
// 0..31, B: 32..63), their steps alternating so that consecutive MFMAs are
// independent, with the dequantization of the next tile into the other buffer
// woven between them one code word at a time: a wave's VALU work issued
// between its own MFMAs runs while they execute.  The order is fixed by
// scheduling barriers; operand reads run two steps ahead.
template <int NPK>
__device__ __forceinline__ void tile_phase1(const AttnBuf<NPK>* __restrict__ B, AttnBuf<NPK>* __restrict__ W,
                                            const f16x8 (&qf)[8], const f16x8 (&qpf)[NPK], int ln, int hh,
                                            const TileRegs& r, const Lane& L, const CodeMasks& cm,
                                            f32x16& sa, f32x16& sb2) {
  const uint8_t* krow = B->khat + ln * KSTR + 16 * hh;
  // K0_hat: s (c - z) + mu in packed fp16 (c - z is exact; one rounding in the fma)
  const uint32_t kz = __builtin_amdgcn_ubfe(r.kzb, L.zsh_k, 2);
  const h2 knz = neg_zero_pair(kz * 0x10001u);
  const _Float16 ksc = __builtin_bit_cast(_Float16, (uint16_t)r.kscale);
  const h2 ks2 = {ksc, ksc};
  // V_hat, keys 2p (low half) and 2p + 1 (high half) of channel 8 oct + c
  const uint32_t cw = r.vcode0 | (r.vcode1 << 16);
  const h2 vs2 = as_h2(r.vscale0 | (r.vscale1 << 16));
  const uint32_t vzt = r.vzb >> L.zsh_v;    // bits 0-1: key 2p, bits 4-5: key 2p + 1
  const h2 vnz = neg_zero_pair((vzt | (vzt << 12)) & 0x00030003u);
  uint8_t* vw = W->vt + vt_offset(8 * L.oct, vslot(2 * L.p));
  u32x4* kw = reinterpret_cast<u32x4*>(W->khat + L.key * KSTR + 32 * L.blk);

  f16x8 fa[8], fb[8];
  fa[0] = *reinterpret_cast<const f16x8*>(krow);
  fb[0] = *reinterpret_cast<const f16x8*>(krow + 32 * KSTR);
  fa[1] = *reinterpret_cast<const f16x8*>(krow + 32);
  fb[1] = *reinterpret_cast<const f16x8*>(krow + 32 * KSTR + 32);
  f16x8 ca[NPK], cb[NPK];
  u32x4 ko[2];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s + 2 < 8) {
      fa[s + 2] = *reinterpret_cast<const f16x8*>(krow + 32 * (s + 2));
      fb[s + 2] = *reinterpret_cast<const f16x8*>(krow + 32 * KSTR + 32 * (s + 2));
    } else if (s == 6) {
      // PSAC step operands: coefficients 16 k + 8 hh .. +8 of key ln (and
      // 32 + ln); zeros past the segment's rank, and in qpf for a segment
      // without PSAC
#pragma unroll
      for (int k = 0; k < NPK; ++k) {
        ca[k] = *reinterpret_cast<const f16x8*>(B->chat + (2 * k + hh) * CPL + ln * 16);
        cb[k] = *reinterpret_cast<const f16x8*>(B->chat + (2 * k + hh) * CPL + (32 + ln) * 16);
      }
    }
    sa = mfma_f16(fa[s], qf[s], sa);
    {
      const h2 d = code_pair(r.kcode, 2 * s, cm) + knz;
      ko[s >> 2][s & 3] = as_u32(__builtin_elementwise_fma(ks2, d, as_h2(r.kmu[s >> 2][s & 3])));
      if ((s & 3) == 3) kw[s >> 2] = ko[s >> 2];
    }
    __builtin_amdgcn_sched_barrier(0);
    sb2 = mfma_f16(fb[s], qf[s], sb2);
    {
      const uint32_t mu2 = __builtin_amdgcn_perm(r.vmu[1][s >> 1], r.vmu[0][s >> 1], (s & 1) ? 0x07060302u : 0x05040100u);
      const h2 d = code_pair(cw, 2 * s, cm) + vnz;
      *reinterpret_cast<uint32_t*>(vw + s * VSTR) = as_u32(__builtin_elementwise_fma(vs2, d, as_h2(mu2)));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  sa = mfma_f16(ca[0], qpf[0], sa);
  store_coeffs<NPK>(r, L, reinterpret_cast<uint8_t*>(W));
  __builtin_amdgcn_sched_barrier(0);
  sb2 = mfma_f16(cb[0], qpf[0], sb2);
  if constexpr (NPK == 2) {
    sa = mfma_f16(ca[1], qpf[1], sa);
    sb2 = mfma_f16(cb[1], qpf[1], sb2);
  }
}

// Lanes l and l ^ 32 hold the two halves of one query column.
__device__ __forceinline__ float pair_max(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// the value held by lane l ^ 32
__device__ __forceinline__ uint32_t pair_other(uint32_t v, int hh) {
  const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return hh ? s[0] : s[1];
}

// One unit: 256 Queries (query block qb) x head h x split `split` of nsplit
// of a key sequence, written to partial set `part`.  DENSE: the key sequence
// is the active BF16 chunk; otherwise the packed segments.
template <bool TOP1, bool DENSE, int NPK, bool EXT>
__device__ __forceinline__ void attention_body(const AttnArgs& a, AttnBuf<NPK>* sb, int qb, int split, int nsplit,
                                               int part, int h) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hh = lane >> 5, ln = lane & 31;
  const int64_t qw0 = (int64_t)qb * AT_Q + wv * AT_QW;
  const bool wave_active = qw0 < a.Tq;
  const int64_t qi = qw0 + ln;
  const bool qvalid = qi < a.Tq;
  const int64_t qoff = (int64_t)h * a.qsh + (qvalid ? qi : 0) * a.qst;
  const Lane L = lane_share<NPK>(tid);

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

  // this split's share of the tile sequence
  const int total = DENSE ? ntiles(a.Ta) : count_tiles(a, lane);
  const int g0 = (int)((int64_t)total * split / nsplit);
  const int count = (int)((int64_t)total * (split + 1) / nsplit) - g0;
  if (count <= 0) {
    if (qvalid && a.nparts > 1 && hh == 0) {
      const int64_t pidx = ((int64_t)part * a.H + h) * a.Tq + qi;
      a.pm[pidx] = -__builtin_inff(); a.pl[pidx] = 0.f;
      if (TOP1) { a.ptv[pidx] = best_v; a.pti[pidx] = best_i; }
    }
    return;
  }
  // positions of tiles n, n + 1, n + 2, n + 3 of the split (past the end a
  // position repeats the last tile, so every stage loads memory that exists)
  Pos P0;
  if constexpr (DENSE) { P0.seg = 0; P0.tile = g0; P0.kbase = a.kbase_a; }
  else P0 = locate(a, g0, lane);
  Pos P1 = count > 1 ? advance<DENSE>(a, P0, seg_T<DENSE>(a, P0.seg)) : P0;
  Pos P2 = count > 2 ? advance<DENSE>(a, P1, seg_T<DENSE>(a, P1.seg)) : P1;
  Pos P3 = count > 3 ? advance<DENSE>(a, P2, seg_T<DENSE>(a, P2.seg)) : P2;
  // Load stages of tile t: packed bytes and indices three tiles ahead (HBM
  // latency), centroid rows two tiles ahead (from the indices), dequantization
  // one tile ahead.  Segment fields: T of tiles n .. n + 2, the arrays of
  // tile n + 3's segment.
  int64_t T0 = seg_T<DENSE>(a, P0.seg), T1 = seg_T<DENSE>(a, P1.seg), T2 = seg_T<DENSE>(a, P2.seg);
  SegDesc sd = desc_for<DENSE, EXT>(a, P3.seg, h);
  // the descriptor of tile n + 2's segment, whose bytes get their stored-format
  // conversions once they have arrived
  SegDesc sdm = desc_for<DENSE, EXT>(a, P2.seg, h);

  // pipeline fill: tile 0 dequantized, tile 1 complete in registers, tile 2's
  // bytes and indices in flight
  const CodeMasks cm = code_masks();
  TileRegs regs, nbytes;
  TileIdx tix;
  {
    const SegDesc d0 = desc_for<DENSE, EXT>(a, P0.seg, h);
    load_idx<DENSE>(d0, P0, L, tix);
    load_bytes<DENSE, NPK, EXT>(d0, P0, L, regs);
    if constexpr (EXT) ext_convert<NPK>(d0, L, regs);
    load_mu<DENSE>(a, P0.seg, P0.tile, h, L, tix, regs);
    if constexpr (DENSE) rows_to_f16(regs);
    dequant_tile<NPK>(regs, L, cm, sb[0]);
    const SegDesc d1 = desc_for<DENSE, EXT>(a, P1.seg, h);
    load_idx<DENSE>(d1, P1, L, tix);
    load_bytes<DENSE, NPK, EXT>(d1, P1, L, regs);
    if constexpr (EXT) ext_convert<NPK>(d1, L, regs);
    load_mu<DENSE>(a, P1.seg, P1.tile, h, L, tix, regs);
    const SegDesc d2 = desc_for<DENSE, EXT>(a, P2.seg, h);
    load_idx<DENSE>(d2, P2, L, tix);
    load_bytes<DENSE, NPK, EXT>(d2, P2, L, nbytes);
  }
  __syncthreads();

  int cur = 0;
  int qp_seg = -1;
  f16x8 qpf[NPK];
#pragma unroll
  for (int k = 0; k < NPK; ++k) qpf[k] = __builtin_bit_cast(f16x8, u32x4{0, 0, 0, 0});
  const h2 ones = as_h2(0x3C003C00u);
  for (int n = 0; n < count; ++n) {
    if (!DENSE && P0.seg != qp_seg) {
      // Q U for this segment: (U^T) (Q^T) on MFMA with the Query fragments as
      // B; the basis fragments come from the workspace (zeros without PSAC;
      // rows n >= the rank read as zeros, past the end of their buffer)
      qp_seg = P0.seg;
      const int rk = __builtin_amdgcn_readfirstlane(seg_at(a, P0.seg).r);
      const rsrc_t ur = buf(a.ut + (int64_t)(P0.seg * a.H + h) * (UT_ROWS * D), rk * D * 2);
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x4 v = ld128(ur, ((ln * 8 + s) * 2 + hh) * 16);
        acc = mfma_f16(__builtin_bit_cast(f16x8, v), qf[s], acc);
      }
      // lane (query, hh) holds (QU)[n] for n = 8 (i / 4) + 4 hh + i % 4 in acc[i];
      // the PSAC k-step k needs n = 16 k + 8 hh .. +8 of its query: four of its
      // own values and four of the partner lane's
#pragma unroll
      for (int k = 0; k < NPK; ++k) {
        float recv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) recv[e] = swap32_f(hh ? acc[8 * k + e] : acc[8 * k + 4 + e]);
        u32x4 pv;
        if (hh == 0) {
          pv[0] = pack_f16x2(acc[8 * k], acc[8 * k + 1]);
          pv[1] = pack_f16x2(acc[8 * k + 2], acc[8 * k + 3]);
          pv[2] = pack_f16x2(recv[0], recv[1]);
          pv[3] = pack_f16x2(recv[2], recv[3]);
        } else {
          pv[0] = pack_f16x2(recv[0], recv[1]);
          pv[1] = pack_f16x2(recv[2], recv[3]);
          pv[2] = pack_f16x2(acc[8 * k + 4], acc[8 * k + 5]);
          pv[3] = pack_f16x2(acc[8 * k + 6], acc[8 * k + 7]);
        }
        qpf[k] = __builtin_bit_cast(f16x8, pv);
      }
    }
    const AttnBuf<NPK>& B = sb[cur];
    const int64_t k0 = (int64_t)P0.tile * AT_K;
    const int nvalid = (int)((T0 - k0) < AT_K ? (T0 - k0) : AT_K);

    // ---- phase 1: S^T for the tile's 64 keys as two 32-key MFMA tiles (A: keys
    //      0..31, B: 32..63), their steps alternating so that consecutive MFMAs
    //      are independent, and in the same instruction stream the dequantization
    //      of the next tile into the other buffer and the loads of the two tiles
    //      after it.  Nothing here branches, so MFMAs and VALU work interleave.
    //      Past the end of the split the stages repeat the last tile (into a
    //      buffer nobody reads), so that no load is conditional.
    f32x16 sa = {}, sb2 = {};
    if constexpr (DENSE) rows_to_f16(regs);
    tile_phase1<NPK>(&sb[cur], &sb[cur ^ 1], qf, qpf, ln, hh, regs, L, cm, sa, sb2);
    // tile n + 2: its bytes arrived during the previous iteration; fetch its
    // centroid rows.  Tile n + 3: bytes and indices.
    take_bytes(regs, nbytes);
    if constexpr (EXT) ext_convert<NPK>(sdm, L, regs);
    load_mu<DENSE>(a, P2.seg, P2.tile, h, L, tix, regs);
    load_bytes<DENSE, NPK, EXT>(sd, P3, L, nbytes);
    load_idx<DENSE>(sd, P3, L, tix);

    if (wave_active) {
      // ---- keys past the segment end (their rows hold centroid 0) ----
      if (nvalid < AT_K) {
        // row c_row(i, hh) = 4 hh + (8 (i / 4) + i % 4) of each 32-key tile
        // against the limit, taken opaquely so the compares use inline constants
        int t;
        asm volatile("v_sub_u32 %0, %1, %2" : "=v"(t) : "s"(nvalid), "v"(4 * hh));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (t <= 8 * (i >> 2) + (i & 3)) sa[i] = -__builtin_inff();
          if (t <= 32 + 8 * (i >> 2) + (i & 3)) sb2[i] = -__builtin_inff();
        }
      }
      // ---- phase 2: the tile's row max; lazy rescale of what was accumulated ----
      float mt = fmaxf(fmaxf(sa[0], sa[1]), sa[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mt = fmaxf(fmaxf(mt, sa[i]), sa[i + 1]);
      mt = fmaxf(fmaxf(mt, sa[15]), sb2[0]);
#pragma unroll
      for (int i = 1; i < 15; i += 2) mt = fmaxf(fmaxf(mt, sb2[i]), sb2[i + 1]);
      mt = fmaxf(mt, sb2[15]);
      if (TOP1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (sa[i] > best_v) { best_v = sa[i]; best_i = (int32_t)(P0.kbase + k0 + c_row(i, hh)); }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (sb2[i] > best_v) { best_v = sb2[i]; best_i = (int32_t)(P0.kbase + k0 + 32 + c_row(i, hh)); }
        }
      }
      mt = pair_max(mt) * sc2;
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
      // ---- phase 3: P = exp2(S sc2 - m) in fp16 and O^T += V^T P; the second
      //      half's exponentials overlap the first half's MFMAs ----
      // physical chunk of logical chunk 2 (2 kt + s2) + hh in row 32 c + ln:
      // 2 ((2 kt + s2) ^ c) + (hh ^ (ln / 16)), see vt_offset
      const uint8_t* vrow = B.vt + ln * VSTR + 16 * (hh ^ (ln >> 4));
      float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const f32x16& sc = kt ? sb2 : sa;
        // V_hat operands: keys (slots) 8 (2 (2 kt + s2) + hh) .. +8 of channel 32 c + ln
        f16x8 vf[4][2];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
            vf[c][s2] = *reinterpret_cast<const f16x8*>(vrow + 32 * c * VSTR + 32 * ((2 * kt + s2) ^ c));
        u32x4 pw[2];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[i], sc2, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[i + 1], sc2, -m_run));
          const h2 pk = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(p0, p1));
          // the denominator sums exactly the fp16 probabilities the P V product uses
          if (i & 2) lsum1 = __builtin_amdgcn_fdot2(pk, ones, lsum1, false);
          else lsum0 = __builtin_amdgcn_fdot2(pk, ones, lsum0, false);
          // PV k-step 2 kt + i / 8, element (i % 8)
          pw[i >> 3][(i & 7) >> 1] = as_u32(pk);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) o_acc[c] = mfma_f16(vf[c][s2], __builtin_bit_cast(f16x8, pw[s2]), o_acc[c]);
      }
      l_run += lsum0 + lsum1;
    }
    __syncthreads();
    P0 = P1; T0 = T1;
    P1 = P2; T1 = T2;
    P2 = P3; T2 = sd.T;
    if constexpr (EXT) sdm = sd;
    if (n + 4 < count) {
      P3 = advance<DENSE>(a, P3, sd.T);
      if (!DENSE && P3.seg != P2.seg) sd = desc_for<DENSE, EXT>(a, P3.seg, h);
    }
    cur ^= 1;
  }

  // ---- epilogue ----
  const float l_tot = pair_sum(l_run);
  if (TOP1) {
    const float ov = __uint_as_float(pair_other(__float_as_uint(best_v), hh));
    const int32_t oi = (int32_t)pair_other((uint32_t)best_i, hh);
    if (ov > best_v || (ov == best_v && oi < best_i)) { best_v = ov; best_i = oi; }
  }
  if (!qvalid) return;
  if (a.nparts == 1) {
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
    const int64_t pidx = ((int64_t)part * a.H + h) * a.Tq + qi;
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

template <bool TOP1, int NPK, bool EXT>
__global__ __launch_bounds__(AT_T, 1) void attention_kernel(AttnArgs a) {
  __shared__ AttnBuf<NPK> sb[2];
  // XCD-aware unit mapping: consecutive units (same head) go to the same XCD
  const int nb = (int)gridDim.x;
  const int per = (nb + 7) / 8;
  const int unit = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (unit >= a.units) return;
  if (unit < a.units_p) {
    const int qb = unit % a.nqb, split = (unit / a.nqb) % a.nsplit, h = unit / (a.nqb * a.nsplit);
    attention_body<TOP1, false, NPK, EXT>(a, sb, qb, split, a.nsplit, split, h);
  } else {
    const int u = unit - a.units_p;
    const int qb = u % a.nqb, split = (u / a.nqb) % a.nsplit_a, h = u / (a.nqb * a.nsplit_a);
    attention_body<TOP1, true, NPK, false>(a, sb, qb, split, a.nsplit_a, a.nsplit + split, h);
  }
}

// Merge split partials.  Grid (ceil(Tq/8), H), 256 threads: eight queries per
// block, 32 threads per query, four channels per thread (16-byte accesses).
template <bool TOP1>
__global__ __launch_bounds__(256) void attention_combine_kernel(AttnArgs a) {
  const int h = blockIdx.y, c = 4 * (threadIdx.x & 31);
  const int64_t qi = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (qi >= a.Tq) return;
  float mx = -__builtin_inff();
  for (int p = 0; p < a.nparts; ++p) mx = fmaxf(mx, a.pm[((int64_t)p * a.H + h) * a.Tq + qi]);
  float l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float bv = -__builtin_inff();
  int32_t bi = 0x7FFFFFFF;
  for (int p = 0; p < a.nparts; ++p) {
    const int64_t pidx = ((int64_t)p * a.H + h) * a.Tq + qi;
    const float pm = a.pm[pidx];
    const float wgt = (pm == -__builtin_inff()) ? 0.f : exp2f(pm - mx);
    l += a.pl[pidx] * wgt;
    const f32x4 v = *reinterpret_cast<const f32x4*>(a.po + pidx * D + c);
    o += v * wgt;
    if (TOP1) {
      const float tv = a.ptv[pidx];
      const int32_t ti = a.pti[pidx];
      if (tv > bv || (tv == bv && ti < bi)) { bv = tv; bi = ti; }
    }
  }
  *reinterpret_cast<f32x4*>(a.out + (qi * a.H + h) * D + c) =
      l > 0.f ? f32x4{o[0] / l, o[1] / l, o[2] / l, o[3] / l} : f32x4{0.f, 0.f, 0.f, 0.f};
  if (c == 0) {
    if (a.lse) a.lse[(int64_t)h * a.Tq + qi] = (mx + log2f(l)) / LOG2E;
    if (TOP1 && a.top1) a.top1[(int64_t)h * a.Tq + qi] = bi;
  }
}

// Log-sum-exp merge of two attention results of the same Queries over disjoint
// key sets: with m = max(la, lb), O = (e^(la - m) Oa + e^(lb - m) Ob) / (e^(la - m) +
// e^(lb - m)) and lse = m + log of that denominator; a part with lse = -inf has
// no keys.  Grid ceil(Tq H / 2), 256 threads: 128 channels of two (query, head)
// rows per block.  out may be oa or ob (each thread reads its elements before
// writing them); lse must not alias la or lb.
__global__ __launch_bounds__(256) void attention_merge_kernel(const float* oa, const float* __restrict__ la,
                                                              const float* ob, const float* __restrict__ lb,
                                                              int64_t Tq, int32_t H, float* out, float* lse) {
  const int64_t r = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  if (r >= Tq * H) return;
  const int c = threadIdx.x & 127;
  const int64_t q = r / H;
  const int h = (int)(r % H);
  const float a = la[(int64_t)h * Tq + q], b = lb[(int64_t)h * Tq + q];
  const float m = fmaxf(a, b);
  const int64_t e = r * D + c;
  if (m == -__builtin_inff()) {
    out[e] = 0.f;
    if (lse && c == 0) lse[(int64_t)h * Tq + q] = -__builtin_inff();
    return;
  }
  const float wa = (a == -__builtin_inff()) ? 0.f : expf(a - m);
  const float wb = (b == -__builtin_inff()) ? 0.f : expf(b - m);
  const float den = wa + wb;
  out[e] = (wa * oa[e] + wb * ob[e]) / den;
  if (lse && c == 0) lse[(int64_t)h * Tq + q] = m + logf(den);
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
    // CU occupancy over whole rounds, minus a cost per split (partial outputs,
    // merge work, pipeline fill per unit); 0.04 measured best on the full-depth
    // layer (4 splits: 1.29-1.31 ms, against 1.31-1.35 ms with 6 at 0.02)
    const double score = (double)n / (double)(rounds * 256) - 0.04 * s;
    if (score > best_score + 1e-9) { best_score = score; best = s; }
  }
  return best;
}

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Split plan: the key sequence (packed keys, then the active chunk's) gets
// attention_splits() splits in all, shared between the two in proportion to
// their keys (each present part at least one); partial sets = splits.
struct AttnPlan { int nsplit, nsplit_a, nparts; };
static AttnPlan attention_plan(int64_t Tq, int32_t H, int64_t packed_keys, int64_t active_keys) {
  const int P = attention_splits(Tq, H, packed_keys + active_keys);
  AttnPlan p{P, 0, P};
  if (active_keys > 0) {
    if (packed_keys == 0) {
      p.nsplit = 0;
      p.nsplit_a = P;
    } else {
      p.nsplit_a = (int)((P * active_keys + (packed_keys + active_keys) / 2) / (packed_keys + active_keys));
      if (p.nsplit_a < 1) p.nsplit_a = 1;
      p.nsplit = P - p.nsplit_a;
      if (p.nsplit < 1) p.nsplit = 1;
    }
    p.nparts = p.nsplit + p.nsplit_a;
  }
  return p;
}

// Workspace for n_segs packed segments and up to (splits + 1) partial sets;
// total_keys counts every key (packed and active).
size_t attention_ws_bytes(int64_t total_keys, int32_t H, int64_t Tq, int32_t n_segs, bool active) {
  size_t bytes = al256((size_t)n_segs * sizeof(qwm_segment)) +
                 al256((size_t)n_segs * H * 2 * TAB_ELEMS * sizeof(uint16_t)) +
                 al256((size_t)n_segs * H * UT_ROWS * D * sizeof(uint16_t));
  const int ns = attention_splits(Tq, H, total_keys) + (active ? 1 : 0);
  if (ns > 1) {
    const size_t n = (size_t)ns * H * Tq;
    bytes += al256(n * D * 4) + 4 * al256(n * 4);
  }
  return bytes;
}

qwm_status launch_attention(const qwm_tokens* q, const qwm_segment* segs, int32_t n_segs, int64_t total_keys,
                            const qwm_tokens* ka, const qwm_tokens* va, float scale, float* out, float* lse,
                            int32_t* top1, void* ws, hipStream_t stream) {
  AttnArgs a{};
  a.q = q->ptr; a.qdtype = q->dtype; a.Tq = q->T; a.qst = q->stride_t; a.qsh = q->stride_h;
  a.n_segs = n_segs; a.scale = scale; a.out = out; a.lse = lse; a.top1 = top1; a.H = q->H;
  const int64_t Ta = ka ? ka->T : 0;
  const AttnPlan plan = attention_plan(q->T, q->H, n_segs > 0 ? total_keys : 0, Ta);
  a.nsplit = plan.nsplit; a.nsplit_a = plan.nsplit_a; a.nparts = plan.nparts;
  a.nqb = (int32_t)((q->T + AT_Q - 1) / AT_Q);
  a.units_p = a.nqb * a.nsplit * q->H;
  a.units = a.units_p + a.nqb * a.nsplit_a * q->H;
  if (ka) {
    a.ka = static_cast<const uint16_t*>(ka->ptr); a.kast = ka->stride_t; a.kash = ka->stride_h;
    a.va = static_cast<const uint16_t*>(va->ptr); a.vast = va->stride_t; a.vash = va->stride_h;
    a.Ta = Ta; a.kbase_a = n_segs > 0 ? total_keys : 0;
  }
  char* p = static_cast<char*>(ws);
  qwm_segment* dsegs = reinterpret_cast<qwm_segment*>(p);
  p += al256((size_t)n_segs * sizeof(qwm_segment));
  a.segs = dsegs;
  a.tabs = reinterpret_cast<uint16_t*>(p);
  p += al256((size_t)n_segs * q->H * 2 * TAB_ELEMS * sizeof(uint16_t));
  a.ut = reinterpret_cast<uint16_t*>(p);
  p += al256((size_t)n_segs * q->H * UT_ROWS * D * sizeof(uint16_t));
  if (a.nparts > 1) {
    const size_t n = (size_t)a.nparts * q->H * q->T;
    a.po = reinterpret_cast<float*>(p); p += al256(n * D * 4);
    a.pm = reinterpret_cast<float*>(p); p += al256(n * 4);
    a.pl = reinterpret_cast<float*>(p); p += al256(n * 4);
    a.ptv = reinterpret_cast<float*>(p); p += al256(n * 4);
    a.pti = reinterpret_cast<int32_t*>(p);
  }
  qwm_status s;
  // the host descriptors travel in kernel arguments, SEG_BATCH per launch
  for (int first = 0; first < n_segs; first += SEG_BATCH) {
    SegBatch b{};
    b.first = first;
    b.count = std::min(SEG_BATCH, n_segs - first);
    for (int i = 0; i < b.count; ++i) b.s[i] = segs[first + i];
    hipLaunchKernelGGL(attention_tables_kernel, dim3((unsigned)(b.count * q->H), D / 16), dim3(NC), 0, stream, b,
                       q->H, dsegs, const_cast<uint16_t*>(a.tabs), const_cast<uint16_t*>(a.ut));
    s = check_launch("attention tables");
    if (s != QWM_OK) return s;
  }
  const int per = (a.units + 7) / 8;
  const dim3 grid((unsigned)(per * 8));
  // one PSAC k-step covers ranks 8 and 16; a rank-32 segment needs two.  The
  // stored-format conversions (compacted coefficients, two-level scales) are
  // compiled in only when a segment uses them.
  int max_r = 8;
  bool ext = false;
  for (int i = 0; i < n_segs; ++i) {
    if (segs[i].U != nullptr && segs[i].r > max_r) max_r = segs[i].r;
    ext = ext || segs[i].k_cdir != nullptr || segs[i].k_scale2 != nullptr || segs[i].v_scale2 != nullptr;
  }
  const int variant = (top1 ? 4 : 0) + (max_r > 16 ? 2 : 0) + (ext ? 1 : 0);
  switch (variant) {
    case 0: hipLaunchKernelGGL((attention_kernel<false, 1, false>), grid, dim3(AT_T), 0, stream, a); break;
    case 1: hipLaunchKernelGGL((attention_kernel<false, 1, true>), grid, dim3(AT_T), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((attention_kernel<false, 2, false>), grid, dim3(AT_T), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((attention_kernel<false, 2, true>), grid, dim3(AT_T), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((attention_kernel<true, 1, false>), grid, dim3(AT_T), 0, stream, a); break;
    case 5: hipLaunchKernelGGL((attention_kernel<true, 1, true>), grid, dim3(AT_T), 0, stream, a); break;
    case 6: hipLaunchKernelGGL((attention_kernel<true, 2, false>), grid, dim3(AT_T), 0, stream, a); break;
    default: hipLaunchKernelGGL((attention_kernel<true, 2, true>), grid, dim3(AT_T), 0, stream, a); break;
  }
  s = check_launch("attention");
  if (s != QWM_OK || a.nparts == 1) return s;
  const dim3 g2((unsigned)((q->T + 7) / 8), (unsigned)q->H);
  if (top1) hipLaunchKernelGGL(attention_combine_kernel<true>, g2, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(attention_combine_kernel<false>, g2, dim3(256), 0, stream, a);
  return check_launch("attention merge");
}

qwm_status launch_attention_merge(const float* oa, const float* la, const float* ob, const float* lb, int64_t Tq,
                                  int32_t H, float* out, float* lse, hipStream_t stream) {
  const int64_t rows = Tq * H;
  hipLaunchKernelGGL(attention_merge_kernel, dim3((unsigned)((rows + 1) / 2)), dim3(256), 0, stream, oa, la, ob, lb, Tq,
                     H, out, lse);
  return check_launch("attention merge of two parts");
}

}  // namespace qwm_host
