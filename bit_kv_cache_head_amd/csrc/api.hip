// C ABI of libquantwm: argument validation, workspace sizing, dispatch.
#include <cstdio>
#include <algorithm>
#include <string>

#include "common.hpp"

namespace qwm_host {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

qwm_status fail(qwm_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

qwm_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QWM_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return QWM_OK;
}

// defined in the kernel translation units
qwm_status launch_stats(const qwm_tokens* q, const qwm_qstats* st, int32_t compute_basis, hipStream_t stream);
qwm_status launch_keys(const qwm_tokens* k, const uint16_t* centroids, const float* w, const uint16_t* U,
                       int32_t M, uint32_t flags, const qwm_packed* out, qwm_diag* diag, void* ws,
                       hipStream_t stream);
qwm_status launch_attention_merge(const float* oa, const float* la, const float* ob, const float* lb, int64_t Tq,
                                  int32_t H, float* out, float* lse, hipStream_t stream);
qwm_status launch_keys_full(const qwm_tokens* k, const uint16_t* centroids, const double* S, const int64_t* n,
                            const float* w, const uint16_t* U, int32_t M, uint32_t flags, const qwm_packed* out,
                            qwm_diag* diag, void* ws, hipStream_t stream);
qwm_status launch_values(const qwm_tokens* v, const uint16_t* centroids, const qwm_packed* out, qwm_diag* diag,
                         void* ws, hipStream_t stream);
qwm_status launch_lloyd(const qwm_tokens* x, int32_t iters, uint64_t seed, const uint16_t* init, uint16_t* centroids,
                        qwm_diag* diag, void* ws, hipStream_t stream);
qwm_status launch_attention(const qwm_tokens* q, const qwm_segment* segs, int32_t n_segs, int64_t total_keys,
                            const qwm_tokens* ka, const qwm_tokens* va, float scale, float* out, float* lse,
                            int32_t* top1, void* ws, hipStream_t stream);
qwm_status launch_reference_top1(const qwm_tokens* q, const qwm_tokens* k, int32_t* top1, hipStream_t stream);
qwm_status launch_decode(const qwm_segment* seg, int32_t H, uint16_t* k_out, uint16_t* v_out, int64_t ost,
                         int64_t osh, hipStream_t stream);
qwm_status launch_centroid_residual(const qwm_tokens* x, const uint16_t* centroids, const uint8_t* idx, float* out,
                                   int64_t ost, int64_t osh, hipStream_t stream);
size_t select_ws_bytes(int64_t T, int32_t H, bool lloyd);
qwm_status noalloc_keys_scratch(void** ptr);
size_t keepfull_ws_bytes(int32_t H, int32_t r);
int64_t coefficient_layout_bytes(int32_t layout, int64_t T, int64_t count, int32_t r);
qwm_status launch_two_level(const qwm_tokens* x, const uint16_t* centroids, const float* w, const uint16_t* U,
                            uint32_t flags, const qwm_packed* io, bool keys, uint8_t* scale_q, uint16_t* scale2,
                            qwm_diag* diag, hipStream_t stream);
qwm_status launch_keep_full(const qwm_tokens* k, const uint16_t* centroids, const double* S, const int64_t* n,
                            const uint16_t* U, const qwm_packed* io, const uint8_t* scale_q, const uint16_t* scale2,
                            void* ws, hipStream_t stream);
qwm_status launch_compact(const qwm_packed* keys, qwm_cdir* dir, uint8_t* arena, int64_t arena_bytes,
                          int64_t* arena_used, qwm_diag* diag, hipStream_t stream);
size_t attention_ws_bytes(int64_t total_keys, int32_t H, int64_t Tq, int32_t n_segs, bool active);

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static qwm_status check_tokens(const qwm_tokens* t, const char* name, bool allow_empty) {
  if (!t) return fail(QWM_ERR_ARG, std::string(name) + ": null descriptor");
  if (t->d != qwm::D) return fail(QWM_ERR_UNSUPPORTED, std::string(name) + ": head dim must be 128");
  if (t->dtype != QWM_BF16 && t->dtype != QWM_F32) return fail(QWM_ERR_UNSUPPORTED, std::string(name) + ": dtype");
  if (t->H < 1) return fail(QWM_ERR_ARG, std::string(name) + ": H < 1");
  if (t->T < 0 || (!allow_empty && t->T < 1)) return fail(QWM_ERR_ARG, std::string(name) + ": bad token count");
  if (t->T > ((int64_t)1 << 31) / t->H) return fail(QWM_ERR_UNSUPPORTED, std::string(name) + ": H*T >= 2^31");
  if (t->T > 0 && !t->ptr) return fail(QWM_ERR_ARG, std::string(name) + ": null data");
  if (t->T > 0 && !aligned(t->ptr, 16)) return fail(QWM_ERR_ARG, std::string(name) + ": data not 16-byte aligned");
  if (t->stride_t < 0 || t->stride_h < 0 || t->stride_t % 8 || t->stride_h % 8)
    return fail(QWM_ERR_ARG, std::string(name) + ": strides must be non-negative multiples of 8 elements");
  if (t->T > 1 && t->stride_t < qwm::D && t->stride_t != 0)
    return fail(QWM_ERR_ARG, std::string(name) + ": token stride smaller than a row");
  return QWM_OK;
}

static qwm_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return QWM_OK;
  if (!ws) return fail(QWM_ERR_WORKSPACE, "workspace is null");
  if (!aligned(ws, 256)) return fail(QWM_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (have < need)
    return fail(QWM_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes, got " +
                                       std::to_string(have));
  return QWM_OK;
}

static qwm_status check_packed(const qwm_packed* p, const qwm_tokens* x, bool keys, bool psac) {
  if (!p) return fail(QWM_ERR_ARG, "packed: null descriptor");
  if (p->T != x->T || p->H != x->H) return fail(QWM_ERR_ARG, "packed: shape differs from the tokens");
  if (!p->codes || !p->idx || !p->scale || !p->zeros) return fail(QWM_ERR_ARG, "packed: null array");
  if (!aligned(p->codes, 16) || !aligned(p->scale, 4) || !aligned(p->zeros, 4))
    return fail(QWM_ERR_ARG, "packed: codes must be 16-byte, scale and zeros 4-byte aligned");
  if (keys) {
    if (!p->c || !p->c_scale) return fail(QWM_ERR_ARG, "packed keys: null c / c_scale");
    if (p->r != 8 && p->r != 16 && p->r != 32) return fail(QWM_ERR_UNSUPPORTED, "packed keys: rank must be 8, 16 or 32");
    if (!aligned(p->c, 8) || !aligned(p->c_scale, 2)) return fail(QWM_ERR_ARG, "packed keys: c misaligned");
  }
  (void)psac;
  return QWM_OK;
}

}  // namespace qwm_host

using namespace qwm_host;

extern "C" {

int32_t qwm_abi_version(void) { return QWM_ABI_VERSION; }

const char* qwm_last_error(void) { return g_last_error.c_str(); }

int64_t qwm_zeros_stride(int64_t T) { return qwm::zeros_stride(T); }

size_t qwm_workspace_bytes(int32_t op, int64_t T, int32_t H, int64_t n, int32_t n_segs) {
  if (T < 0 || H < 1) return 0;
  switch (op) {
    case QWM_OP_STATS: return 0;
    case QWM_OP_CENTROIDS: return select_ws_bytes(T, H, true);
    case QWM_OP_KEYS:
    case QWM_OP_VALUES: return select_ws_bytes(T, H, false);
    case QWM_OP_ATTENTION: return n_segs >= 1 ? attention_ws_bytes(T, H, n, n_segs, false) : 0;
    case QWM_OP_ATTENTION_ACTIVE: return n_segs >= 0 ? attention_ws_bytes(T, H, n, n_segs, true) : 0;
    case QWM_OP_KEEP_FULL: return (n == 8 || n == 16 || n == 32) ? keepfull_ws_bytes(H, (int32_t)n) : 0;
    default: return 0;
  }
}

qwm_status qwm_update_query_stats(const qwm_tokens* q, const qwm_qstats* st, int32_t compute_basis, void* ws,
                                  size_t ws_bytes, qwm_stream stream) {
  (void)ws; (void)ws_bytes;
  qwm_status s = check_tokens(q, "queries", true);
  if (s != QWM_OK) return s;
  if (!st) return fail(QWM_ERR_ARG, "stats: null descriptor");
  if (st->H != q->H || st->d != qwm::D) return fail(QWM_ERR_ARG, "stats: H / d differ from the queries");
  if (st->r != 8 && st->r != 16 && st->r != 32) return fail(QWM_ERR_UNSUPPORTED, "stats: rank must be 8, 16 or 32");
  if (!st->S || !st->n || !st->w) return fail(QWM_ERR_ARG, "stats: null S / n / w");
  if (!aligned(st->S, 8) || !aligned(st->n, 8) || !aligned(st->w, 4)) return fail(QWM_ERR_ARG, "stats: misaligned");
  if (compute_basis && (!st->U || !st->lambda || !st->energy))
    return fail(QWM_ERR_ARG, "stats: null U / lambda / energy");
  return launch_stats(q, st, compute_basis, static_cast<hipStream_t>(stream));
}

qwm_status qwm_build_centroids(const qwm_tokens* x, int32_t n_centroids, int32_t iters, uint64_t seed,
                               const uint16_t* init, uint16_t* centroids, qwm_diag* diag, void* ws,
                               size_t ws_bytes, qwm_stream stream) {
  qwm_status s = check_tokens(x, "tokens", false);
  if (s != QWM_OK) return s;
  if (n_centroids != qwm::NC) return fail(QWM_ERR_UNSUPPORTED, "n_centroids must be 256");
  if (iters < 0 || iters > 1000) return fail(QWM_ERR_ARG, "iters out of range [0, 1000]");
  if (!centroids || !aligned(centroids, 16)) return fail(QWM_ERR_ARG, "centroids: null or not 16-byte aligned");
  if (init && !aligned(init, 16)) return fail(QWM_ERR_ARG, "init: not 16-byte aligned");
  if (!init && x->T < qwm::NC) return fail(QWM_ERR_ARG, "seeded start needs at least 256 tokens");
  if (diag && !aligned(diag, 8)) return fail(QWM_ERR_ARG, "diag misaligned");
  s = check_ws(ws, ws_bytes, select_ws_bytes(x->T, x->H, true));
  if (s != QWM_OK) return s;
  return launch_lloyd(x, iters, seed, init, centroids, diag, ws, static_cast<hipStream_t>(stream));
}

static qwm_status check_keys_args(const qwm_tokens* k, const uint16_t* centroids, const float* w, const uint16_t* U,
                                  int32_t M, uint32_t flags, const qwm_packed* out, qwm_diag* diag) {
  qwm_status s = check_tokens(k, "keys", false);
  if (s != QWM_OK) return s;
  if (!centroids || !aligned(centroids, 16)) return fail(QWM_ERR_ARG, "centroids: null or not 16-byte aligned");
  if (flags & ~(uint32_t)(QWM_QSAC | QWM_PSAC | QWM_PSAC_KEEP)) return fail(QWM_ERR_ARG, "unknown flag bits");
  if ((flags & QWM_QSAC) && (M < 1 || M > qwm::NC)) return fail(QWM_ERR_ARG, "M must be in [1, 256]");
  if (w && !aligned(w, 4)) return fail(QWM_ERR_ARG, "w misaligned");
  if (U && !aligned(U, 16)) return fail(QWM_ERR_ARG, "U not 16-byte aligned");
  if (diag && !aligned(diag, 8)) return fail(QWM_ERR_ARG, "diag misaligned");
  return check_packed(out, k, true, (flags & QWM_PSAC) && U);
}

qwm_status qwm_quantize_keys(const qwm_tokens* k, const uint16_t* centroids, const float* w, const uint16_t* U,
                             int32_t M, uint32_t flags, const qwm_packed* out, qwm_diag* diag, void* ws,
                             size_t ws_bytes, qwm_stream stream) {
  qwm_status s = check_keys_args(k, centroids, w, U, M, flags, out, diag);
  if (s != QWM_OK) return s;
  s = check_ws(ws, ws_bytes, select_ws_bytes(k->T, k->H, false));
  if (s != QWM_OK) return s;
  return launch_keys(k, centroids, w, U, (flags & QWM_QSAC) ? M : 1, flags, out, diag, ws,
                     static_cast<hipStream_t>(stream));
}

qwm_status qwm_quantize_keys_noalloc(const qwm_tokens* k, const uint16_t* centroids, const float* w,
                                     const uint16_t* U, int32_t M, uint32_t flags, const qwm_packed* out,
                                     qwm_diag* diag, qwm_stream stream) {
  qwm_status s = check_keys_args(k, centroids, w, U, M, flags, out, diag);
  if (s != QWM_OK) return s;
  if (k->H > QWM_NOALLOC_MAX_HEADS || (int64_t)k->H * k->T > (int64_t)QWM_NOALLOC_MAX_TOKEN_HEADS)
    return fail(QWM_ERR_UNSUPPORTED, "no-allocation keys: at most " + std::to_string(QWM_NOALLOC_MAX_HEADS) +
                                         " heads and " + std::to_string(QWM_NOALLOC_MAX_TOKEN_HEADS) +
                                         " token-heads (H * T) per call");
  void* ws = nullptr;
  if ((s = noalloc_keys_scratch(&ws)) != QWM_OK) return s;
  return launch_keys(k, centroids, w, U, (flags & QWM_QSAC) ? M : 1, flags, out, diag, ws,
                     static_cast<hipStream_t>(stream));
}

qwm_status qwm_quantize_keys_fullq(const qwm_tokens* k, const uint16_t* centroids, const double* S,
                                   const int64_t* n, const float* w, const uint16_t* U, int32_t M, uint32_t flags,
                                   const qwm_packed* out, qwm_diag* diag, void* ws, size_t ws_bytes,
                                   qwm_stream stream) {
  qwm_status s = check_tokens(k, "keys", false);
  if (s != QWM_OK) return s;
  if (!centroids || !aligned(centroids, 16)) return fail(QWM_ERR_ARG, "centroids: null or not 16-byte aligned");
  if (!S || !n || !aligned(S, 8) || !aligned(n, 8)) return fail(QWM_ERR_ARG, "S / n: null or misaligned");
  if (flags & ~(uint32_t)(QWM_QSAC | QWM_PSAC | QWM_PSAC_KEEP)) return fail(QWM_ERR_ARG, "unknown flag bits");
  if (!(flags & QWM_QSAC)) return fail(QWM_ERR_ARG, "the full-matrix distance is a QSAC variant: set QWM_QSAC");
  if (M < 1 || M > qwm::NC) return fail(QWM_ERR_ARG, "M must be in [1, 256]");
  if (w && !aligned(w, 4)) return fail(QWM_ERR_ARG, "w misaligned");
  if (U && !aligned(U, 16)) return fail(QWM_ERR_ARG, "U not 16-byte aligned");
  if (diag && !aligned(diag, 8)) return fail(QWM_ERR_ARG, "diag misaligned");
  s = check_packed(out, k, true, (flags & QWM_PSAC) && U);
  if (s != QWM_OK) return s;
  s = check_ws(ws, ws_bytes, select_ws_bytes(k->T, k->H, false));
  if (s != QWM_OK) return s;
  return launch_keys_full(k, centroids, S, n, w, U, M, flags, out, diag, ws, static_cast<hipStream_t>(stream));
}

qwm_status qwm_quantize_values(const qwm_tokens* v, const uint16_t* centroids, const qwm_packed* out,
                               qwm_diag* diag, void* ws, size_t ws_bytes, qwm_stream stream) {
  qwm_status s = check_tokens(v, "values", false);
  if (s != QWM_OK) return s;
  if (!centroids || !aligned(centroids, 16)) return fail(QWM_ERR_ARG, "centroids: null or not 16-byte aligned");
  if (diag && !aligned(diag, 8)) return fail(QWM_ERR_ARG, "diag misaligned");
  s = check_packed(out, v, false, false);
  if (s != QWM_OK) return s;
  s = check_ws(ws, ws_bytes, select_ws_bytes(v->T, v->H, false));
  if (s != QWM_OK) return s;
  return launch_values(v, centroids, out, diag, ws, static_cast<hipStream_t>(stream));
}

// Every descriptor of a host segment array, before any HIP call: T in
// [1, 2^26) (the kernel reaches a segment-head's rows through 32-bit buffer
// ranges), every array the attention reads present and aligned, the total
// key count (returned in *total) below 2^31 (top-1 indices are int32).
static qwm_status check_segments(const qwm_segment* segs, int32_t n_segs, int64_t* total) {
  *total = 0;
  for (int32_t i = 0; i < n_segs; ++i) {
    const qwm_segment& g = segs[i];
    const std::string at = "segment " + std::to_string(i) + ": ";
    if (g.T < 1 || g.T >= ((int64_t)1 << 26)) return fail(QWM_ERR_ARG, at + "T must be in [1, 2^26)");
    if (g.r != 8 && g.r != 16 && g.r != 32) return fail(QWM_ERR_UNSUPPORTED, at + "rank must be 8, 16 or 32");
    if (!g.k_codes || !g.k_idx || !g.k_scale || !g.k_zeros || !g.v_codes || !g.v_idx || !g.v_scale ||
        !g.v_zeros || !g.k_centroids || !g.v_centroids)
      return fail(QWM_ERR_ARG, at + "a packed array or centroid table is null");
    if (g.U && (!g.k_c || !g.k_c_scale)) return fail(QWM_ERR_ARG, at + "a basis without PSAC coefficients");
    if (!aligned(g.k_codes, 16) || !aligned(g.v_codes, 16) || !aligned(g.k_scale, 4) || !aligned(g.v_scale, 4) ||
        !aligned(g.k_zeros, 4) || !aligned(g.v_zeros, 4) || !aligned(g.k_centroids, 16) ||
        !aligned(g.v_centroids, 16) || (g.U && (!aligned(g.U, 16) || !aligned(g.k_c, 8) || !aligned(g.k_c_scale, 2))))
      return fail(QWM_ERR_ARG, at + "misaligned array (codes and tables 16 B, scales and zeros 4 B, c 8 B, U 16 B)");
    if (g.k_cdir && (!g.k_carena || !aligned(g.k_cdir, 8) || !aligned(g.k_carena, 16)))
      return fail(QWM_ERR_ARG, at + "a coefficient directory needs its arena (directory 8-byte, arena 16-byte aligned)");
    if ((g.k_scale2 && !aligned(g.k_scale2, 4)) || (g.v_scale2 && !aligned(g.v_scale2, 4)))
      return fail(QWM_ERR_ARG, at + "second-level scales misaligned");
    *total += g.T;
    if (*total >= ((int64_t)1 << 31)) return fail(QWM_ERR_UNSUPPORTED, "more than 2^31 - 1 keys in all");
  }
  return QWM_OK;
}

static qwm_status check_attention_common(const qwm_tokens* q, float scale, const float* out, const float* lse,
                                         const int32_t* top1) {
  qwm_status s = check_tokens(q, "queries", false);
  if (s != QWM_OK) return s;
  if (!(scale > 0.0f) || !__builtin_isfinite(scale)) return fail(QWM_ERR_ARG, "scale must be finite and positive");
  if (!out || !aligned(out, 16)) return fail(QWM_ERR_ARG, "out: null or not 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(QWM_ERR_ARG, "lse misaligned");
  if (top1 && !aligned(top1, 4)) return fail(QWM_ERR_ARG, "top1 misaligned");
  return QWM_OK;
}

qwm_status qwm_attention(const qwm_tokens* q, const qwm_segment* segs, int32_t n_segs, float scale, float* out,
                         float* lse, int32_t* top1, void* ws, size_t ws_bytes, qwm_stream stream) {
  qwm_status s = check_attention_common(q, scale, out, lse, top1);
  if (s != QWM_OK) return s;
  if (n_segs < 1 || n_segs > 4096) return fail(QWM_ERR_ARG, "n_segs must be in [1, 4096]");
  if (!segs) return fail(QWM_ERR_ARG, "segments: null host array");
  int64_t total_keys = 0;
  if ((s = check_segments(segs, n_segs, &total_keys)) != QWM_OK) return s;
  s = check_ws(ws, ws_bytes, attention_ws_bytes(total_keys, q->H, q->T, n_segs, false));
  if (s != QWM_OK) return s;
  return launch_attention(q, segs, n_segs, total_keys, nullptr, nullptr, scale, out, lse, top1, ws,
                          static_cast<hipStream_t>(stream));
}

qwm_status qwm_decode_segment(const qwm_segment* seg, int32_t H, uint16_t* k_out, uint16_t* v_out,
                              int64_t out_stride_t, int64_t out_stride_h, qwm_stream stream) {
  if (!seg) return fail(QWM_ERR_ARG, "decode: null segment descriptor");
  if (H < 1 || seg->T < 1) return fail(QWM_ERR_ARG, "decode: H and T must be positive");
  if ((int64_t)H * seg->T >= ((int64_t)1 << 31)) return fail(QWM_ERR_UNSUPPORTED, "decode: H*T >= 2^31");
  if (!seg->k_codes || !seg->k_idx || !seg->k_scale || !seg->k_zeros || !seg->v_codes || !seg->v_idx ||
      !seg->v_scale || !seg->v_zeros || !seg->k_centroids || !seg->v_centroids)
    return fail(QWM_ERR_ARG, "decode: a packed array or centroid table is null");
  if (seg->U && (!seg->k_c || !seg->k_c_scale)) return fail(QWM_ERR_ARG, "decode: PSAC basis without coefficients");
  if (seg->r != 8 && seg->r != 16 && seg->r != 32) return fail(QWM_ERR_UNSUPPORTED, "decode: rank must be 8, 16 or 32");
  if (seg->k_cdir && !seg->k_carena) return fail(QWM_ERR_ARG, "decode: a coefficient directory needs its arena");
  if (!aligned(seg->k_codes, 16) || !aligned(seg->v_codes, 16) || !aligned(seg->k_centroids, 16) ||
      !aligned(seg->v_centroids, 16) || !aligned(seg->k_scale, 4) || !aligned(seg->v_scale, 4))
    return fail(QWM_ERR_ARG, "decode: misaligned packed arrays");
  if (!k_out || !v_out || !aligned(k_out, 16) || !aligned(v_out, 16))
    return fail(QWM_ERR_ARG, "decode: outputs null or not 16-byte aligned");
  if (out_stride_t < qwm::D || out_stride_h < 0 || out_stride_t % 8 || out_stride_h % 8)
    return fail(QWM_ERR_ARG, "decode: output strides must be multiples of 8 elements, token stride >= d");
  return launch_decode(seg, H, k_out, v_out, out_stride_t, out_stride_h, static_cast<hipStream_t>(stream));
}

qwm_status qwm_centroid_residual(const qwm_tokens* x, const uint16_t* centroids, const uint8_t* idx, float* out,
                                 int64_t out_stride_t, int64_t out_stride_h, qwm_stream stream) {
  qwm_status s = check_tokens(x, "tokens", false);
  if (s != QWM_OK) return s;
  if (!centroids || !aligned(centroids, 16) || !idx) return fail(QWM_ERR_ARG, "residual: null or misaligned table/idx");
  if (!out || !aligned(out, 16)) return fail(QWM_ERR_ARG, "residual: output null or not 16-byte aligned");
  if (out_stride_t < qwm::D || out_stride_h < 0 || out_stride_t % 4 || out_stride_h % 4)
    return fail(QWM_ERR_ARG, "residual: output strides must be multiples of 4 elements, token stride >= d");
  return launch_centroid_residual(x, centroids, idx, out, out_stride_t, out_stride_h, static_cast<hipStream_t>(stream));
}

qwm_status qwm_attention_merge(const float* out_a, const float* lse_a, const float* out_b, const float* lse_b,
                               int64_t Tq, int32_t H, float* out, float* lse, qwm_stream stream) {
  if (Tq < 1 || H < 1 || Tq * H >= ((int64_t)1 << 31)) return fail(QWM_ERR_ARG, "merge: Tq, H out of range");
  if (!out_a || !lse_a || !out_b || !lse_b || !out) return fail(QWM_ERR_ARG, "merge: null buffer");
  if (!aligned(out_a, 4) || !aligned(lse_a, 4) || !aligned(out_b, 4) || !aligned(lse_b, 4) || !aligned(out, 4) ||
      (lse && !aligned(lse, 4)))
    return fail(QWM_ERR_ARG, "merge: misaligned buffer");
  if (lse && (lse == lse_a || lse == lse_b)) return fail(QWM_ERR_ARG, "merge: lse must not alias lse_a or lse_b");
  return launch_attention_merge(out_a, lse_a, out_b, lse_b, Tq, H, out, lse, static_cast<hipStream_t>(stream));
}

qwm_status qwm_attention_active(const qwm_tokens* q, const qwm_segment* segs, int32_t n_segs,
                                const qwm_tokens* k_active, const qwm_tokens* v_active, float scale, float* out,
                                float* lse, int32_t* top1, void* ws, size_t ws_bytes, qwm_stream stream) {
  qwm_status s = check_attention_common(q, scale, out, lse, top1);
  if (s != QWM_OK) return s;
  if (n_segs < 0 || n_segs > 4096) return fail(QWM_ERR_ARG, "n_segs must be in [0, 4096]");
  if (n_segs > 0 && !segs) return fail(QWM_ERR_ARG, "segments: null host array");
  int64_t total_keys = 0;
  if ((s = check_segments(segs, n_segs, &total_keys)) != QWM_OK) return s;
  if ((s = check_tokens(k_active, "active keys", false)) != QWM_OK) return s;
  if ((s = check_tokens(v_active, "active values", false)) != QWM_OK) return s;
  if (k_active->dtype != QWM_BF16 || v_active->dtype != QWM_BF16)
    return fail(QWM_ERR_UNSUPPORTED, "the active chunk must be bf16");
  if (k_active->T != v_active->T || k_active->H != q->H || v_active->H != q->H)
    return fail(QWM_ERR_ARG, "active chunk: K and V must share T, and H must match the queries");
  if ((k_active->T > 1 && k_active->stride_t == 0) || (v_active->T > 1 && v_active->stride_t == 0))
    return fail(QWM_ERR_ARG, "active chunk: zero token stride");
  if (k_active->T * std::max<int64_t>(k_active->stride_t, qwm::D) >= ((int64_t)1 << 30) ||
      v_active->T * std::max<int64_t>(v_active->stride_t, qwm::D) >= ((int64_t)1 << 30))
    return fail(QWM_ERR_UNSUPPORTED, "active chunk: T * stride_t must stay below 2^30 elements");
  if (total_keys + k_active->T >= ((int64_t)1 << 31)) return fail(QWM_ERR_UNSUPPORTED, "more than 2^31 - 1 keys in all");
  s = check_ws(ws, ws_bytes, attention_ws_bytes(total_keys + k_active->T, q->H, q->T, n_segs, true));
  if (s != QWM_OK) return s;
  return launch_attention(q, segs, n_segs, total_keys, k_active, v_active, scale, out, lse, top1, ws,
                          static_cast<hipStream_t>(stream));
}

qwm_status qwm_two_level_scales(const qwm_tokens* x, const uint16_t* centroids, const float* w, const uint16_t* U,
                                uint32_t flags, int32_t keys, const qwm_packed* inout, uint8_t* scale_q,
                                uint16_t* scale2, qwm_diag* diag, qwm_stream stream) {
  qwm_status s = check_tokens(x, "tokens", false);
  if (s != QWM_OK) return s;
  if (!centroids || !aligned(centroids, 16)) return fail(QWM_ERR_ARG, "centroids: null or not 16-byte aligned");
  if (flags & ~(uint32_t)(QWM_QSAC | QWM_PSAC | QWM_PSAC_KEEP)) return fail(QWM_ERR_ARG, "unknown flag bits");
  if (w && !aligned(w, 4)) return fail(QWM_ERR_ARG, "w misaligned");
  if (U && !aligned(U, 16)) return fail(QWM_ERR_ARG, "U not 16-byte aligned");
  if (diag && !aligned(diag, 8)) return fail(QWM_ERR_ARG, "diag misaligned");
  if ((s = check_packed(inout, x, keys != 0, false)) != QWM_OK) return s;
  if (!scale_q || !scale2 || !aligned(scale_q, 2) || !aligned(scale2, 4))
    return fail(QWM_ERR_ARG, "scale_q / scale2: null or misaligned");
  return launch_two_level(x, centroids, w, keys ? U : nullptr, keys ? flags : 0u, inout, keys != 0, scale_q, scale2,
                          diag, static_cast<hipStream_t>(stream));
}

qwm_status qwm_psac_keep_full(const qwm_tokens* k, const uint16_t* centroids, const double* S, const int64_t* n,
                              const uint16_t* U, const qwm_packed* inout, const uint8_t* scale_q,
                              const uint16_t* scale2, void* ws, size_t ws_bytes, qwm_stream stream) {
  qwm_status s = check_tokens(k, "keys", false);
  if (s != QWM_OK) return s;
  if (!centroids || !aligned(centroids, 16)) return fail(QWM_ERR_ARG, "centroids: null or not 16-byte aligned");
  if (!S || !n || !aligned(S, 8) || !aligned(n, 8)) return fail(QWM_ERR_ARG, "S / n: null or misaligned");
  if (!U || !aligned(U, 16)) return fail(QWM_ERR_ARG, "U: null or not 16-byte aligned");
  if ((s = check_packed(inout, k, true, true)) != QWM_OK) return s;
  if (scale2 && (!scale_q || !aligned(scale2, 4))) return fail(QWM_ERR_ARG, "two-level scales: scale_q missing");
  s = check_ws(ws, ws_bytes, keepfull_ws_bytes(k->H, inout->r));
  if (s != QWM_OK) return s;
  return launch_keep_full(k, centroids, S, n, U, inout, scale_q, scale2, ws, static_cast<hipStream_t>(stream));
}

qwm_status qwm_compact_coefficients(const qwm_packed* keys, qwm_cdir* dir, uint8_t* arena, int64_t arena_bytes,
                                    int64_t* arena_used, qwm_diag* diag, qwm_stream stream) {
  if (!keys) return fail(QWM_ERR_ARG, "keys: null descriptor");
  if (keys->T < 1 || keys->H < 1 || keys->T >= ((int64_t)1 << 26)) return fail(QWM_ERR_ARG, "keys: T in [1, 2^26), H >= 1");
  if (!keys->c || !keys->c_scale || !aligned(keys->c, 8) || !aligned(keys->c_scale, 2))
    return fail(QWM_ERR_ARG, "keys: c / c_scale null or misaligned");
  if (keys->r != 8 && keys->r != 16 && keys->r != 32) return fail(QWM_ERR_UNSUPPORTED, "rank must be 8, 16 or 32");
  if (!dir || !aligned(dir, 8)) return fail(QWM_ERR_ARG, "dir: null or misaligned");
  if (!arena || !aligned(arena, 256) || arena_bytes < 0) return fail(QWM_ERR_ARG, "arena: null or not 256-byte aligned");
  if (!arena_used || !aligned(arena_used, 8)) return fail(QWM_ERR_ARG, "arena_used: null or misaligned");
  if (diag && !aligned(diag, 8)) return fail(QWM_ERR_ARG, "diag misaligned");
  return launch_compact(keys, dir, arena, arena_bytes, arena_used, diag, static_cast<hipStream_t>(stream));
}

int64_t qwm_coefficient_bytes(int32_t layout, int64_t T, int64_t count, int32_t r) {
  if (T < 0 || count < 0 || count > T || (r != 8 && r != 16 && r != 32)) return -1;
  if (layout != QWM_LAYOUT_DENSE && layout != QWM_LAYOUT_SPARSE) return -1;
  return coefficient_layout_bytes(layout, T, count, r);
}

qwm_status qwm_reference_top1(const qwm_tokens* q, const qwm_tokens* k, int32_t* top1, qwm_stream stream) {
  qwm_status s = check_tokens(q, "queries", false);
  if (s != QWM_OK) return s;
  s = check_tokens(k, "keys", false);
  if (s != QWM_OK) return s;
  if (q->dtype != QWM_BF16 || k->dtype != QWM_BF16)
    return fail(QWM_ERR_UNSUPPORTED, "reference top-1: queries and keys must be bf16");
  if (q->H != k->H) return fail(QWM_ERR_ARG, "reference top-1: queries and keys differ in H");
  if (k->T > ((int64_t)1 << 31) - 64) return fail(QWM_ERR_UNSUPPORTED, "reference top-1: too many keys");
  if (!top1 || !aligned(top1, 4)) return fail(QWM_ERR_ARG, "top1: null or misaligned");
  return launch_reference_top1(q, k, top1, static_cast<hipStream_t>(stream));
}

}  // extern "C"
