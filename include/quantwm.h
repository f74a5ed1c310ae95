/*
 * quantwm.h — C ABI of libquantwm: the data-parallel hot path of QuantWM's
 * training-free, strictly causal 2-bit KV cache (Zhao et al., "QuantWM:
 * Temporally Consistent 2-Bit KV Cache Quantization for World Models and
 * Video Generation", arXiv 2609.26425 v2), for AMD MI355X (gfx950).
 *
 * Conventions shared by every call
 *  - Every buffer argument is DEVICE memory owned by the caller, except the
 *    descriptor arrays (qwm_tokens, qwm_qstats, qwm_packed, qwm_segment),
 *    which live on the host and are read during the call only.  The library
 *    never allocates, frees or keeps a pointer after a call returns.
 *  - Every call validates its arguments on the host first (no HIP call is made
 *    when validation fails), then only enqueues kernels on `stream` (a
 *    hipStream_t; NULL = the default stream) and returns.  Results are ready
 *    when the stream reaches that point.
 *  - Return value: QWM_OK, or an error code; qwm_last_error() returns a
 *    thread-local description of the last failure.  No exception crosses the
 *    ABI.  Calls are reentrant; calls that share output or state buffers must
 *    be ordered by the caller (same stream).
 *  - Shapes: head dim d = 128, residual groups of 64 channels (G = 2),
 *    n_c = 256 centroids (the configuration of the paper's implementation
 *    details, Sec. 5.1 / App. D.1), PSAC rank r = 8 by default and 16 or 32
 *    for the paper's rank ablation (App. C.2, Table 9).
 *  - bf16 and fp16 values travel as uint16_t bit patterns.
 *  - Token tensors are [T][H][d] with element strides (channel stride 1).
 *
 * Packed chunk layout (one chunk of T tokens, H heads; qwm_packed):
 *    codes   [H][T][d/4]  u8   INT2 residual codes, channel 4b+i in bits 2i..2i+1 of byte b
 *    idx     [H][T]       u8   centroid index
 *    scale   [H][T][G]    fp16 group step size s_g
 *    zeros   [H][zstride] u8   zero-points: token t owns the 4-bit field z_0 | z_1 << 2
 *                              in byte t/2 (low nibble for even t); zstride =
 *                              qwm_zeros_stride(T) = ceil(T/2) rounded up to 4
 *    c       [H][T][r]    i8   PSAC coefficients (keys only)
 *    c_scale [H][T]       fp16 PSAC coefficient scale (keys only)
 *  Dequantization: k0_hat_c = mu[idx]_c + s_g (q_c - z_g) (g = c / 64),
 *                  k_hat = k0_hat + (c_scale * c) U^T,  v_hat = mu_v[idx] + s (q - z).
 */
#ifndef QUANTWM_H
#define QUANTWM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QWM_ABI_VERSION 6
#define QWM_HEAD_DIM 128
#define QWM_GROUP 64
#define QWM_CENTROIDS 256
#define QWM_RANK 8        /* default PSAC rank */
#define QWM_MAX_RANK 32   /* supported ranks: 8, 16, 32 */

typedef enum {
  QWM_OK = 0,
  QWM_ERR_ARG = 1,          /* null / misaligned pointer, bad shape or stride, bad value */
  QWM_ERR_UNSUPPORTED = 2,  /* a shape this build does not implement (d, n_c, r, dtype) */
  QWM_ERR_WORKSPACE = 3,    /* workspace missing or smaller than qwm_workspace_bytes() */
  QWM_ERR_HIP = 4           /* a HIP launch failed; qwm_last_error() has the HIP text */
} qwm_status;

typedef enum { QWM_F32 = 0, QWM_BF16 = 1 } qwm_dtype;

/* Key-quantization flags.  0 = nearest centroid only (the QVG-style baseline). */
enum { QWM_QSAC = 1u, QWM_PSAC = 2u,
       /* the PSAC keep test (QuantWM method step (4)): a key keeps its
        * coefficients only if they lower its Query-weighted error
        * sum_c w_c e_c^2 (w under QSAC, else 1); otherwise C = 0, c_scale = 0.
        * The decision is taken in fp32. */
       QWM_PSAC_KEEP = 4u };

/* Workspace-sizing operation ids for qwm_workspace_bytes(). */
enum { QWM_OP_STATS = 0, QWM_OP_CENTROIDS = 1, QWM_OP_KEYS = 2, QWM_OP_VALUES = 3,
       QWM_OP_ATTENTION = 4, QWM_OP_ATTENTION_ACTIVE = 5, QWM_OP_KEEP_FULL = 6 };

typedef void* qwm_stream; /* hipStream_t */

/* A token tensor: element (t, h, c) at ptr + t*stride_t + h*stride_h + c. */
typedef struct {
  const void* ptr;   /* device; 16-byte aligned; rows of d elements contiguous */
  int32_t dtype;     /* qwm_dtype */
  int32_t H;         /* heads */
  int32_t d;         /* channels per head, must be 128 */
  int32_t reserved;
  int64_t T;         /* tokens */
  int64_t stride_t;  /* elements between consecutive tokens (multiple of 8) */
  int64_t stride_h;  /* elements between consecutive heads (multiple of 8) */
} qwm_tokens;

/* Per-head Query statistics (QuantWM Sec. 4.1-4.2, App. C.3, App. D.1). */
typedef struct {
  double* S;        /* [H][d][d] running sum of q q^T (in/out) */
  int64_t* n;       /* [H] Queries seen so far (in/out) */
  float* w;         /* [H][d] channel sensitivity diag(S)/n, 1 while n == 0 (out) */
  uint16_t* U;      /* [H][d][r] bf16 top-r eigenvectors of S/n (in/out: a finite nonzero U warm-starts
                       the eigen-solver; zero it, or leave the previous output, before a call;
                       a U with a non-finite entry is ignored; zero while n == 0) */
  float* lambda;    /* [H][r] their eigenvalues, descending (out) */
  float* energy;    /* [H] sum of the top-r eigenvalues / trace (out) */
  int32_t* iters;   /* [H] eigen-iterations used, negative if not converged; may be NULL */
  int32_t H, d, r, reserved;   /* r: 8, 16 or 32 (U [H][d][r], lambda [H][r]) */
} qwm_qstats;

/* One packed chunk (layout above).  c and c_scale are NULL for Values; for
 * keys c is [H][T][r] with r = 8, 16 or 32. */
typedef struct {
  uint8_t* codes;
  uint8_t* idx;
  uint16_t* scale;
  uint8_t* zeros;
  int8_t* c;
  uint16_t* c_scale;
  int64_t T;
  int32_t H, r;
} qwm_packed;

/* Optional device-side counters (int64, accumulated with atomics). */
typedef struct {
  int64_t nonfinite_rows;     /* tokens with a NaN/Inf channel: stored as idx 0, codes 0 */
  int64_t exact_fallbacks;    /* tokens whose centroid choice needed the exact (slow) path */
  int64_t scale_saturations;  /* group ranges beyond 3 * 65504, or PSAC coefficients beyond
                                 127 * 65504 (the fp16 scale saturates) */
  int64_t layout_overflows;   /* qwm_compact_coefficients: heads the arena could not hold */
} qwm_diag;

/* Where one head's PSAC coefficients of a chunk live after
 * qwm_compact_coefficients (QuantWM App. D.1: each chunk keeps the smaller of
 * a dense and a sparse layout, sparse indices included).  At arena + offset:
 *   dense  (layout 0): c [T][r] i8, then c_scale [T] fp16;
 *   sparse (layout 1): bitmap [ceil(T/64)] u64 (key 64 w + b kept iff bit b of
 *          word w), the kept count before each word [ceil(T/64)] u32, then the
 *          kept keys' c [count][r] i8 and c_scale [count] fp16 in key order.
 * Every section starts on a 16-byte boundary.  A key keeps coefficients iff its
 * c_scale is nonzero.  layout -1: the arena was too small (nothing stored). */
#define QWM_LAYOUT_DENSE 0
#define QWM_LAYOUT_SPARSE 1
#define QWM_LAYOUT_OVERFLOW (-1)
typedef struct {
  int32_t layout;
  int32_t count;    /* keys that keep coefficients */
  int64_t offset;   /* byte offset in the arena */
} qwm_cdir;

/* One cached chunk as read by qwm_attention.  Pointers address the whole
 * chunk ([H][...] arrays); centroid tables are [H][256][d] bf16; U is
 * [H][d][r] bf16 or NULL (no PSAC term: cold-start chunk or PSAC off); r is
 * the chunk's PSAC rank (8, 16 or 32: k_c is [H][T][r]).
 * k_cdir / k_carena: NULL, or the chunk's compacted coefficients
 * ([H] directory entries and their arena; k_c and k_c_scale are then unused).
 * k_scale2 / v_scale2: NULL for fp16 group steps in k_scale / v_scale, or the
 * [H][G] fp16 second-level scales of a two-level chunk, whose k_scale / v_scale
 * then hold [H][T][G] INT8 step codes (see qwm_two_level_scales). */
typedef struct {
  const uint8_t* k_codes; const uint8_t* k_idx; const uint16_t* k_scale; const uint8_t* k_zeros;
  const int8_t* k_c; const uint16_t* k_c_scale;
  const uint8_t* v_codes; const uint8_t* v_idx; const uint16_t* v_scale; const uint8_t* v_zeros;
  const uint16_t* k_centroids; const uint16_t* v_centroids; const uint16_t* U;
  int64_t T;
  int32_t r, reserved;
  const qwm_cdir* k_cdir; const uint8_t* k_carena;
  const uint16_t* k_scale2; const uint16_t* v_scale2;
} qwm_segment;

/* Update the per-head Query statistics with the Queries q (T may be 0) and
 * refresh w; with compute_basis != 0 also the principal basis U, lambda,
 * energy (QuantWM method step (1) and (4); Sec. 4.2: M_h = (1/N) sum q q^T,
 * w = diag(M_h), U_r = top-8 eigenvectors of M_h stored in BF16).
 * S accumulates in fp64; q may be QWM_BF16 or QWM_F32.
 * Eigenvector order: eigenvalue descending; sign: largest-|entry| positive.
 * r = 8: block subspace iteration warm-started from U; r = 16 or 32 (the
 * rank ablation): one-sided Jacobi on the whole 128 x 128 matrix, which
 * neither reads U nor reports iterations in a comparable way (iters = sweeps).
 * Workspace: qwm_workspace_bytes(QWM_OP_STATS, ...) bytes (0 today). */
qwm_status qwm_update_query_stats(const qwm_tokens* q, const qwm_qstats* st, int32_t compute_basis,
                                  void* ws, size_t ws_bytes, qwm_stream stream);

/* Build a table of n_centroids BF16 centroids per head for the tokens x by
 * `iters` Lloyd iterations (QVG's K-means, which QuantWM builds on: QuantWM
 * Sec. 2; QVG Sec. 2A/2C).  init == NULL: Forgy start with 256 distinct
 * tokens drawn by a SplitMix64-driven partial Fisher-Yates shuffle seeded with
 * seed + (head << 32); otherwise warm start from init ([H][256][d] bf16, may
 * equal centroids).  Assignment: nearest centroid (ties -> lowest index),
 * exact; update: bf16(mean of the members); empty clusters keep their value.
 * The mean is bf16(fl64(sum) / n) with the member sum exact: in 64-bit fixed
 * point per (head, channel), or, for a head holding a value finer than that
 * fixed-point unit, in fp64 in token order.  After the first iteration a token
 * is re-assigned only when distance bounds (upper to its centroid, lower to
 * the others, moved by how far the means moved) no longer settle its centroid.
 * Rows with a NaN or Inf channel take no part; diag->nonfinite_rows counts
 * them once per call.
 * Output centroids [H][256][d] bf16.  Requires T >= 256 when init == NULL.
 * Workspace: qwm_workspace_bytes(QWM_OP_CENTROIDS, T, H, ...). */
qwm_status qwm_build_centroids(const qwm_tokens* x, int32_t n_centroids, int32_t iters, uint64_t seed,
                               const uint16_t* init, uint16_t* centroids, qwm_diag* diag,
                               void* ws, size_t ws_bytes, qwm_stream stream);

/* Quantize one chunk of Keys (QuantWM Sec. 4.1 QSAC, Sec. 4.2 PSAC; method
 * steps (2)-(4)).  flags & QWM_QSAC: Query-aware distance d_Q with weights w
 * (NULL -> w = 1, the cold start), the M (1..256) nearest candidates by
 * (d_Q, index), final choice by (S, index) with S = sum_g (sum_{c in g} w_c) R_g^2,
 * R_g = max(0, max r) - min(0, min r) over the residual r = fl32(k - mu) in group g.
 * Without QWM_QSAC: nearest centroid.  Codec: s_g = smallest fp16 with 3 s_g >= R_g,
 * z_g = clamp(rne(-lo_g / s_g), 0, 3), q_c = clamp(rne(r_c / s_g) + z_g, 0, 3)
 * (rne = round half to even of the exact quotient; s_g = 0 -> z = q = 0).
 * flags & QWM_PSAC with U != NULL: E = k - k0_hat, C = E U (U [H][d][r] bf16,
 * r = out->r: 8, or 16 / 32 for the rank ablation, whose coefficients come from
 * a second, exact fp64 pass),
 * c_scale = smallest fp16 with 127 c_scale >= max|C|, c = clamp(rne(C / c_scale),
 * -127, 127); otherwise c = 0 and c_scale = 0.
 * out->T must equal k->T and out->H k->H.  Workspace: QWM_OP_KEYS. */
qwm_status qwm_quantize_keys(const qwm_tokens* k, const uint16_t* centroids, const float* w,
                             const uint16_t* U, int32_t M, uint32_t flags, const qwm_packed* out,
                             qwm_diag* diag, void* ws, size_t ws_bytes, qwm_stream stream);

/* qwm_quantize_keys for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and results, with no workspace argument.  The scratch they need
 * lives in a static device array of the library, one per device (about
 * 8.6 MB, held until the process ends), sized for at most
 * QWM_NOALLOC_MAX_HEADS heads and QWM_NOALLOC_MAX_TOKEN_HEADS token-heads
 * (H * T) per call; larger calls return QWM_ERR_UNSUPPORTED before any HIP
 * call.  Every call on one device shares that array: calls that may overlap
 * on one device (different streams, or threads without ordering) race and
 * must be ordered by the caller.  Each call re-initialises what it reads
 * (the work counter is cleared by its own first kernel, no memset), so no
 * state carries over from the previous call.  The call allocates and frees
 * nothing; its first call on a device looks up the array's address. */
#define QWM_NOALLOC_MAX_HEADS 64
#define QWM_NOALLOC_MAX_TOKEN_HEADS (1 << 21)
qwm_status qwm_quantize_keys_noalloc(const qwm_tokens* k, const uint16_t* centroids, const float* w,
                                     const uint16_t* U, int32_t M, uint32_t flags, const qwm_packed* out,
                                     qwm_diag* diag, qwm_stream stream);

/* Two-level group scales (rainbus digest, method step (3): group scales in
 * INT8 under an FP16 second level) for a chunk already quantized by
 * qwm_quantize_keys (keys != 0) or qwm_quantize_values (keys == 0): per (head,
 * group g) the second-level scale s2_g is the smallest power of two p >= 2^-24
 * with 255 p >= the largest fp16 step of the group; each token's step code is
 * q = min(ceil(s / p), floor(65504 / p)) and its effective step q p (an exact
 * fp16 value, never below s, so the codes still cover the range).  The codes
 * and zero-points are re-encoded with the effective steps; for keys the PSAC
 * coefficients are recomputed in fp64 from the new error (same flags, w and U
 * as the quantizing call; QWM_PSAC_KEEP applies the diagonal keep test).
 * x, centroids: the inputs of the quantizing call.  inout: the chunk (reads
 * idx and the fp16 scale array; rewrites codes, zeros and, for keys, c and
 * c_scale).  scale_q [H][T][G] u8, scale2 [H][G] fp16: outputs.  Afterwards
 * attention and the decoder read the chunk with k_scale = scale_q and
 * k_scale2 = scale2 (or the V fields).  No workspace. */
qwm_status qwm_two_level_scales(const qwm_tokens* x, const uint16_t* centroids, const float* w, const uint16_t* U,
                                uint32_t flags, int32_t keys, const qwm_packed* inout, uint8_t* scale_q,
                                uint16_t* scale2, qwm_diag* diag, qwm_stream stream);

/* The keep test with the full Query second moment (method step (4): the
 * coefficients stay only where they lower the Query-weighted error, here
 * e^T M_h e with M_h = S_h / n_h, the objective of the method section), as a
 * pass over keys quantized without QWM_PSAC_KEEP: a key keeps its
 * coefficients iff D^T S (D - 2 e) < 0, D = (c_scale c) U^T, e = k - k0_hat
 * recomputed from its stored codes and step (fp16 scales, or the two-level
 * scale_q and scale2 when scale2 is not NULL); otherwise c = 0, c_scale = 0.
 * Heads with n_h = 0 are left as they are.  S [H][128][128] fp64 and n [H] as
 * qwm_update_query_stats keeps them; U [H][d][r] the basis the keys were coded
 * with.  Decided in fp64 through U^T S and U^T S U.  Workspace:
 * QWM_OP_KEEP_FULL (T ignored, n = r). */
qwm_status qwm_psac_keep_full(const qwm_tokens* k, const uint16_t* centroids, const double* S, const int64_t* n,
                              const uint16_t* U, const qwm_packed* inout, const uint8_t* scale_q,
                              const uint16_t* scale2, void* ws, size_t ws_bytes, qwm_stream stream);

/* Store a chunk's PSAC coefficients in the smaller of the dense and the sparse
 * layout, per head (QuantWM App. D.1; the layouts are described at qwm_cdir).
 * keys: the chunk (reads c, c_scale, T, H, r).  Each head takes its bytes
 * from the arena with one device-side atomic add on *arena_used (int64,
 * device; the caller sets it, e.g. to 0) and records layout, count and offset
 * in dir[h] (device).  A head that does not fit gets layout -1 and is counted
 * in diag->layout_overflows.  arena: device, 256-byte aligned, arena_bytes
 * long; qwm_coefficient_bytes gives a head's size under either layout (the
 * dense one is the most a head can need). */
qwm_status qwm_compact_coefficients(const qwm_packed* keys, qwm_cdir* dir, uint8_t* arena, int64_t arena_bytes,
                                    int64_t* arena_used, qwm_diag* diag, qwm_stream stream);

/* Bytes of one head's coefficients under a layout (QWM_LAYOUT_DENSE or
 * QWM_LAYOUT_SPARSE) with T keys of which `count` keep coefficients, rank r. */
int64_t qwm_coefficient_bytes(int32_t layout, int64_t T, int64_t count, int32_t r);

/* The full-matrix ablation of QSAC (QuantWM App. C.4): as qwm_quantize_keys
 * with QWM_QSAC set, except that the M candidates are the M smallest by
 * ((k - mu)^T M_h (k - mu), index), M_h = S_h / n_h the Query second-moment
 * matrix (S [H][128][128] fp64 and n [H] int64 as qwm_update_query_stats keeps
 * them; M_h = I while n_h = 0).  The score S = sum_g W_g R_g^2, the codec, PSAC
 * and the keep test keep the diagonal weights w, as in that ablation.  Every
 * token takes the exact fp64 path (expanded form k^T S k - 2 (S k).mu + mu^T S mu),
 * so the call is much slower than the diagonal one; candidates whose quadratic
 * forms agree to about 1e-12 relative may order differently from a direct-form
 * evaluation.  flags: QWM_QSAC required; QWM_PSAC, QWM_PSAC_KEEP as above.
 * Workspace: QWM_OP_KEYS. */
qwm_status qwm_quantize_keys_fullq(const qwm_tokens* k, const uint16_t* centroids, const double* S,
                                   const int64_t* n, const float* w, const uint16_t* U, int32_t M,
                                   uint32_t flags, const qwm_packed* out, qwm_diag* diag, void* ws,
                                   size_t ws_bytes, qwm_stream stream);

/* Quantize one chunk of Values: nearest centroid plus the INT2 codec above,
 * no compensation (QuantWM Sec. 2 centroid-residual code; PSAC is Key-only).
 * Workspace: QWM_OP_VALUES. */
qwm_status qwm_quantize_values(const qwm_tokens* v, const uint16_t* centroids, const qwm_packed* out,
                               qwm_diag* diag, void* ws, size_t ws_bytes, qwm_stream stream);

/* Attention of the Queries q over every key of every segment (no mask):
 * out = softmax(scale * (Q K0_hat^T + (Q U) (c_scale c)^T)) V_hat
 * (the logit-side PSAC compensation of QuantWM's method section; the logits
 * of Sec. 3.3 with scale = 1/sqrt(d)).
 * segs: HOST array of n_segs descriptors (1 <= n_segs <= 4096) whose pointers
 * address device memory.  The library validates every descriptor before any
 * HIP call (QWM_ERR_ARG: T outside [1, 2^26) -- the kernel reaches a
 * segment's rows through 32-bit buffer ranges --, a null packed array or
 * table, a basis without coefficients, codes / tables / U not 16-byte, scales
 * / zeros not 4-byte, c not 8-byte aligned; QWM_ERR_UNSUPPORTED: 2^31 keys or
 * more in all), sums the keys itself and copies the descriptors into the
 * workspace through kernel arguments, so the host array may be freed as soon
 * as the call returns.  Keys are numbered in segment order.
 * q: bf16 or fp32 [Tq][H][d]; its values must lie in fp16's range
 * (|q| <= 65504), as must every centroid value and every reconstruction
 * mu + s (q - z): the dequantized tiles and Q are fp16 MFMA operands.
 * out [Tq][H][d] fp32; lse [H][Tq] fp32 (natural log of the softmax
 * denominator, may be NULL); top1 [H][Tq] int32 = argmax of the logits over
 * all keys (may be NULL).  Workspace: QWM_OP_ATTENTION with T = total keys,
 * n = Tq (query count) and n_segs. */
qwm_status qwm_attention(const qwm_tokens* q, const qwm_segment* segs, int32_t n_segs, float scale, float* out,
                         float* lse, int32_t* top1, void* ws, size_t ws_bytes, qwm_stream stream);

/* Log-sum-exp merge of two attention results of the same Queries over
 * disjoint key sets, e.g. the cached chunks and the newest one, computed by two
 * qwm_attention calls with lse.  The softmax of the method section's logits
 * over the union is the two parts' outputs weighted by e^lse: with
 * m = max(lse_a, lse_b), out = (e^(lse_a - m) out_a + e^(lse_b - m) out_b) /
 * (e^(lse_a - m) + e^(lse_b - m)) and lse = m + log of that denominator.
 * out_a, out_b, out [Tq][H][d] fp32; lse_a, lse_b, lse [H][Tq] fp32 (natural
 * log; -inf marks a part without keys; a row with no keys in either part gets
 * out = 0, lse = -inf).  lse may be NULL.  out may be out_a or out_b; lse must
 * not alias lse_a or lse_b (QWM_ERR_ARG).  Device buffers owned by the caller;
 * no workspace. */
qwm_status qwm_attention_merge(const float* out_a, const float* lse_a, const float* out_b, const float* lse_b,
                               int64_t Tq, int32_t H, float* out, float* lse, qwm_stream stream);

/* qwm_attention over the packed segments plus the active chunk, which stays
 * BF16 until it completes (QuantWM App. D.1: completed chunks are packed, the
 * active one is kept as it is).  segs: host array as for qwm_attention, same
 * checks; n_segs may be 0 (then segs may be NULL).  k_active, v_active:
 * [Ta][H][d] bf16 token descriptors (Ta >= 1, H equal to the queries', rows
 * 16-byte aligned, Ta * stride_t < 2^30 elements); row values must lie in
 * fp16's range (the kernel's tiles are fp16 MFMA operands).  Keys are
 * numbered packed segments first, then the active chunk (index
 * sum of the segments' T + t), for top1.  The active chunk runs on its own
 * key splits in the same launch; the log-sum-exp merge joins them.
 * Workspace: QWM_OP_ATTENTION_ACTIVE with T = all keys (packed + active),
 * n = Tq and n_segs. */
qwm_status qwm_attention_active(const qwm_tokens* q, const qwm_segment* segs, int32_t n_segs,
                                const qwm_tokens* k_active, const qwm_tokens* v_active, float scale, float* out,
                                float* lse, int32_t* top1, void* ws, size_t ws_bytes, qwm_stream stream);

/* Reconstruct one packed chunk in BF16: the decoder of QuantWM App. D.1 /
 * Fig. 9, which rebuilds temporary BF16 keys and values for a dense
 * attention (kept here to compare that design with the fused kernel).
 * K_hat = mu + s (q - z) + (c_s C) U^T (the PSAC term only when seg->U is
 * not NULL) and V_hat = mu + s (q - z), each element the bf16 RNE of its
 * exact value.  seg: HOST descriptor of a packed chunk (device pointers),
 * H heads; k_out, v_out: [T][H][d] bf16 device buffers
 * with element strides out_stride_t (>= d) and out_stride_h, 16-byte
 * aligned rows.  No workspace. */
qwm_status qwm_decode_segment(const qwm_segment* seg, int32_t H, uint16_t* k_out, uint16_t* v_out,
                              int64_t out_stride_t, int64_t out_stride_h, qwm_stream stream);

/* The residual of every token against its assigned centroid, in fp32:
 * out[t][h][c] = fl32(x[t][h][c] - centroids[h][idx[h][t]][c]).  This is the
 * centroid subtraction of QVG's smoothing step (QVG summary Sec. 2A); its
 * progressive residual quantization (Sec. 2B) repeats it stage by stage on
 * the previous stage's residual (bit_kv_cache_head_amd.prq_quantize composes
 * the stages from this call, qwm_build_centroids and qwm_quantize_values).
 * x: bf16 or fp32 tokens; centroids [H][256][d] bf16; idx [H][T] u8; out
 * [T][H][d] fp32 with element strides (multiples of 4, token stride >= d),
 * 16-byte aligned.  No workspace. */
qwm_status qwm_centroid_residual(const qwm_tokens* x, const uint16_t* centroids, const uint8_t* idx, float* out,
                                 int64_t out_stride_t, int64_t out_stride_h, qwm_stream stream);

/* Top-1 key of every Query over unquantized keys, the reference side of the
 * token-shift metric (QuantWM v2 Sec. 5.3: how often the key a Query attends
 * to most differs between the quantized cache and BF16).
 * top1[h][i] = argmax_j q_i . k_j (lowest j on ties), logits accumulated in
 * fp32 from exact bf16 products.  q: [Tq][H][d] bf16, k: [Tk][H][d] bf16 (all
 * keys in cache order); top1: [H][Tq] int32, device.  No workspace.
 * Returns QWM_ERR_UNSUPPORTED for fp32 inputs. */
qwm_status qwm_reference_top1(const qwm_tokens* q, const qwm_tokens* k, int32_t* top1, qwm_stream stream);

/* Bytes of workspace an operation needs (256-byte aligned pointer required).
 * QWM_OP_ATTENTION: T = total cached keys, n = number of queries, n_segs =
 * number of segments.  The workspace holds the segment descriptors, fp16
 * copies of every segment's centroid tables (n_segs * H * 128 KiB), every
 * segment's U_r as fp16 MFMA fragments (n_segs * H * 2 KiB) and the split-key
 * partials.
 * QWM_OP_ATTENTION_ACTIVE: the same with T = all keys (packed + active) and
 * one more partial set.  The other operations ignore n and n_segs. */
size_t qwm_workspace_bytes(int32_t op, int64_t T, int32_t H, int64_t n, int32_t n_segs);

/* Row stride of the zeros array for a chunk of T tokens. */
int64_t qwm_zeros_stride(int64_t T);

const char* qwm_last_error(void);
int32_t qwm_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QUANTWM_H */
