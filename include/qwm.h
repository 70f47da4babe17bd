/*
 * qwm.h -- C ABI of the QuantWM 2-bit KV cache for MI355X (gfx950).
 *
 * QuantWM (arXiv 2609.26425; abstracts on fugumt.com and ai.info, article
 * on roboind.com) keeps the KV cache of an autoregressive video world model
 * in 2 bits per element:
 *   - QSAC (roboind.com article, section "Step 1"; the abstracts name it as
 *     clustering aware of quantization sensitivity): each Key takes a high-precision
 *     centroid chosen by historical-Query sensitivity and residual range, and
 *     the Key-centroid residual is stored as per-group INT2;
 *   - Values are stored as plain per-group INT2;
 *   - PSAC (section "Step 2"; attention compensation in a principal subspace): the Key
 *     error left after quantization is projected on the top-r principal
 *     directions of historical Queries, r coefficients per token are kept,
 *     and (q . U_r) . coef is added back to every attention logit.
 * Two switches give the baseline the article ("Step 1") compares against,
 * QVG, and the ablations between: the centroid rule (QSAC objective or the
 * nearest centroid) and the PSAC rank (0 turns compensation off). The
 * article's attention analysis ("Table 1") counts how often a Query's
 * top-scoring historical token changes under quantization;
 * qwm_attend_top1 computes that token for the cache and for full-precision
 * Keys.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor argument is a DEVICE pointer owned by the caller,
 *   contiguous, row-major, on the device that was current at qwm_create.
 *   The batch dimension (B = 1) is folded into heads.
 *     q, k, v, k_self, v_self, q_hist, keys : [heads][n][head_dim] in the
 *         cache dtype (QWM_BF16: bfloat16 bit patterns; QWM_F32: float).
 *     out : [heads][n_q][head_dim] float.
 *     C   : [heads][n_centroids][head_dim] in the cache dtype.
 *     S_G : [heads][head_dim / group] float.     U_r : [heads][head_dim][rank] float.
 * - The library allocates nothing. All of its state lives in a caller
 *   supplied device arena of qwm_arena_bytes() bytes (e.g. a torch uint8
 *   tensor). The handle itself is a small host object.
 * - Work is enqueued on the HIP stream given at qwm_create; the caller keeps
 *   input buffers alive until that stream has passed the call (every read of
 *   a caller buffer is enqueued on it). Three calls block the host:
 *   qwm_profile_read waits for the timing events it reads,
 *   qwm_profile_work for the counter it reads, and qwm_destroy
 *   waits for the eigensolve stream (when one was started) before releasing
 *   it. Every other call only enqueues work. The one exception
 *   to the single stream is the eigensolve of qwm_build_subspace, which
 *   reads arena memory only and runs on a stream of the library's own
 *   (default priority) so that later work overlaps it; the cache stream
 *   waits for it before the staged calibration is committed, imported over
 *   or exported, and before the next qwm_build_subspace.
 * - A handle is not thread-safe; calls on one handle must not overlap.
 * - Every call returns a qwm_status and never throws. Arguments are checked
 *   on the host before anything is enqueued; a call that fails a check has
 *   no side effect. qwm_last_error() returns a message for the last failure
 *   of the calling thread.
 * - Non-finite inputs are undefined behaviour, and so are Key and Value
 *   magnitudes at or above 65504 and group ranges (max - min of 32 channels,
 *   Key residuals included) at or above 65472: zero-points, steps, their
 *   triples and the dequantized k and v are fp16.
 */
#ifndef QWM_H_
#define QWM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qwm_cache qwm_cache; /* opaque */

typedef enum {
  QWM_OK = 0,
  QWM_ERR_INVALID_ARG = -1,    /* null pointer, negative size, bad enum value */
  QWM_ERR_UNSUPPORTED = -2,    /* head_dim not 64/128, group not 32, n_centroids not 1..256,
                                  rank not 0..16, max_epochs not 1..64 */
  QWM_ERR_CAPACITY = -3,       /* length + n > capacity, n beyond a max_* bound, too many epochs */
  QWM_ERR_STATE = -4,          /* append/attend before a committed epoch; build_centroids
                                  before build_subspace */
  QWM_ERR_HIP = -5,            /* a HIP runtime or launch error (message holds the HIP text) */
  QWM_ERR_ARENA_TOO_SMALL = -6 /* arena smaller than qwm_arena_bytes() or misaligned */
} qwm_status;

typedef enum { QWM_BF16 = 0, QWM_F32 = 1 } qwm_dtype;

typedef enum {
  QWM_SELF_NONE = 0,   /* no self segment */
  QWM_SELF_FULL = 1,   /* every Query sees every self token (bidirectional chunk) */
  QWM_SELF_CAUSAL = 2  /* Query i sees self tokens 0..i (requires n_self == n_q) */
} qwm_self_mask;

/* Centroid rule of quantize-on-insert and of the centroid build. */
typedef enum {
  QWM_OBJ_QSAC = 0,    /* QSAC: sum_G S_G (max_G r - min_G r)^2 (roboind.com "Step 1") */
  QWM_OBJ_NEAREST = 1, /* QVG baseline: nearest centroid, sum_j r_j^2 per group in
                          channel order, groups added in order (float32) */
  QWM_OBJ_POSTQ = 2    /* the error the INT2 quantization actually leaves:
                          sum_G S_G sum_j (r_j - rhat_j)^2, rhat from the cache's own
                          per-group quantizer (float32, channel order, groups in order) */
} qwm_objective;

typedef struct {
  int32_t heads;            /* >= 1 */
  int32_t head_dim;         /* 64 or 128 */
  int32_t group;            /* channels per INT2 group: 32 */
  int32_t n_centroids;      /* 1..256 (ids are stored as u8) */
  int32_t rank;             /* PSAC rank r: 0..16 (0: no compensation, no coefficients) */
  int32_t max_epochs;       /* calibration epochs kept: 1..64 */
  int64_t capacity_tokens;  /* tokens per head the cache can hold, 1 .. 2^26 */
  int32_t dtype;            /* qwm_dtype of K/V/Q inputs and of the centroid table */
  int32_t objective;        /* qwm_objective */
  int64_t max_query_tokens; /* largest n_q of qwm_attend (sizes split-KV scratch) */
  int64_t max_build_tokens; /* largest n_keys of qwm_build_centroids, 1 .. 2^22 */
} qwm_desc;

/* Bytes of device arena a cache with this description needs (alignment 256). */
qwm_status qwm_arena_bytes(const qwm_desc* desc, size_t* bytes);

/* Bytes the stored state of a cache with this description occupies when it
 * holds n_tokens tokens per head in n_epochs epochs, from the arena layout:
 *   record_bytes = heads * n_tokens * (head_dim/4 K codes + head_dim/4 V codes
 *                  + 4 (head_dim/group) K zero-point|step words + the same for
 *                  V + 1 centroid id + 2 rank PSAC coefficients),
 *   table_bytes  = n_epochs * heads * (n_centroids * head_dim centroid values
 *                  in the cache dtype + 4 (head_dim/group) S_G + 4 head_dim rank U_r).
 * A bf16 K/V cache of the same tokens takes heads * n_tokens * 4 * head_dim
 * bytes; their ratio is the compression the roboind.com article reports
 * ("Figure 4"), which counts centroids, quantization parameters and
 * compensation data. Host arithmetic only (no device needed).
 * 0 <= n_tokens <= capacity_tokens, 0 <= n_epochs <= max_epochs. */
qwm_status qwm_storage_bytes(const qwm_desc* desc, int64_t n_tokens, int32_t n_epochs, size_t* record_bytes,
                             size_t* table_bytes);

/* Create a cache in `dev_arena` (device memory, 256-byte aligned, at least
 * qwm_arena_bytes bytes, owned by the caller and kept alive until
 * qwm_destroy). `stream` is a hipStream_t (NULL = the default stream). The
 * cache starts empty with no committed epoch. */
qwm_status qwm_create(const qwm_desc* desc, void* dev_arena, size_t arena_bytes, void* stream,
                      qwm_cache** out);
qwm_status qwm_destroy(qwm_cache* cache);

/* PSAC basis and QSAC sensitivity from n_hist historical Queries q_hist
 * [heads][n_hist][head_dim] (fugumt.com abstract: QSAC weighs channels by how
 * sensitive historical Queries are to them, PSAC works in their dominant
 * subspace; roboind.com "Step 2": the energy of historical Queries sits in a
 * few principal directions).
 * S_G = sum over the group's channels of mean q_j^2 (float64, stored float32);
 * U_r = top-r eigenvectors of the uncentered Gram Q^T Q (float64 on the
 * device: Householder tridiagonalization, multisection, twisted
 * factorization), largest-magnitude entry of each column positive. The
 * result goes to a staged epoch that qwm_build_centroids commits. S_G is
 * ready on the cache stream when the call returns; U_r is computed on the
 * library's eigensolve stream (see above); at rank 0 there is no U_r and
 * nothing runs there. 1 <= n_hist. */
qwm_status qwm_build_subspace(qwm_cache* cache, const void* q_hist, int64_t n_hist);

/* QSAC centroid table from n_keys Keys [heads][n_keys][head_dim]
 * (roboind.com "Step 1": Keys are grouped around high-precision centers):
 * seeds c_i = key floor(i * n_keys / n_centroids), then `iters` Lloyd
 * iterations that assign by the cache's centroid rule (the QSAC objective of
 * the staged sensitivity, or the nearest centroid) and replace each centroid
 * by the float64 mean of its Keys rounded once to the cache dtype (an empty
 * cluster keeps its centroid). Commits the staged epoch: tokens appended from
 * now on use it. An epoch that holds no token yet is replaced rather than
 * kept. Needs a staged qwm_build_subspace, except with QWM_OBJ_NEAREST at
 * rank 0, where the epoch's S_G is then zero.
 * 1 <= n_keys <= max_build_tokens, 0 <= iters. */
qwm_status qwm_build_centroids(qwm_cache* cache, const void* keys, int64_t n_keys, int32_t iters);

/* Quantize-on-insert of n_tokens new tokens k, v [heads][n_tokens][head_dim]
 * with the current epoch. Per token and head:
 *   id = argmin_c sum_G S_G (max_G(k - c) - min_G(k - c))^2 in float32, ties
 *        to the smallest id (QSAC, roboind.com "Step 1"), or with
 *        QWM_OBJ_NEAREST / QWM_OBJ_POSTQ argmin_c of the squared distance /
 *        the weighted post-quantization error (qwm_objective);
 *   the residual k - c_id and the Value each get per-group (32 channels)
 *   asymmetric INT2: fp16 zero-point = largest fp16 <= group min, fp16 step =
 *   smallest fp16 >= (max - zp) / 3 whose triple is an fp16 value (so every
 *   code * step is exactly an fp16), codes = clamp(rint((x - zp) / step), 0, 3);
 *   coef = U_r^T (k - (c_id + reconstructed residual)), float64, rounded once
 *   to fp16 (PSAC, "Step 2"); none at rank 0.
 * The records go to positions length .. length + n_tokens - 1 and the length
 * advances. Bit-identical whether tokens arrive in one call or several.
 * n_tokens = 0 does nothing after the state check and reads nothing: k and
 * v may then be NULL. */
qwm_status qwm_quantize_append(qwm_cache* cache, const void* k, const void* v, int64_t n_tokens);

/* Attention of n_q Queries q [heads][n_q][head_dim] over every cached token
 * (all of them are in the chunk's past) plus an optional self segment of
 * n_self full-precision tokens k_self/v_self [heads][n_self][head_dim]. The
 * logit of cached token j is (q . khat_j + (q . U_r^(e(j))) . coef_j) *
 * softmax_scale, khat = c_id + zp + code * step (fugumt.com abstract: PSAC puts
 * the Key error left after quantization back along the dominant Query
 * subspace so the logits stay stable); self logits
 * are q . k_self * softmax_scale. Softmax over all visible tokens, output the
 * probability-weighted sum of the dequantized / self Values into out
 * [heads][n_q][head_dim] float. 1 <= n_q <= max_query_tokens; k_self and
 * v_self may be NULL only with n_self == 0 and mask QWM_SELF_NONE. */
qwm_status qwm_attend(qwm_cache* cache, const void* q, int64_t n_q, const void* k_self,
                      const void* v_self, int64_t n_self, int32_t mask, float softmax_scale,
                      float* out);

/* qwm_attend for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments and result, but the call's scratch (the q . U_r table,
 * the q . C table of the decode path and the split-KV partials) lives in a
 * static device array of the library, 64 MiB on each device, instead of the
 * cache's arena. n_q is bounded by that array, not by max_query_tokens: the
 * tables need heads * epochs * n_q * 64 bytes (plus heads * epochs *
 * n_centroids * 16 * ceil(n_q / 16) * 4 on the decode path, n_q <= 48), and
 * a call whose tables do not fit returns QWM_ERR_CAPACITY before anything is
 * enqueued; the partials take what is left (fewer KV splits, down to none).
 * On the prefill path of a bf16 head_dim-128 cache an fp16 copy of the
 * epochs' centroid tables (heads * epochs * n_centroids * 256 bytes) comes
 * before the partials where it fits; without it the kernel converts the
 * rows it reads (same results).
 * It calls nothing that allocates (no hipMalloc, no hipEventCreate: kernel
 * timing is not recorded for it). Every call on one device shares the array,
 * which keeps the previous call's contents (a call writes every entry it
 * reads, so nothing needs clearing): calls that overlap on one device, from
 * any caches or streams, race. */
qwm_status qwm_attend_noalloc(qwm_cache* cache, const void* q, int64_t n_q, const void* k_self,
                              const void* v_self, int64_t n_self, int32_t mask, float softmax_scale, float* out);

qwm_status qwm_length(const qwm_cache* cache, int64_t* n_tokens);
qwm_status qwm_epochs(const qwm_cache* cache, int32_t* n_epochs);

/* Drop every token at position >= n_tokens and every epoch that starts after
 * n_tokens; the last remaining epoch becomes current. 0 <= n_tokens <= length. */
qwm_status qwm_truncate(qwm_cache* cache, int64_t n_tokens);

/* ---- calibration import/export and inspection (tests, diagnostics) ---- */

/* Stage a calibration given by the caller (C in the cache dtype, S_G and U_r
 * float, device pointers, layouts as above) and commit it as a new epoch.
 * S_G may be NULL with QWM_OBJ_NEAREST (stored as zeros), U_r at rank 0. */
qwm_status qwm_import_calibration(qwm_cache* cache, const void* C, const float* S_G, const float* U_r);

/* Copy epoch `epoch`'s calibration (or the staged one when epoch == -1) into
 * caller device buffers C, S_G, U_r (any may be NULL). */
qwm_status qwm_export_calibration(const qwm_cache* cache, int32_t epoch, void* C, float* S_G, float* U_r);

/* Bytes qwm_export writes for tokens [t0, t1): heads * (t1 - t0) *
 * (2 * head_dim / 4 + 8 * (head_dim / group) + 1 + 2 * rank + 2). */
qwm_status qwm_export_bytes(const qwm_cache* cache, int64_t t0, int64_t t1, size_t* bytes);

/* Write the records of tokens [t0, t1) into the device buffer `dev_buf` in
 * the canonical layout: for each head, the fields one after the other,
 *   K codes [n][head_dim/4] u8 (byte b holds channels 4b..4b+3, channel 4b+t
 *   in bits 2t..2t+1), V codes [n][head_dim/4] u8, K zp [n][G] fp16, K step
 *   [n][G] fp16, V zp, V step, centroid id [n] u8, PSAC coef [n][rank] fp16,
 *   epoch index [n] u16,
 * with n = t1 - t0 and G = head_dim / group. */
qwm_status qwm_export(const qwm_cache* cache, int64_t t0, int64_t t1, void* dev_buf);

/* Compensated, scaled logits of n_q Queries q [heads][n_q][head_dim] against
 * every cached token of one head: logits [n_q][length] float. They come from
 * the general attention kernel, whose Key operand is khat split into fp16 hi
 * and lo parts; qwm_attend on bf16 caches with head_dim 128 uses a kernel
 * with exact fp16 operands instead (centroid, code times step, zero-point
 * and PSAC terms). Both equal the definition up to the float32 rounding of
 * their sums. */
qwm_status qwm_attend_logits(qwm_cache* cache, const void* q, int64_t n_q, int32_t head,
                             float softmax_scale, float* logits);

/* Top-scoring token per Query (the article's attention analysis, roboind.com
 * "Table 1"): top1 [heads][n_q] int32 receives, for each head and Query of q
 * [heads][n_q][head_dim], the index of the token with the largest logit, the
 * smallest index among equal logits. Without k_ref (n_ref == 0) the tokens are
 * the cached ones and the logit is the compensated q . khat_j + (q . U_r) .
 * coef_j of qwm_attend (unscaled); with k_ref [heads][n_ref][head_dim] in the
 * cache dtype (1 <= n_ref <= 2^22) they are those full-precision Keys and the
 * logit is q . k_j. Both go through the general attention kernel (as
 * qwm_attend_logits), whose float32 logits decide the order. */
qwm_status qwm_attend_top1(qwm_cache* cache, const void* q, int64_t n_q, const void* k_ref, int64_t n_ref,
                           int32_t* top1);

/* ---- kernel timing (HIP events around each launch, on the stream it runs on) ---- */

typedef enum {
  QWM_K_QUANTIZE = 0,   /* quantize-append */
  QWM_K_ATTEND = 1,     /* attention main loop */
  QWM_K_MERGE = 2,      /* split-KV merge */
  QWM_K_QU = 3,         /* per-epoch q . U_r prologue */
  QWM_K_GRAM = 4,       /* Gram matrix + sensitivity */
  QWM_K_EIGEN = 5,      /* eigensolver (on the eigensolve stream) */
  QWM_K_ASSIGN = 6,     /* k-means assignment */
  QWM_K_UPDATE = 7,     /* k-means centroid update */
  QWM_K_OTHER = 8,      /* seeding, shadows, export */
  QWM_K_COUNT = 9
} qwm_kernel_id;

/* Enable (1) or disable (0) event timing; enabling clears the counters. */
qwm_status qwm_profile_enable(qwm_cache* cache, int32_t enable);
/* Total milliseconds and launch count of kernel class `kid` since enabling.
 * Synchronizes the cache stream. */
qwm_status qwm_profile_read(qwm_cache* cache, int32_t kid, double* total_ms, int64_t* launches);
/* Work of the centroid rule (QSAC assignment, roboind.com article, section
 * "Step 1") done by launches of class `kid` since profiling was enabled, as
 * channel evaluations: one is a (Key, centroid, channel) residual term
 * r = k - c with its share of the group's max, min or square. A full
 * assignment pass (QWM_K_QUANTIZE, and the first k-means iteration under
 * QWM_K_ASSIGN) makes heads x tokens x n_centroids x head_dim of them; the
 * pruned k-means assignment counts those its waves computed, so the figure
 * is the work done, not the brute-force bound. Other classes report 0.
 * Synchronizes the cache stream when a pruned launch has counted; fails with
 * QWM_ERR_INVALID_ARG on a NULL argument or a bad class. */
qwm_status qwm_profile_work(qwm_cache* cache, int32_t kid, double* evaluations);

const char* qwm_last_error(void);
const char* qwm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QWM_H_ */
