// Internal declarations shared by the host library and the kernel translation
// units of the QuantWM 2-bit KV cache (gfx950). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qwm {

constexpr int kGroup = 32;       // channels per INT2 group
constexpr int kRankPad = 16;     // PSAC rank padded for the MFMA contraction
constexpr int kTileKV = 64;      // tokens per attention tile
constexpr int kTileQ = 256;      // most Queries per attention workgroup (8 waves x 32)
constexpr int kAttnThreads = 512;
constexpr int kMaxEpochs = 64;
constexpr int kMaxSegments = kMaxEpochs + 1;  // epochs + the self segment
constexpr int kGramMaxChunks = 8;   // historical-Query chunks per head in the Gram
constexpr int kObjQsac = 0;         // centroid rule: QSAC objective
constexpr int kObjNearest = 1;      // centroid rule: nearest centroid (QVG)
constexpr int kObjPostq = 2;        // centroid rule: weighted error after INT2 quantization

// Per-head structure-of-arrays cache. Every per-head array holds capP token
// slots (capacity rounded up to a tile multiple) so tile loads never leave the
// head's rows.
struct CacheView {
  uint8_t* kcode;    // [H][capP][D/4]   canonical 2-bit packing
  uint8_t* vcode;    // [H][capP][D/4]
  uint32_t* kparam;  // [H][capP][nG]    zp fp16 bits | step fp16 bits << 16
  uint32_t* vparam;  // [H][capP][nG]
  uint8_t* ids;      // [H][capP]
  uint16_t* coef;    // [H][capP][r]     fp16 bits
  int64_t capP;
};

// Calibration of one epoch slot.
struct EpochView {
  const void* C;       // [H][m][D] cache dtype
  const float* S;      // [H][nG]
  const float* U;      // [H][D][r]
};

// ---------------------------------------------------------------- quantize
struct QuantArgs {
  const void* k;           // [H][n][D]
  const void* v;           // [H][n][D] (nullptr: assignment only, for k-means)
  int64_t n;               // tokens per head in this call
  const float* C32;        // [H][m][D] float copy of the current centroid table
  const float* S;          // [H][nG]
  const double* U64;       // [H][D][r] float64 copy of U_r (nullptr: no PSAC)
  CacheView cache;         // destination (ignored when v == nullptr)
  int64_t pos0;            // first destination slot
  uint8_t* ids_out;        // assignment-only output [H][n] (k-means)
  int H, m, r;
  int obj;                 // kObjQsac, kObjNearest or kObjPostq
  uint2* part;             // not null: split centroid scan, [2][H][n] best (J bits, id) per half
                           // (used by the assignment-only passes of the k-means)
};
// Split scans need n <= kQuantSplitMaxTokens (the size of their buffer).
constexpr int64_t kQuantSplitMaxTokens = 4096;
constexpr int kQuantBlocksPerCU = 3;  // resident 4-wave quantize workgroups per CU (166 VGPRs)
hipError_t launch_quantize(int D, int dtype, const QuantArgs& a, hipStream_t s);

// ---------------------------------------------------------------- k-means
hipError_t launch_kmeans_seed(int D, int dtype, const void* keys, int64_t n, int H, int m,
                              void* C, float* C32, hipStream_t s);
hipError_t launch_kmeans_update(int D, int dtype, const void* keys, const uint8_t* ids, int64_t n,
                                int H, int m, void* C, float* C32, hipStream_t s);
// Pruned assignment for k-means iterations after the first: tokens grouped
// by their previous id (perm [H][n], off/woff [H][257]), then the assignment
// skipping candidates that provably lose.
hipError_t launch_kmeans_bucket(const uint8_t* ids, int64_t n, int H, int m, int32_t* perm, int32_t* off,
                                int32_t* woff, hipStream_t s);
// With `work` not null, the pruned assignment adds to *work the channel
// evaluations it made: for every wave, the Keys it holds times 32 times the
// group terms it computed (the cost of the previous centroid included).
// ccd[h][b][c] = sqrt of the rule's cost between centroids b and c (the
// pruned assignment's bound), every pair of every head
hipError_t launch_kmeans_ccd(int D, int obj, int H, int m, const float* C32, const float* S, float* ccd,
                             hipStream_t s);
hipError_t launch_kmeans_assign_pruned(int D, int dtype, int obj, const void* keys, int64_t n, int H, int m,
                                       const float* C32, const float* S, const int32_t* perm, const int32_t* off,
                                       const int32_t* woff, const float* ccd, uint8_t* ids_out,
                                       unsigned long long* work, hipStream_t s);
// p[0 .. n) = v
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s);
// Copy a staged calibration (C, S, U) into an epoch slot and write its shadows.
hipError_t launch_commit(int D, int dtype, const void* Cs, const float* Ss, const float* Us, void* Cd, float* Sd,
                         float* Ud, int H, int m, int r, float* C32, double* U64, hipStream_t s);
// Float (and float64 U) shadows of a committed epoch, used by quantize.
hipError_t launch_shadow(int D, int dtype, const void* C, const float* U, int H, int m, int r,
                         float* C32, double* U64, hipStream_t s);

// ---------------------------------------------------------------- calibration
// Partial Grams [H][chunks][D][D] (chunks = gram_chunks(n) <= kGramMaxChunks).
int gram_chunks(int64_t n);
hipError_t launch_gram(int D, int dtype, const void* q, int64_t n, int H, double* gram, hipStream_t s);
// Per-chunk partials of the Gram diagonal [H][chunks][D] (the same chunks).
hipError_t launch_diag(int D, int dtype, const void* q, int64_t n, int H, double* diag, hipStream_t s);
// S_G [H][D/32] from the diagonal partials (added in chunk order).
hipError_t launch_sens(int D, const double* diag, int nchunk, int64_t n_hist, int H, float* S, hipStream_t s);
// Eigensolve of each head's Gram (sum of the chunk partials) -> U_r [H][D][r].
hipError_t launch_eigen(int D, const double* gram, int nchunk, int H, int r, float* U, hipStream_t s);

// ---------------------------------------------------------------- attention
struct AttnPlan {
  int n_seg;
  int32_t seg_start[kMaxSegments];   // first token of the segment (self: index into self K/V)
  int32_t seg_len[kMaxSegments];
  int32_t seg_epoch[kMaxSegments];   // epoch slot, or -1 for the self segment
  int32_t tile_prefix[kMaxSegments + 1];
};

struct AttnArgs {
  const void* q;          // [H][nq][D]
  const float* qU;        // [H][E][nq][16] float (q . U_r per epoch slot, zero padded)
  const void* kself;      // [H][nself][D]
  const void* vself;
  int64_t nq, nself;
  int causal_self;
  float scale_log2;       // softmax_scale * log2(e)
  float scale;            // softmax_scale
  CacheView cache;
  const void* Cbase;      // epoch slot 0 centroid table; slot e at + e * epoch_C_stride bytes
  int64_t epoch_C_stride; // bytes
  void* C16;              // bf16 head_dim-128 prefill: room for an fp16 copy of slots 0..n_epoch_slots-1
                          // (same layout), or null: the tiles then convert the bf16 rows
  int n_epoch_slots;      // E of qU
  int H, m, r;
  int splits;
  int qpb;                // Queries per workgroup: a multiple of 32, at most kTileQ
  float* out;             // [H][nq][D] (splits == 1)
  float* part_o;          // [splits][H][nq][D]
  float* part_ml;         // [splits][H][nq][2]
  float* logits;          // logits mode: [nq][len] of head `logit_head`
  int32_t* top1;          // top-1 mode: [H][nq] token index of the largest logit
  int logit_head;
  int64_t logit_len;
};
hipError_t launch_qu(int D, int dtype, const void* q, int64_t nq, int H, int r, const float* Ubase,
                     int64_t epoch_U_stride_floats, int E, float* qU, hipStream_t s);
hipError_t launch_attend(int D, int dtype, const AttnArgs& a, const AttnPlan& p, hipStream_t s);
// bf16, head_dim 128: the exact-operand pipelined kernel (kern_attend_bf16.hip)
hipError_t launch_attend_bf16(const AttnArgs& a, const AttnPlan& p, hipStream_t s);
hipError_t launch_attend_logits(int D, int dtype, const AttnArgs& a, const AttnPlan& p, hipStream_t s);
hipError_t launch_merge(int D, const AttnArgs& a, hipStream_t s);
// Top-1 mode: per (head, Query) the token with the largest unscaled logit
// (first on a tie); with splits > 1 the partials go to part_ml and
// launch_top1_merge combines them.
hipError_t launch_attend_top1(int D, int dtype, const AttnArgs& a, const AttnPlan& p, hipStream_t s);
hipError_t launch_top1_merge(const AttnArgs& a, hipStream_t s);

// ---------------------------------------------------------------- decode
// Few Queries per head (bf16, head_dim 128, no self segment): the Key side
// runs on the 2-bit codes with a q . C table; one wave per workgroup.
struct DecodeArgs {
  const void* q;      // [H][nq][128] bf16
  const float* qc;    // [H][E][m][nqp] float: q . C_c of every epoch
  const float* qU;    // [H][E][nq][16] float
  CacheView cache;
  int64_t nq;
  int nqp;            // row length of qc (multiple of 16, >= nq)
  int H, m, r, E;
  float scale_log2;   // softmax_scale * log2(e)
  int splits;
  float* out;         // [H][nq][128] (splits == 1)
  float* part_o;      // [splits][H][nq][128]
  float* part_ml;     // [splits][H][nq][2]
};
// sign: the sign of the softmax scale, carried by the table
hipError_t launch_qc(const void* q, int64_t nq, int nqp, const void* Cbase, int64_t epoch_C_stride, int H, int m,
                     int E, float sign, float* qc, hipStream_t s);
constexpr int kDecodeQ = 16;        // Queries per decode workgroup
// largest n_q served by the decode kernel: each 16-Query block streams the
// cache on its own, so from the fourth block on the prefill kernel (which
// stages every tile once per workgroup) is the faster one
constexpr int kDecodeMaxQ = 48;
constexpr int kDecodeWavesPerCU = 8;  // resident decode workgroups per CU (2 waves per SIMD)
hipError_t launch_decode(const DecodeArgs& a, const AttnPlan& p, hipStream_t s);

// ---------------------------------------------------------------- export
struct ExportArgs {
  CacheView cache;
  int64_t t0, n;
  const int32_t* epoch_of_token;  // not used; epochs passed as ranges below
  int n_epochs;
  int32_t epoch_start[kMaxEpochs + 1];
  int H, D, nG, r;
  uint8_t* out;
};
hipError_t launch_export(const ExportArgs& a, hipStream_t s);

}  // namespace qwm
