// Attention over the 2-bit QuantWM cache with PSAC logit compensation (gfx950):
// the general kernel (float32 caches, head_dim 64, and the logits and top-1
// modes); bf16 caches with head_dim 128 attend through kern_attend_bf16.hip.
//
// Method (QuantWM; fugumt.com abstract: PSAC puts the Key error left after
// quantization back along the dominant Query subspace so the attention logits
// stay stable; roboind.com "Step 2"): for cached token j of epoch e(j)
//   l_ij = (q_i . khat_j + (q_i U_r^(e(j))) . coef_j) * scale,
//   khat_j = c_id(j) + zp + code * step   (per 32-channel group),
// plus optional full-precision self tokens of the attending chunk; softmax
// over all visible tokens and o_i = sum_j p_ij vhat_j.
//
// Mapping to CDNA4:
//  * one workgroup = 8 waves = up to 256 Queries of one head (the Queries
//    spread evenly over the workgroups in 32-Query waves), one split of the KV
//    sequence; the KV sequence is walked in 64-token tiles that never cross an
//    epoch boundary or the cache/self boundary;
//  * each tile is dequantized ONCE per workgroup into one of two LDS stages
//    (every thread: one 16-channel half group of one token's khat and vhat):
//    khat as float16 hi + lo pairs
//    (hi = fp16(x), lo = fp16(x - hi), 22 significant bits) with the r PSAC
//    coefficients next to them, vhat^T as hi + lo; the packed words of the
//    next tile are loaded into registers before the current tile's MFMA work;
//  * logits come from v_mfma_f32_16x16x32_f16 with the contraction dimension
//    [khat_hi | khat_lo | coef] x [q | q | qU_hi, qU_lo]: one MFMA chain per
//    16x16 block computes q.khat and the PSAC term together;
//  * online softmax in float32 with cross-lane max over the 4 lane groups
//    that share a Query, P in fp16, o += vhat^T P^T by MFMA with vhat hi and
//    lo, row sums of the same fp16 P by v_dot2_f32_f16.
// The hi/lo splits keep logits within ~1e-6 and outputs within ~5e-4 (row
// max relative) of float64.
#include "qwm_dev.h"
#include "qwm_internal.h"

namespace qwm {

namespace {

template <int D>
struct AttnShape {
  static constexpr int KS = D / 32;             // 32-channel contraction steps
  static constexpr int KROW = 2 * D + 16 + 8;   // halfs per khat row: hi | lo | coef[16] | pad
  static constexpr int VROW = kTileKV + 8;      // halfs per vhat^T row
  static constexpr int NG = D / kGroup;
  static constexpr int KITEMS = kTileKV * NG * 2;         // (token, 16-channel half group) items
  static constexpr int VITEMS = kTileKV * NG * 2;         // (token, 16-channel half group) items
  static constexpr int KST = kTileKV * KROW;              // halfs of one khat stage
  static constexpr int VST = D * VROW;                    // halfs of one vhat^T (hi or lo) stage
};

__device__ __forceinline__ floatx4 mfma16(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// Two floats -> two fp16 (round to nearest even), one v_cvt_pk_f16_f32.
__device__ __forceinline__ half2v pk_f16(float x, float y) { return __builtin_convertvector(float2v{x, y}, half2v); }

// x -> hi = fp16(x), lo = fp16(x - hi) for a pair of floats: hi + lo carries
// 22 significant bits of x.
__device__ __forceinline__ void split2(float x0, float x1, half2v& hi, half2v& lo) {
  hi = pk_f16(x0, x1);
  lo = pk_f16(x0 - (float)hi[0], x1 - (float)hi[1]);
}

template <int DT, int N>
__device__ __forceinline__ void load_span(const void* base, int64_t off, float (&x)[N]) {
  if constexpr (DT == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const uint4 w = p[i];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[8 * i + 2 * k] = __uint_as_float(ww[k] << 16);
        x[8 * i + 2 * k + 1] = __uint_as_float(ww[k] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const float4 w = p[i];
      x[4 * i] = w.x;
      x[4 * i + 1] = w.y;
      x[4 * i + 2] = w.z;
      x[4 * i + 3] = w.w;
    }
  }
}

// Value c (0..7) of an 8-value span of raw words: bf16 pairs in one uint4,
// or float32 in two.
template <int DT>
__device__ __forceinline__ float span_elem(const uint4* w, int c) {
  if constexpr (DT == 0) {
    const uint4 v = w[0];
    const uint32_t ww = (c >> 1) == 0 ? v.x : (c >> 1) == 1 ? v.y : (c >> 1) == 2 ? v.z : v.w;
    return __uint_as_float((c & 1) ? (ww & 0xFFFF0000u) : (ww << 16));
  } else {
    const uint4 v = w[c >> 2];
    const int k = c & 3;
    return __uint_as_float(k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w);
  }
}

struct TileInfo {
  int ep;      // epoch slot, -1 for the self segment
  int tstart;  // first token (cache position, or index into the self K/V)
  int tcount;  // tokens in the tile (<= 64)
};

__device__ __forceinline__ TileInfo tile_info(const AttnPlan& p, int tile) {
  int sg = 0;
  while (p.tile_prefix[sg + 1] <= tile) ++sg;
  TileInfo ti;
  ti.ep = p.seg_epoch[sg];
  ti.tstart = p.seg_start[sg] + (tile - p.tile_prefix[sg]) * kTileKV;
  const int tend = p.seg_start[sg] + p.seg_len[sg];
  ti.tcount = (tend - ti.tstart) < kTileKV ? (tend - ti.tstart) : kTileKV;
  return ti;
}

// Attention workgroup: 8 waves = up to 256 Queries of one head over the tiles
// [tlo, thi) of one split. Two LDS stages: while the waves run the MFMA and
// softmax work of tile i from one stage, the packed words of tile i+1 are
// already in registers (loaded before that work) and are dequantized into the
// other stage after it, so global latency hides behind the MFMA chains and
// one barrier per tile suffices. Every thread builds the khat and the vhat^T
// entries of one token (its lane) and one 16-channel half group (its wave).
// MODE: kModeAttend (softmax and P.V), kModeLogits (write one head's scaled
// logits), kModeTop1 (per Query the index of the largest unscaled logit).
constexpr int kModeAttend = 0, kModeLogits = 1, kModeTop1 = 2;

template <int D, int DT, int MODE>
__global__ __launch_bounds__(kAttnThreads) void attend_kernel(const AttnArgs a, const AttnPlan p) {
  constexpr bool LOGITS = (MODE == kModeLogits), TOP1 = (MODE == kModeTop1), NOV = (MODE != kModeAttend);
  using Sh = AttnShape<D>;
  constexpr int KS = Sh::KS, KROW = Sh::KROW, VROW = Sh::VROW, NG = Sh::NG;
  constexpr bool QLO = (DT == 1);  // float32 Queries also carry a lo part
  constexpr int KST = Sh::KST, VST = NOV ? 0 : Sh::VST;
  constexpr int KITEMS = Sh::KITEMS, VITEMS = Sh::VITEMS;
  static_assert(KITEMS <= kAttnThreads && VITEMS <= kAttnThreads, "dequant items must fit one pass");
  // Raw words one thread holds for the next tile: khat values (16 cache-dtype
  // values), khat code/param word, 8 coefficients, vhat code/param word and
  // 16 self Values of one token.
  constexpr int NK = (DT == 0) ? 2 : 4;  // uint4 words of 16 input values
  constexpr int RK = 0, RKW = NK, RCF = NK + 1, RVC = NK + 2, RVS = NK + 3;
  constexpr int NR = RVS + NK;
  __shared__ __attribute__((aligned(16))) _Float16 lds[2 * (KST + 2 * VST) + 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int h = LOGITS ? a.logit_head : (int)blockIdx.z;
  const int split = blockIdx.y;
  const int64_t qw0 = (int64_t)blockIdx.x * a.qpb + wave * 32;
  // waves past the workgroup's Queries, or whose 32 Queries are all padding,
  // skip the math (they still stage tiles)
  const bool wave_live = wave * 32 < a.qpb && qw0 < a.nq;
  // wave-uniform producer roles (items are whole waves)
  // (always true at head_dim 128, where every thread holds one khat and one
  // vhat item; at 64 only waves 0-3 do)
  const bool is_k = KITEMS >= kAttnThreads || wave < KITEMS / 64;
  const bool is_v = !NOV && (VITEMS >= kAttnThreads || wave < VITEMS / 64);
  // softmax in the log2 domain with a positive factor; a negative scale is
  // carried by negated Queries (exact in fp16)
  const float qsign = (!NOV && a.scale_log2 < 0.0f) ? -1.0f : 1.0f;
  const float cl2 = a.scale_log2 * qsign;

  const int T = p.tile_prefix[p.n_seg];
  const int tlo = (int)(((int64_t)T * split) / a.splits);
  const int thi = (int)(((int64_t)T * (split + 1)) / a.splits);

  // producer items: khat and vhat of token kt, channels 16*kq .. 16*kq+15
  // (group kq/2)
  const int kt = lane, kq = wave;

  uint4 raw[NR];
  int id_next = 0;

  // Per-head bases (wave-uniform, scalar registers) and 32-bit per-thread
  // offsets: every per-head region is below 4 GiB (capacity <= 2^26 tokens).
  constexpr int ESZ = (DT == 0) ? 2 : 4;
  const uint8_t* kcode_h = a.cache.kcode + (size_t)h * a.cache.capP * (D / 4);
  const uint8_t* vcode_h = a.cache.vcode + (size_t)h * a.cache.capP * (D / 4);
  const uint32_t* kparam_h = a.cache.kparam + (size_t)h * a.cache.capP * NG;
  const uint32_t* vparam_h = a.cache.vparam + (size_t)h * a.cache.capP * NG;
  const uint8_t* ids_h = a.cache.ids + (size_t)h * a.cache.capP;
  const uint16_t* coef_h = a.cache.coef + (size_t)h * a.cache.capP * a.r;
  const char* kself_h = reinterpret_cast<const char*>(a.kself) + (size_t)h * a.nself * D * ESZ;
  const char* vself_h = reinterpret_cast<const char*>(a.vself) + (size_t)h * a.nself * D * ESZ;
  const char* C_h = reinterpret_cast<const char*>(a.Cbase) + (size_t)h * a.m * D * ESZ;

  // Token indices are clamped into the tile (tcount >= 1), so every load is
  // unconditional and lands straight in its register: a register that is
  // the target of a load still in flight must not be written on another path,
  // or the wait for it would also wait for the whole prefetch. Rows past
  // tcount hold a copy of the last token: finite values whose logits the
  // softmax masks to -inf, so they get p = 0 and add nothing.
  auto load_id = [&](const TileInfo& ti) -> int {
    const int t = kt < ti.tcount ? kt : ti.tcount - 1;
    return ids_h[ti.ep >= 0 ? (uint32_t)(ti.tstart + t) : 0u];  // self tiles: a valid dummy
  };
  // Issue the global loads of one tile's packed words (no use of the data).
  // Every load is issued on every tile; the ones a tile does not need read a
  // valid dummy address (the head's first cache slot), so no register is
  // written on one path and left alone on another.
  auto load_raw = [&](const TileInfo& ti, int id) {
    const bool cache = ti.ep >= 0;  // wave-uniform
    if (is_k) {
      const uint32_t slot = (uint32_t)(ti.tstart + (kt < ti.tcount ? kt : ti.tcount - 1));
      const uint32_t cs = cache ? slot : 0u;
      const char* Ce = C_h + (size_t)(cache ? ti.ep : 0) * a.epoch_C_stride;  // uniform
      const uint4* src = cache ? reinterpret_cast<const uint4*>(Ce + ((uint32_t)id * D + 16 * kq) * ESZ)
                               : reinterpret_cast<const uint4*>(kself_h + (slot * D + 16 * kq) * ESZ);
#pragma unroll
      for (int i = 0; i < NK; ++i) raw[RK + i] = src[i];
      raw[RKW].x = *reinterpret_cast<const uint32_t*>(kcode_h + cs * (D / 4) + 4 * kq);
      raw[RKW].y = kparam_h[cs * NG + (kq >> 1)];
      // coefficients 8*kq .. 8*kq+7 of the token (halves past r are zeroed at
      // store); r even: four dword loads, r odd: halves one by one
      const uint16_t* cf = coef_h + cs * (uint32_t)a.r + (kq < 2 ? 8 * kq : 0);
      if ((a.r & 1) == 0) {
        const uint32_t* cw = reinterpret_cast<const uint32_t*>(cf);
        raw[RCF] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
      } else {
        uint32_t cc[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const int j = (kq < 2 ? 8 * kq : 0) + 2 * s2;
          const uint32_t lo = (j < a.r) ? cf[2 * s2] : 0u;
          const uint32_t hi = (j + 1 < a.r) ? cf[2 * s2 + 1] : 0u;
          cc[s2] = lo | (hi << 16);
        }
        raw[RCF] = make_uint4(cc[0], cc[1], cc[2], cc[3]);
      }
    }
    if (is_v) {
      const uint32_t slot = (uint32_t)(ti.tstart + (kt < ti.tcount ? kt : ti.tcount - 1));
      const uint32_t cs = cache ? slot : 0u;
      raw[RVC].x = *reinterpret_cast<const uint32_t*>(vcode_h + cs * (D / 4) + 4 * kq);
      raw[RVC].y = vparam_h[cs * NG + (kq >> 1)];
      const uint4* src = cache ? reinterpret_cast<const uint4*>(vcode_h)
                               : reinterpret_cast<const uint4*>(vself_h + (slot * D + 16 * kq) * ESZ);
#pragma unroll
      for (int i = 0; i < NK; ++i) raw[RVS + i] = src[i];
    }
  };
  auto store_coef = [&](const TileInfo& ti, int st) {
    if (kq < 2) {
      _Float16* row = lds + st * (KST + 2 * VST) + kt * KROW;
      uint4 cfw = raw[RCF];
      const int j0 = 8 * kq;  // halves j0 .. j0+7; keep those below r
      const bool use = ti.ep >= 0;
      cfw.x = (use && j0 + 0 < a.r) ? (j0 + 1 < a.r ? cfw.x : cfw.x & 0xFFFFu) : 0u;
      cfw.y = (use && j0 + 2 < a.r) ? (j0 + 3 < a.r ? cfw.y : cfw.y & 0xFFFFu) : 0u;
      cfw.z = (use && j0 + 4 < a.r) ? (j0 + 5 < a.r ? cfw.z : cfw.z & 0xFFFFu) : 0u;
      cfw.w = (use && j0 + 6 < a.r) ? (j0 + 7 < a.r ? cfw.w : cfw.w & 0xFFFFu) : 0u;
      *reinterpret_cast<uint4*>(row + 2 * D + 8 * kq) = cfw;
    }
  };
  // Dequantize the loaded words into LDS stage `st`, in 16 pieces: part 0
  // and 1 are khat channels 16*kq .. +7 and +8 .. +15, parts 2 and 3 the same
  // halves of vhat; piece pc of a part is its channels 2pc and 2pc+1. Pieces
  // are branch-free (self tiles take zero step and zero point for khat and
  // select the raw Values for vhat), so the caller can spread them between
  // MFMAs; khat halves are stored with the part's last piece. The
  // coefficients (waves 0 and 1) are stored by store_coef. All parts write
  // disjoint LDS words.
  struct DequantPieces {
    half8 h8, l8;
  };
  auto dequant_piece = [&](const TileInfo& ti, int st, int part, int pc, DequantPieces& dq) {
    _Float16* Ks = lds + st * (KST + 2 * VST);
    const bool cache = ti.ep >= 0;
    const int c = 2 * pc;
    if (part < 2) {
      if (!is_k) return;
      const int u = part;
      const uint32_t kp = cache ? raw[RKW].y : 0u;  // self: k + (code*0 + 0) = k
      const float zpf = half_bits_to_float(kp & 0xFFFFu), scf = half_bits_to_float(kp >> 16);
      const uint32_t w = raw[RKW].x;
      float x0 = span_elem<DT>(raw + RK + u * (NK / 2), c);
      float x1 = span_elem<DT>(raw + RK + u * (NK / 2), c + 1);
      x0 = x0 + __builtin_fmaf((float)((w >> (16 * u + 2 * c)) & 3u), scf, zpf);
      x1 = x1 + __builtin_fmaf((float)((w >> (16 * u + 2 * c + 2)) & 3u), scf, zpf);
      half2v hi, lo;
      split2(x0, x1, hi, lo);
      dq.h8[c] = hi[0];
      dq.h8[c + 1] = hi[1];
      dq.l8[c] = lo[0];
      dq.l8[c + 1] = lo[1];
      if (pc == 3) {
        _Float16* row = Ks + kt * KROW;
        *reinterpret_cast<half8*>(row + 16 * kq + 8 * u) = dq.h8;
        *reinterpret_cast<half8*>(row + D + 16 * kq + 8 * u) = dq.l8;
      }
    } else if constexpr (!NOV) {
      if (!is_v) return;
      const int u = part - 2;
      _Float16* Vh = Ks + KST;
      _Float16* Vl = Vh + VST;
      // token j of the tile goes to column 32*(j/32) + 8*gg + 4*b + u of
      // the vhat^T rows (b = bit 4, gg = bits 2-3, u = bits 0-1 of j): the
      // order in which the P fragment of lane group gg holds tokens
      // {4gg..4gg+3, 16+4gg..16+4gg+3} of each 32-token step
      const int col = (kt & ~31) + 8 * ((kt >> 2) & 3) + 4 * ((kt >> 4) & 1) + (kt & 3);
      const float zpf = half_bits_to_float(raw[RVC].y & 0xFFFFu), scf = half_bits_to_float(raw[RVC].y >> 16);
      const uint32_t w = raw[RVC].x;
      const uint32_t msel = cache ? 0xFFFFFFFFu : 0u;
      float x[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float xc = __builtin_fmaf((float)((w >> (16 * u + 2 * (c + e))) & 3u), scf, zpf);
        const float xs = span_elem<DT>(raw + RVS + u * (NK / 2), c + e);
        x[e] = __uint_as_float((__float_as_uint(xc) & msel) | (__float_as_uint(xs) & ~msel));
      }
      half2v hi, lo;
      split2(x[0], x[1], hi, lo);
      const int row = 16 * kq + 8 * u + c;
      Vh[row * VROW + col] = hi[0];
      Vh[(row + 1) * VROW + col] = hi[1];
      Vl[row * VROW + col] = lo[0];
      Vl[(row + 1) * VROW + col] = lo[1];
    }
  };
  auto store_part = [&](const TileInfo& ti, int st, int part) {
    DequantPieces dq;
#pragma unroll
    for (int pc = 0; pc < 4; ++pc) dequant_piece(ti, st, part, pc, dq);
  };
  auto store_stage = [&](const TileInfo& ti, int st) {
#pragma unroll
    for (int part = 0; part < 4; ++part) store_part(ti, st, part);
    store_coef(ti, st);
  };

  // Query fragments (B operand): Query qw0 + 16*qb + l16, channels 32*ks + 8*g .. +7.
  half8 qh[2][KS];
  half8 ql[2][QLO ? KS : 1];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t qi = qw0 + 16 * qb + l16;
    const bool qv = qi < a.nq;
    const int64_t base = ((int64_t)h * a.nq + (qv ? qi : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
      load_span<DT, 8>(a.q, base + 32 * ks + 8 * g, x);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const float x0 = qv ? qsign * x[2 * s2] : 0.0f, x1 = qv ? qsign * x[2 * s2 + 1] : 0.0f;
        half2v hi, lo;
        split2(x0, x1, hi, lo);
        qh[qb][ks][2 * s2] = hi[0];
        qh[qb][ks][2 * s2 + 1] = hi[1];
        if constexpr (QLO) {
          ql[qb][ks][2 * s2] = lo[0];
          ql[qb][ks][2 * s2 + 1] = lo[1];
        }
      }
    }
  }
  half8 qu[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) qu[qb][s2] = (_Float16)0.0f;
  int cur_epoch = -2;

  floatx4 O[2][NOV ? 1 : D / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int cb = 0; cb < (NOV ? 1 : D / 16); ++cb) O[qb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  // top-1 mode: this lane's best logit and its token index per Query block
  float bval[2] = {-__builtin_inff(), -__builtin_inff()};
  int bidx[2] = {0x7fffffff, 0x7fffffff};
  // per lane: this lane's share of the row sum of the fp16 P (the values the
  // PV product uses), float32
  float lrow[2] = {0.0f, 0.0f};
  float mrow[2] = {-__builtin_inff(), -__builtin_inff()};
  const half2v one2 = {(_Float16)1.0f, (_Float16)1.0f};

  // Every wave loads the packed words of tile i+1, runs the MFMA and softmax
  // work of tile i, then writes tile i+1 to the other LDS stage. (Running
  // half of the waves in the opposite order, to overlap one wave's MFMA
  // chains with the other's dequantization, measured slower.)
  if (tlo < thi) {
    const TileInfo t0 = tile_info(p, tlo);
    load_raw(t0, load_id(t0));
    store_stage(t0, 0);
    if (tlo + 1 < thi) id_next = load_id(tile_info(p, tlo + 1));
  }
  __syncthreads();

  for (int tile = tlo; tile < thi; ++tile) {
    const int st = (tile - tlo) & 1;
    const TileInfo ti = tile_info(p, tile);
    TileInfo tn{};
    if (tile + 1 < thi) tn = tile_info(p, tile + 1);
    if (tile + 1 < thi) {
      load_raw(tn, id_next);
      if (tile + 2 < thi) id_next = load_id(tile_info(p, tile + 2));
    }

    if (wave_live) {
      const _Float16* Ks = lds + st * (KST + 2 * VST);
      const int ep = ti.ep;
      // ---- per-epoch PSAC Query fragment: lanes g<2 hold qU_hi, g>=2 qU_lo
      if (ep != cur_epoch) {
        cur_epoch = ep;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int64_t qi = qw0 + 16 * qb + l16;
          if (ep >= 0 && qi < a.nq && a.r > 0) {
            const float* src =
                a.qU + (((int64_t)h * a.n_epoch_slots + ep) * a.nq + qi) * kRankPad + 8 * (g & 1);
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
              half2v hi, lo;
              split2(qsign * src[2 * s2], qsign * src[2 * s2 + 1], hi, lo);
              qu[qb][2 * s2] = (g < 2) ? hi[0] : lo[0];
              qu[qb][2 * s2 + 1] = (g < 2) ? hi[1] : lo[1];
            }
          } else {
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) qu[qb][s2] = (_Float16)0.0f;
          }
        }
      }

      // ---- logits: S^T blocks [16 tokens x 16 Queries]
      floatx4 S[2][4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) S[qb][tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // keep the scheduler from hoisting every operand read of the loop
        // (register pressure): one 32-channel step at a time
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const _Float16* r0 = Ks + (16 * tb + l16) * KROW + 32 * ks + 8 * g;
          const half8 ahi = *reinterpret_cast<const half8*>(r0);
          const half8 alo = *reinterpret_cast<const half8*>(r0 + D);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            S[qb][tb] = mfma16(ahi, qh[qb][ks], S[qb][tb]);
            S[qb][tb] = mfma16(alo, qh[qb][ks], S[qb][tb]);
            if constexpr (QLO) S[qb][tb] = mfma16(ahi, ql[qb][ks], S[qb][tb]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const half8 ac = *reinterpret_cast<const half8*>(Ks + (16 * tb + l16) * KROW + 2 * D + 8 * (g & 1));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) S[qb][tb] = mfma16(ac, qu[qb], S[qb][tb]);
      }

      if constexpr (LOGITS) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int64_t qi = qw0 + 16 * qb + l16;
          if (qi < a.nq) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int j = 16 * tb + 4 * g + v;
                if (j < ti.tcount) a.logits[qi * a.logit_len + ti.tstart + j] = S[qb][tb][v] * a.scale;
              }
          }
        }
      } else if constexpr (TOP1) {
        // this lane's tokens of the tile in ascending order: a strict compare
        // keeps the first of equal logits
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int j = 16 * tb + 4 * g + v;
              if (j < ti.tcount && S[qb][tb][v] > bval[qb]) {
                bval[qb] = S[qb][tb][v];
                bidx[qb] = ti.tstart + j;
              }
            }
      } else {
        // ---- online softmax (log2 domain). The running max is only raised
        // when a row's new max exceeds it by more than 8 (p <= 2^8 stays exact
        // enough in fp16 and float32), so the output rescale is rare.
        const bool full = (ti.tcount == kTileKV) && !(ep < 0 && a.causal_self);
        half8 pf[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int64_t qi = qw0 + 16 * qb + l16;
          if (!full) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int j = 16 * tb + 4 * g + v;
                bool ok = j < ti.tcount;
                if (ep < 0 && a.causal_self) ok = ok && ((int64_t)(ti.tstart + j) <= qi);
                if (!ok) S[qb][tb][v] = -__builtin_inff();
              }
          }
          float mx = -__builtin_inff();
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v) mx = fmaxf(mx, S[qb][tb][v]);
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          mx *= cl2;
          const bool raise = mx > mrow[qb] + 8.0f;
          if (__ballot(raise)) {  // wave-uniform: rescale every lane (alpha = 1 where unchanged)
            const float mnew = raise ? mx : mrow[qb];
            const float alpha = (mrow[qb] == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(mrow[qb] - mnew);
            mrow[qb] = mnew;
            lrow[qb] *= alpha;
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb) O[qb][cb] *= alpha;
          }
          // mrow is finite as soon as any logit of the row is: a row still at
          // -inf has only masked (-inf) logits, and exp2(-inf * c + 0) = 0
          const float nm = (mrow[qb] == -__builtin_inff()) ? 0.0f : -mrow[qb];
          float pv[4][4];
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v) pv[tb][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][tb][v], cl2, nm));
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const half2v p0 = pk_f16(pv[2 * ks][0], pv[2 * ks][1]), p1 = pk_f16(pv[2 * ks][2], pv[2 * ks][3]);
            const half2v p2 = pk_f16(pv[2 * ks + 1][0], pv[2 * ks + 1][1]);
            const half2v p3 = pk_f16(pv[2 * ks + 1][2], pv[2 * ks + 1][3]);
            pf[qb][ks] = half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
            // exact fp16 values summed in float32: v_dot2_f32_f16 with (1, 1)
            float l = lrow[qb];
            l = __builtin_amdgcn_fdot2(p0, one2, l, false);
            l = __builtin_amdgcn_fdot2(p1, one2, l, false);
            l = __builtin_amdgcn_fdot2(p2, one2, l, false);
            l = __builtin_amdgcn_fdot2(p3, one2, l, false);
            lrow[qb] = l;
          }
        }
        // ---- o^T += vhat^T P^T, with the next tile's dequantization spread
        // between the MFMAs: independent VALU work the wave issues while its
        // MFMAs run (it writes the other LDS stage). After the last tile this
        // stages stale words into the unused stage: harmless, and it keeps
        // the code branch-free.
        const _Float16* Vh = Ks + KST;
        const _Float16* Vl = Vh + VST;
        if constexpr (D == 128) {
          // 16 steps of (ks, cb); step i also runs piece i % 4 of dequant
          // part i / 4. The next step's operands are read before the piece.
          constexpr int NSTEP = 2 * (D / 16);
          half8 ah = *reinterpret_cast<const half8*>(Vh + l16 * VROW + 8 * g);
          half8 al = *reinterpret_cast<const half8*>(Vl + l16 * VROW + 8 * g);
          DequantPieces dq;
#pragma unroll
          for (int i = 0; i < NSTEP; ++i) {
            const int ks = i / (D / 16), cb = i % (D / 16);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) O[qb][cb] = mfma16(ah, pf[qb][ks], O[qb][cb]);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) O[qb][cb] = mfma16(al, pf[qb][ks], O[qb][cb]);
            if (i + 1 < NSTEP) {
              const int ks1 = (i + 1) / (D / 16), cb1 = (i + 1) % (D / 16);
              const int off = (16 * cb1 + l16) * VROW + 32 * ks1 + 8 * g;
              ah = *reinterpret_cast<const half8*>(Vh + off);
              al = *reinterpret_cast<const half8*>(Vl + off);
            }
            __builtin_amdgcn_sched_barrier(0);
            dequant_piece(tn, st ^ 1, i / 4, i % 4, dq);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            store_part(tn, st ^ 1, 2 * ks);
            store_part(tn, st ^ 1, 2 * ks + 1);
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb) {
              const int off = (16 * cb + l16) * VROW + 32 * ks + 8 * g;
              const half8 ah = *reinterpret_cast<const half8*>(Vh + off);
              const half8 al = *reinterpret_cast<const half8*>(Vl + off);
#pragma unroll
              for (int qb = 0; qb < 2; ++qb) {
                O[qb][cb] = mfma16(ah, pf[qb][ks], O[qb][cb]);
                O[qb][cb] = mfma16(al, pf[qb][ks], O[qb][cb]);
              }
            }
          }
        }
      }
    }

    // waves that ran the P.V product have staged the next tile's khat and
    // vhat already
    if (tile + 1 < thi) {
      if (NOV || !wave_live) {
        store_stage(tn, st ^ 1);
      } else {
        store_coef(tn, st ^ 1);
      }
    }
    __syncthreads();
  }

  if constexpr (TOP1) {
    if (!wave_live) return;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // the four lane groups holding this Query: larger logit, then smaller index
      float bv = bval[qb];
      int bi = bidx[qb];
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      const int64_t qi = qw0 + 16 * qb + l16;
      if (qi >= a.nq || g != 0) continue;
      if (a.splits == 1) {
        a.top1[(int64_t)h * a.nq + qi] = bi;
      } else {
        const int64_t row = ((int64_t)split * a.H + h) * a.nq + qi;
        a.part_ml[row * 2] = bv;
        a.part_ml[row * 2 + 1] = __int_as_float(bi);
      }
    }
  }
  if constexpr (!NOV) {
    if (!wave_live) return;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float l = lrow[qb];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      const int64_t qi = qw0 + 16 * qb + l16;
      if (qi >= a.nq) continue;
      if (a.splits == 1) {
        const float inv = 1.0f / l;
        float* dst = a.out + ((int64_t)h * a.nq + qi) * D + 4 * g;
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) {
          const floatx4 o = O[qb][cb] * inv;
          *reinterpret_cast<float4*>(dst + 16 * cb) = make_float4(o[0], o[1], o[2], o[3]);
        }
      } else {
        const int64_t row = ((int64_t)split * a.H + h) * a.nq + qi;
        float* dst = a.part_o + row * D + 4 * g;
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) {
          const floatx4 o = O[qb][cb];
          *reinterpret_cast<float4*>(dst + 16 * cb) = make_float4(o[0], o[1], o[2], o[3]);
        }
        if (g == 0) {
          a.part_ml[row * 2] = mrow[qb];
          a.part_ml[row * 2 + 1] = l;
        }
      }
    }
  }
}

// Top-1 over the split partials (value, index) of each (head, Query): the
// larger logit wins, the smaller token index on a tie.
__global__ __launch_bounds__(256) void top1_merge_kernel(const AttnArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)a.H * a.nq;
  if (row >= rows) return;
  float bv = -__builtin_inff();
  int bi = 0x7fffffff;
  for (int s = 0; s < a.splits; ++s) {
    const float v = a.part_ml[(s * rows + row) * 2];
    const int i = __float_as_int(a.part_ml[(s * rows + row) * 2 + 1]);
    if (v > bv || (v == bv && i < bi)) {
      bv = v;
      bi = i;
    }
  }
  a.top1[row] = bi;
}

// Log-sum-exp merge of the split-KV partials (log2 domain), two shapes:
// merge_kernel runs one thread per (head, Query, 4 channels) over every
// split, for many rows and few splits (the prefill path); merge_rows_kernel
// runs one workgroup per (head, Query) row with thread = (4 channels, split
// group), split group sg taking splits sg, sg + SG, ... with a running
// maximum of its own, and combines the SG partial sums in group order
// through LDS, for few rows and many splits (the decode path: up to 64).
// Every split's partial row is read once.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const AttnArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)a.H * a.nq;
  if (idx >= rows * (D / 4)) return;
  const int64_t row = idx / (D / 4);  // h * nq + qi
  const int c4 = (int)(idx % (D / 4));
  float M = -__builtin_inff();
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.part_ml[(s * rows + row) * 2]);
  float L = 0.0f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < a.splits; ++s) {
    const int64_t pr = s * rows + row;
    const float m = a.part_ml[pr * 2];
    const float w = (m == -__builtin_inff()) ? 0.0f : exp2f(m - M);
    L += a.part_ml[pr * 2 + 1] * w;
    const float4 po = *reinterpret_cast<const float4*>(a.part_o + pr * D + 4 * c4);
    o.x += po.x * w;
    o.y += po.y * w;
    o.z += po.z * w;
    o.w += po.w * w;
  }
  const float inv = 1.0f / L;
  *reinterpret_cast<float4*>(a.out + row * D + 4 * c4) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
}

constexpr int kMergeRowThreads = 512;

template <int D>
__global__ __launch_bounds__(kMergeRowThreads) void merge_rows_kernel(const AttnArgs a) {
  constexpr int CQ = D / 4;                   // channel quads per row
  constexpr int SG = kMergeRowThreads / CQ;  // split groups
  __shared__ float4 red_o[SG][CQ];
  __shared__ float red_l[SG][CQ], red_m[SG][CQ];
  const int64_t row = blockIdx.x;  // h * nq + qi
  const int64_t rows = (int64_t)a.H * a.nq;
  const int c4 = threadIdx.x % CQ, sg = threadIdx.x / CQ;
  // each split group keeps its own running maximum (partials rescaled when
  // it grows), so no thread has to read every split's maximum first
  float mg = -__builtin_inff(), L = 0.0f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = sg; s < a.splits; s += SG) {
    const int64_t pr = s * rows + row;
    const float m = a.part_ml[pr * 2];
    if (m > mg) {
      const float f = (mg == -__builtin_inff()) ? 0.0f : exp2f(mg - m);
      L *= f;
      o.x *= f;
      o.y *= f;
      o.z *= f;
      o.w *= f;
      mg = m;
    }
    const float w = (m == -__builtin_inff()) ? 0.0f : exp2f(m - mg);
    L += a.part_ml[pr * 2 + 1] * w;
    const float4 po = *reinterpret_cast<const float4*>(a.part_o + pr * D + 4 * c4);
    o.x += po.x * w;
    o.y += po.y * w;
    o.z += po.z * w;
    o.w += po.w * w;
  }
  red_o[sg][c4] = o;
  red_l[sg][c4] = L;
  red_m[sg][c4] = mg;
  __syncthreads();
  if (sg != 0) return;
  float M = mg;
#pragma unroll
  for (int g = 1; g < SG; ++g) M = fmaxf(M, red_m[g][c4]);
  o = make_float4(0.f, 0.f, 0.f, 0.f);
  L = 0.0f;
#pragma unroll
  for (int g = 0; g < SG; ++g) {
    const float m = red_m[g][c4];
    const float f = (m == -__builtin_inff()) ? 0.0f : exp2f(m - M);
    const float4 p = red_o[g][c4];
    o.x += p.x * f;
    o.y += p.y * f;
    o.z += p.z * f;
    o.w += p.w * f;
    L += red_l[g][c4] * f;
  }
  const float inv = 1.0f / L;
  *reinterpret_cast<float4*>(a.out + row * D + 4 * c4) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
}

// q . U_r for every epoch slot: qU[h][e][i][k] (k < 16, zero for k >= r).
// One wave per 64 Queries of one head and one epoch slot: D[Query][rank] =
// q U by v_mfma_f32_16x16x32_f16 with the Query fragments in fp16 (bf16
// inputs are exact; float32 inputs add a lo part) and U as fp16 hi + lo
// (products exact, float32 sums).
template <int D, int DT>
__global__ __launch_bounds__(64) void qu_kernel(const void* q, int64_t nq, int r, const float* Ubase,
                                                int64_t ustride, int E, float* qU) {
  constexpr int KS = D / 32;
  constexpr int QB = 4;  // 16-Query blocks per wave: the U fragments are loaded once for all of them
  const int lane = threadIdx.x, g = lane >> 4, l16 = lane & 15;
  const int h = blockIdx.y;
  // one epoch slot per workgroup (blockIdx.z): the slots' U loads and MFMA
  // chains run side by side instead of one after another
  const int ep = blockIdx.z;
  // B: U column l16 (rank), channels 32ks + 8g .. +7, as fp16 hi + lo;
  // ranks past r are zero
  const bool rv = l16 < r;
  const float* U = Ubase + (int64_t)ep * ustride + (int64_t)h * D * r;
  half8 uh[KS], ul[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = rv ? U[(32 * ks + 8 * g + e) * r + l16] : 0.0f;
      const _Float16 hi = (_Float16)x;
      uh[ks][e] = hi;
      ul[ks][e] = (_Float16)(x - (float)hi);
    }
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t q0 = ((int64_t)blockIdx.x * QB + qb) * 16;
    if (q0 >= nq) break;  // wave-uniform
    // A: Query q0 + l16, channels 32ks + 8g .. +7, in one 16-byte load per
    // step (two for float32)
    const int64_t qi = q0 + l16 < nq ? q0 + l16 : nq - 1;
    const int64_t row = ((int64_t)h * nq + qi) * D;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
      if constexpr (DT == 0) {
        const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) + row + 32 * ks + 8 * g);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[2 * k] = __uint_as_float(ww[k] << 16);
          x[2 * k + 1] = __uint_as_float(ww[k] & 0xFFFF0000u);
        }
      } else {
        const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) + row + 32 * ks + 8 * g);
        const float4 a0 = src[0], a1 = src[1];
        x[0] = a0.x; x[1] = a0.y; x[2] = a0.z; x[3] = a0.w;
        x[4] = a1.x; x[5] = a1.y; x[6] = a1.z; x[7] = a1.w;
      }
      half8 qa, qlo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const _Float16 hi = (_Float16)x[e];
        qa[e] = hi;
        qlo[e] = (_Float16)(x[e] - (float)hi);
      }
      acc = mfma16(qa, uh[ks], acc);
      acc = mfma16(qa, ul[ks], acc);
      if constexpr (DT == 1) acc = mfma16(qlo, uh[ks], acc);
    }
    // D[Query 4g + v][rank l16]
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t qo = q0 + 4 * g + v;
      if (qo < nq) qU[(((int64_t)h * E + ep) * nq + qo) * kRankPad + l16] = acc[v];
    }
  }
}

}  // namespace

hipError_t launch_qu(int D, int dtype, const void* q, int64_t nq, int H, int r, const float* Ubase,
                     int64_t ustride, int E, float* qU, hipStream_t s) {
  if (E < 1) return hipSuccess;
  dim3 grid((unsigned)((nq + 63) / 64), (unsigned)H, (unsigned)E), block(64);
  if (D == 128 && dtype == 0)
    hipLaunchKernelGGL((qu_kernel<128, 0>), grid, block, 0, s, q, nq, r, Ubase, ustride, E, qU);
  else if (D == 128)
    hipLaunchKernelGGL((qu_kernel<128, 1>), grid, block, 0, s, q, nq, r, Ubase, ustride, E, qU);
  else if (dtype == 0)
    hipLaunchKernelGGL((qu_kernel<64, 0>), grid, block, 0, s, q, nq, r, Ubase, ustride, E, qU);
  else
    hipLaunchKernelGGL((qu_kernel<64, 1>), grid, block, 0, s, q, nq, r, Ubase, ustride, E, qU);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_attend_impl(int D, int dtype, const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  dim3 grid((unsigned)((a.nq + a.qpb - 1) / a.qpb), (unsigned)a.splits,
            MODE == kModeLogits ? 1u : (unsigned)a.H);
  dim3 block(kAttnThreads);
  if (D == 128 && dtype == 0)
    hipLaunchKernelGGL((attend_kernel<128, 0, MODE>), grid, block, 0, s, a, p);
  else if (D == 128)
    hipLaunchKernelGGL((attend_kernel<128, 1, MODE>), grid, block, 0, s, a, p);
  else if (dtype == 0)
    hipLaunchKernelGGL((attend_kernel<64, 0, MODE>), grid, block, 0, s, a, p);
  else
    hipLaunchKernelGGL((attend_kernel<64, 1, MODE>), grid, block, 0, s, a, p);
  return hipGetLastError();
}

hipError_t launch_attend(int D, int dtype, const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  if (D == 128 && dtype == 0) return launch_attend_bf16(a, p, s);
  return launch_attend_impl<kModeAttend>(D, dtype, a, p, s);
}
hipError_t launch_attend_logits(int D, int dtype, const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  return launch_attend_impl<kModeLogits>(D, dtype, a, p, s);
}
hipError_t launch_attend_top1(int D, int dtype, const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  return launch_attend_impl<kModeTop1>(D, dtype, a, p, s);
}

hipError_t launch_top1_merge(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.H * a.nq;
  hipLaunchKernelGGL(top1_merge_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(int D, const AttnArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.H * a.nq;
  if (a.splits >= 16) {  // few rows, many splits: a workgroup per row
    dim3 grid((unsigned)rows), block(kMergeRowThreads);
    if (D == 128)
      hipLaunchKernelGGL((merge_rows_kernel<128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((merge_rows_kernel<64>), grid, block, 0, s, a);
  } else {
    dim3 grid((unsigned)((rows * (D / 4) + 255) / 256)), block(256);
    if (D == 128)
      hipLaunchKernelGGL((merge_kernel<128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((merge_kernel<64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- export
namespace {
__global__ void export_kernel(const ExportArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y;
  if (t >= a.n) return;
  const int D = a.D, nG = a.nG, r = a.r;
  const int64_t n = a.n;
  const int64_t B = n * (D / 2 + 8 * nG + 1 + 2 * r + 2);
  uint8_t* base = a.out + (int64_t)h * B;
  const int64_t o_kc = 0, o_vc = n * (D / 4), o_kzp = n * (D / 2);
  const int64_t o_ksc = o_kzp + 2 * n * nG, o_vzp = o_ksc + 2 * n * nG, o_vsc = o_vzp + 2 * n * nG;
  const int64_t o_id = o_vsc + 2 * n * nG, o_cf = o_id + n, o_ep = o_cf + 2 * n * r;
  const int64_t pos = a.t0 + t;
  const int64_t slot = (int64_t)h * a.cache.capP + pos;
  for (int b = 0; b < D / 4; ++b) {
    base[o_kc + t * (D / 4) + b] = a.cache.kcode[slot * (D / 4) + b];
    base[o_vc + t * (D / 4) + b] = a.cache.vcode[slot * (D / 4) + b];
  }
  for (int G = 0; G < nG; ++G) {
    const uint32_t kp = a.cache.kparam[slot * nG + G], vp = a.cache.vparam[slot * nG + G];
    const int64_t e = 2 * (t * nG + G);
    base[o_kzp + e] = kp & 0xFF;
    base[o_kzp + e + 1] = (kp >> 8) & 0xFF;
    base[o_ksc + e] = (kp >> 16) & 0xFF;
    base[o_ksc + e + 1] = (kp >> 24) & 0xFF;
    base[o_vzp + e] = vp & 0xFF;
    base[o_vzp + e + 1] = (vp >> 8) & 0xFF;
    base[o_vsc + e] = (vp >> 16) & 0xFF;
    base[o_vsc + e + 1] = (vp >> 24) & 0xFF;
  }
  base[o_id + t] = a.cache.ids[slot];
  for (int i = 0; i < r; ++i) {
    const uint16_t c = a.cache.coef[slot * r + i];
    base[o_cf + 2 * (t * r + i)] = c & 0xFF;
    base[o_cf + 2 * (t * r + i) + 1] = c >> 8;
  }
  int e = 0;
  for (int i = 1; i < a.n_epochs; ++i)
    if (a.epoch_start[i] <= pos) e = i;
  base[o_ep + 2 * t] = (uint8_t)(e & 0xFF);
  base[o_ep + 2 * t + 1] = (uint8_t)(e >> 8);
}
}  // namespace

hipError_t launch_export(const ExportArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  dim3 grid((unsigned)((a.n + 255) / 256), (unsigned)a.H), block(256);
  hipLaunchKernelGGL(export_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace qwm
