// Attention over the 2-bit QuantWM cache, bf16 inputs and head_dim 128
// (gfx950): the prefill path of qwm_attend (more than 64 Queries per head,
// or a self segment).
//
// Method (QuantWM; fugumt.com abstract: PSAC puts the Key error left after
// quantization back along the dominant Query subspace so the attention logits
// stay stable; roboind.com "Step 1" and "Step 2"): for cached token j of
// epoch e(j) with centroid c, per-group zero-point zp_G, step s_G and 2-bit
// codes,
//   l_ij = (q_i . c + sum_G zp_G (sum of q_i over G) + q_i . (code * s)
//           + (q_i U_r^(e(j))) . coef_j) * scale,
// plus optional full-precision self tokens of the attending chunk; softmax
// over all visible tokens and o_i = sum_j p_ij (zp + code * s)_j.
//
// Every operand is exact in fp16 or split so that no product loses a bit:
//  * c: bf16 centroid rows converted to fp16 (exact in fp16's range);
//  * code * s: the step is chosen so that 3 s is an fp16 value, so every
//    code * s (code 0..3) is one;
//  * q: bf16 Queries in fp16 (exact); the group sums of q as fp16 hi + lo;
//  * q U_r as fp16 hi against the fp16 coefficients, plus the lo part for
//    the 8 leading principal directions (which carry most of the Query
//    energy; the lo parts of the other 8 are the one rounding left on the
//    Key side, about 2^-12 of their already small share);
//  * Values: o = P (code * s) + P zp, the zero-point term on its own MFMA
//    with four rows (one per group) that is added to the output at the end.
// The only roundings are the fp32 accumulations and P in fp16.
//
// Mapping to CDNA4:
//  * one workgroup = 8 waves = up to 256 Queries of one head (32 per wave),
//    one split of the KV tiles (64 tokens, never crossing an epoch or the
//    cache/self boundary);
//  * the tile's K operands ([c | code*s | coef, zp]) and V^T operands are
//    built ONCE per workgroup in LDS (thread = one token x 16 channels of K,
//    two tokens x 8 channels of V^T);
//  * two wave groups in opposite phase: each SIMD holds one wave of waves
//    0-3 and one of waves 4-7. In step i the first group runs the softmax
//    and P . V of tile i, builds its share of the next stages and then the
//    logits of tile i+1; the second group starts with the logits of tile i.
//    So while one wave of a SIMD is on the VALU (softmax, stage
//    construction) the other is on the MFMA pipe. K stages are triple
//    buffered (tiles i and i+1 are read while i+2 is built), V stages double
//    buffered; one barrier per tile.
#include "qwm_codes.h"
#include "qwm_dev.h"
#include "qwm_internal.h"

namespace qwm {

namespace {

typedef float float2v __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kNG = kD / kGroup;
constexpr int kKRow = 296;   // halves per token row of a K stage: c (128) | code*s (128) | X (32) | pad (8)
constexpr int kCsOff = 128;  // code * s
constexpr int kXOff = 256;   // X: coef 0..15 | zp_0..3, zp_0..3 | coef 0..7
constexpr int kVRow = 72;    // halves per row of a V stage (64 token slots + pad)
constexpr int kVRows = 144;  // 128 channels, 4 zero-point rows, 12 zero rows
constexpr int kKSt = kTileKV * kKRow;
constexpr int kVSt = kVRows * kVRow;
constexpr int kKStages = 3, kVStages = 2;

__device__ __forceinline__ floatx4 mfma16(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half2v pk_f16(float x, float y) { return __builtin_convertvector(float2v{x, y}, half2v); }
// two bf16 (one word) -> two fp16
__device__ __forceinline__ half2v bf2_to_h2(uint32_t w) {
  return pk_f16(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
}
__device__ __forceinline__ uint32_t h2_bits(half2v h) { return __builtin_bit_cast(uint32_t, h); }
// x combined with lane l ^ 16 / l ^ 32 through the gfx950 row-swap
// permutes (VALU; a __shfl_xor becomes an LDS-pipe ds_bpermute): after the
// swap of a register with itself the two results hold, in every lane, the
// lane's own value and its partner's.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {  // x + partner (addition commutes exactly)
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The 16 codes of one 32-bit word (code c of channel c in bits 2c..2c+1)
// times the step s (fp16 bits s_bits), as fp16 pairs (channels 2p, 2p+1 in
// out[p]).
__device__ __forceinline__ void codes_times_step(uint32_t w, uint32_t s_bits, uint32_t (&out)[8]) {
  const CodeScale cs = code_scale(s_bits | (s_bits << 16));
  uint32_t x[8];  // codes 2p, 2p+1 of half `half` (x[4 half + p]) in bits 0-1 and 16-17
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t h = (w >> (16 * half)) & 0xFFFFu;
    const uint32_t y = h | (h << 14);  // code 2p at bits 4p, code 2p+1 at bits 16+4p
#pragma unroll
    for (int p = 0; p < 4; ++p) x[4 * half + p] = y >> (4 * p);
  }
  code_pairs(x, cs, out);
}

struct TileInfo {
  int ep;      // epoch slot, -1 for the self segment
  int tstart;  // first token (cache position, or index into the self K/V)
  int tcount;  // tokens in the tile (1..64)
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

// Raw words one thread stages for the K operands of a tile (token = lane,
// channels 16 kq .. 16 kq + 15 with kq = wave): the centroid (or self Key)
// slice as 16 bf16, the code word, the group's parameter word and 8 PSAC
// coefficients (waves 0 and 1).
struct RawK {
  uint4 c0, c1, cf;
  uint32_t code, prm;
};
// ... and for the V^T operands, where a thread takes two neighbouring tokens
// (2 p and 2 p + 1, p = lane mod 32) and 8 channels (16 kq + 8 hh .. +7,
// hh = lane / 32): both tokens' code and parameter words, and their self
// Value slices (SELF kernels only).
struct RawV {
  uint32_t code0, code1, prm0, prm1;
  uint4 s0, s1;
};

// The centroid tables of epoch slots 0 .. n - 1 (n * H * m rows of 128 bf16)
// as fp16, rounded to nearest even: read by the tile loads of the kernel
// below, so that no workgroup converts a centroid row per tile.
__global__ __launch_bounds__(256) void c16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const uint4 w = src[i];
    dst[i] = make_uint4(h2_bits(bf2_to_h2(w.x)), h2_bits(bf2_to_h2(w.y)), h2_bits(bf2_to_h2(w.z)),
                        h2_bits(bf2_to_h2(w.w)));
  }
}

// SELF: the plan may hold a self segment (full-precision K/V of the chunk).
// C16: the centroid rows come from the fp16 copy (a.C16) instead of the bf16
// tables.
template <bool SELF, bool C16>
__global__ __launch_bounds__(kAttnThreads) void attend_bf16_kernel(const AttnArgs a, const AttnPlan p) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[kKStages * kKSt + kVStages * kVSt];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  // Workgroups go to the 8 XCDs in turn (dispatch id mod 8). Renumber them so
  // that each XCD receives one contiguous run of logical ids, Query blocks
  // fastest: the Query blocks of one (head, split) then run side by side on
  // one XCD and read each KV tile once into its L2 (a bijection of the grid
  // whatever the dispatch order).
  int h, split, qblk;
  {
    const int nwg = (int)gridDim.x, bid = (int)blockIdx.x;
    const int per = nwg >> 3, rem = nwg & 7, xcd = bid & 7;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + (bid >> 3);
    const int nqb = (int)((a.nq + a.qpb - 1) / a.qpb);
    qblk = logical % nqb;
    const int hs = logical / nqb;
    split = hs % a.splits;
    h = hs / a.splits;
  }
  const int64_t qw0 = (int64_t)qblk * a.qpb + wave * 32;
  const bool wave_live = wave * 32 < a.qpb && qw0 < a.nq;
  const bool lead = wave < 4;  // the group that computes the next tile's logits at the end of a step
  const int kq = wave;  // producer channel slice 16 kq .. 16 kq + 15 (group kq / 2)
  // softmax in the log2 domain with a positive factor; a negative scale is
  // carried by negated Queries (exact in fp16)
  const float qsign = (a.scale_log2 < 0.0f) ? -1.0f : 1.0f;
  const float cl2 = a.scale_log2 * qsign;

  const int T = p.tile_prefix[p.n_seg];
  const int tlo = (int)(((int64_t)T * split) / a.splits);
  const int thi = (int)(((int64_t)T * (split + 1)) / a.splits);

  // per-head bases; per-token offsets fit 32 bits (capacity <= 2^26)
  const uint8_t* kcode_h = a.cache.kcode + (size_t)h * a.cache.capP * (kD / 4);
  const uint8_t* vcode_h = a.cache.vcode + (size_t)h * a.cache.capP * (kD / 4);
  const uint32_t* kparam_h = a.cache.kparam + (size_t)h * a.cache.capP * kNG;
  const uint32_t* vparam_h = a.cache.vparam + (size_t)h * a.cache.capP * kNG;
  const uint8_t* ids_h = a.cache.ids + (size_t)h * a.cache.capP;
  const uint16_t* coef_h = a.cache.coef + (size_t)h * a.cache.capP * a.r;
  const uint16_t* kself_h = reinterpret_cast<const uint16_t*>(a.kself) + (size_t)h * a.nself * kD;
  const uint16_t* vself_h = reinterpret_cast<const uint16_t*>(a.vself) + (size_t)h * a.nself * kD;
  // centroid rows: 128 halves (bf16, or fp16 in the copy), same layout
  const char* C_h = reinterpret_cast<const char*>(C16 ? a.C16 : a.Cbase) + (size_t)h * a.m * kD * 2;

  // rows of the stages that never change: the zero rows 132..143 of each V
  // stage
  for (int e = tid; e < kVStages * 12 * kVRow; e += kAttnThreads) {
    const int st = e / (12 * kVRow), r = e % (12 * kVRow);
    lds[kKStages * kKSt + st * kVSt + 132 * kVRow + r] = (_Float16)0.0f;
  }

  // ---- producer: loads (no use of the data) and stage construction
  // Token indices are clamped into the tile (tcount >= 1) and loads a tile
  // does not need read a valid dummy address (the head's first cache slot),
  // so every load is unconditional: no register a load is still filling is
  // written on another path.
  auto load_id = [&](const TileInfo& ti) -> uint32_t {
    const int t = lane < ti.tcount ? lane : ti.tcount - 1;
    return ids_h[(!SELF || ti.ep >= 0) ? (uint32_t)(ti.tstart + t) : 0u];
  };
  // coefficient halves 8 kq .. 8 kq + 7 that lie below r (waves 0 and 1),
  // as masks of the four words: wave-uniform, computed once
  uint32_t cfm[4];
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    const int j = 8 * kq + 2 * s2;
    cfm[s2] = (kq < 2 && j < a.r) ? (j + 1 < a.r ? 0xFFFFFFFFu : 0xFFFFu) : 0u;
  }
  auto load_k = [&](RawK& r, const TileInfo& ti, uint32_t id) {
    const bool cache = !SELF || ti.ep >= 0;
    const uint32_t slot = (uint32_t)(ti.tstart + (lane < ti.tcount ? lane : ti.tcount - 1));
    const uint32_t cs = cache ? slot : 0u;
    const uint4* src =
        cache ? reinterpret_cast<const uint4*>(C_h + (size_t)ti.ep * a.epoch_C_stride + ((size_t)id * kD + 16 * kq) * 2)
              : reinterpret_cast<const uint4*>(kself_h + (size_t)slot * kD + 16 * kq);
    r.c0 = src[0];
    r.c1 = src[1];
    r.code = *reinterpret_cast<const uint32_t*>(kcode_h + cs * (kD / 4) + 4 * kq);
    r.prm = kparam_h[cs * kNG + (kq >> 1)];
    // coefficients 8 kq .. 8 kq + 7 (waves 0, 1; halves past r are zeroed at
    // store): r even, four dword loads; r odd, halves one by one
    const uint16_t* cf = coef_h + cs * (uint32_t)a.r + (kq < 2 ? 8 * kq : 0);
    if ((a.r & 1) == 0) {
      const uint32_t* cw = reinterpret_cast<const uint32_t*>(cf);
      r.cf = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    } else {
      uint32_t cc[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const int j = (kq < 2 ? 8 * kq : 0) + 2 * s2;
        const uint32_t lo = (j < a.r) ? cf[2 * s2] : 0u;
        const uint32_t hi = (j + 1 < a.r) ? cf[2 * s2 + 1] : 0u;
        cc[s2] = lo | (hi << 16);
      }
      r.cf = make_uint4(cc[0], cc[1], cc[2], cc[3]);
    }
  };
  auto load_v = [&](RawV& r, const TileInfo& ti) {
    const bool cache = !SELF || ti.ep >= 0;
    const int j0 = 2 * (lane & 31);
    const uint32_t slot0 = (uint32_t)(ti.tstart + (j0 < ti.tcount ? j0 : ti.tcount - 1));
    const uint32_t slot1 = (uint32_t)(ti.tstart + (j0 + 1 < ti.tcount ? j0 + 1 : ti.tcount - 1));
    const uint32_t cs0 = cache ? slot0 : 0u, cs1 = cache ? slot1 : 0u;
    r.code0 = *reinterpret_cast<const uint32_t*>(vcode_h + cs0 * (kD / 4) + 4 * kq);
    r.code1 = *reinterpret_cast<const uint32_t*>(vcode_h + cs1 * (kD / 4) + 4 * kq);
    r.prm0 = vparam_h[cs0 * kNG + (kq >> 1)];
    r.prm1 = vparam_h[cs1 * kNG + (kq >> 1)];
    if constexpr (SELF) {
      const int ch = 16 * kq + 8 * (lane >> 5);
      r.s0 = cache ? *reinterpret_cast<const uint4*>(vcode_h)
                   : *reinterpret_cast<const uint4*>(vself_h + (size_t)slot0 * kD + ch);
      r.s1 = cache ? *reinterpret_cast<const uint4*>(vcode_h)
                   : *reinterpret_cast<const uint4*>(vself_h + (size_t)slot1 * kD + ch);
    }
  };
  // K stage row of the thread's token: c (or the self Key), code * s, and
  // the X block (coefficients from waves 0 and 1, the leading 8 once more
  // from wave 0, the group's zero-point from the even waves); self tokens
  // have zero code, step, zero-point and coefficients.
  auto store_k = [&](const RawK& r, const TileInfo& ti, _Float16* Ks) {
    const bool cache = !SELF || ti.ep >= 0;
    _Float16* row = Ks + lane * kKRow;
    const uint32_t cw[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
    uint32_t ch[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ch[i] = (C16 && cache) ? cw[i] : h2_bits(bf2_to_h2(cw[i]));
    *reinterpret_cast<uint4*>(row + 16 * kq) = make_uint4(ch[0], ch[1], ch[2], ch[3]);
    *reinterpret_cast<uint4*>(row + 16 * kq + 8) = make_uint4(ch[4], ch[5], ch[6], ch[7]);
    const uint32_t prm = cache ? r.prm : 0u;
    uint32_t cs[8];
    codes_times_step(cache ? r.code : 0u, prm >> 16, cs);
    *reinterpret_cast<uint4*>(row + kCsOff + 16 * kq) = make_uint4(cs[0], cs[1], cs[2], cs[3]);
    *reinterpret_cast<uint4*>(row + kCsOff + 16 * kq + 8) = make_uint4(cs[4], cs[5], cs[6], cs[7]);
    if ((kq & 1) == 0) {
      const _Float16 zp = __builtin_bit_cast(_Float16, (uint16_t)(prm & 0xFFFFu));
      row[kXOff + 16 + (kq >> 1)] = zp;
      row[kXOff + 20 + (kq >> 1)] = zp;
    }
    if (kq < 2) {
      uint4 cfw = make_uint4(r.cf.x & cfm[0], r.cf.y & cfm[1], r.cf.z & cfm[2], r.cf.w & cfm[3]);
      if (!cache) cfw = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(row + kXOff + 8 * kq) = cfw;
      if (kq == 0) *reinterpret_cast<uint4*>(row + kXOff + 24) = cfw;  // coef 0..7 again, against q U lo
    }
  };
  // V stage: (code * s)^T rows 16 kq .. 16 kq + 15 (or the self Values) and
  // the group's zero-point row 128 + kq / 2. Token j of the tile goes to
  // column 32 (j / 32) + 8 gg + 4 b + u (b = bit 4, gg = bits 2-3, u = bits
  // 0-1 of j): the order in which lane group gg holds the tokens of a
  // 32-token step in its P fragment. Tokens 2p and 2p + 1 land in
  // neighbouring columns, so the thread writes one dword per channel: the
  // two tokens' codes of a channel are gathered into one word (token 2p in
  // bits 0-1, 2p + 1 in bits 16-17) and turned into an fp16 pair at once.
  // The two half-waves write rows 8 apart (the same banks) in separate
  // cycles.
  auto store_v = [&](const RawV& r, const TileInfo& ti, _Float16* Vs) {
    const bool cache = !SELF || ti.ep >= 0;
    const int hh = lane >> 5, j0 = 2 * (lane & 31);
    const int col = (j0 & ~31) + 8 * ((j0 >> 2) & 3) + 4 * ((j0 >> 4) & 1) + (j0 & 3);
    uint32_t v[8];
    if (!SELF || cache) {
      // both tokens' codes of channels 8 hh .. 8 hh + 7: channel c in bits
      // 2c (token 2p) and 16 + 2c (token 2p + 1)
      const uint32_t z = __builtin_amdgcn_perm(r.code1, r.code0, hh ? 0x07060302u : 0x05040100u);
      const CodeScale cs = code_scale(__builtin_amdgcn_perm(r.prm1, r.prm0, 0x07060302u));
      uint32_t x[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) x[c] = z >> (2 * c);
      code_pairs(x, cs, v);
    } else {
      // self Values: channel 2i / 2i + 1 in the low / high half of word i
      const uint32_t a[4] = {r.s0.x, r.s0.y, r.s0.z, r.s0.w};
      const uint32_t b[4] = {r.s1.x, r.s1.y, r.s1.z, r.s1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = h2_bits(pk_f16(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16)));
        v[2 * i + 1] = h2_bits(pk_f16(__uint_as_float(a[i] & 0xFFFF0000u), __uint_as_float(b[i] & 0xFFFF0000u)));
      }
    }
    uint32_t* base = reinterpret_cast<uint32_t*>(Vs + (16 * kq + 8 * hh) * kVRow + col);
#pragma unroll
    for (int c = 0; c < 8; ++c) base[c * (kVRow / 2)] = v[c];
    if ((kq & 1) == 0 && hh == 0) {
      const uint32_t z = cache ? __builtin_amdgcn_perm(r.prm1, r.prm0, 0x05040100u) : 0u;
      *reinterpret_cast<uint32_t*>(Vs + (128 + (kq >> 1)) * kVRow + col) = z;
    }
  };

  // ---- Query operands (B): Query qw0 + 16 qb + l16, channels 32 ks + 8 g .. +7
  half8 qh[2][4];
  // B operand of the X MFMA, by lane group: 0: q U hi 0..7, 1: q U hi 8..15,
  // 2: [group sums of q hi | lo], 3: q U lo 0..7
  half8 xw[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t qi = qw0 + 16 * qb + l16;
    const bool qv = qi < a.nq;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)h * a.nq + (qv ? qi : 0)) * kD;
    float gs[kNG];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 w = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
      float s = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x0 = qv ? qsign * __uint_as_float(ww[k] << 16) : 0.0f;
        const float x1 = qv ? qsign * __uint_as_float(ww[k] & 0xFFFF0000u) : 0.0f;
        qh[qb][ks][2 * k] = (_Float16)x0;
        qh[qb][ks][2 * k + 1] = (_Float16)x1;
        s += x0;
        s += x1;
      }
      // group ks = channels 32 ks .. 32 ks + 31: the four lane groups' parts
      gs[ks] = add_xor32(add_xor16(s));
    }
#pragma unroll
    for (int G = 0; G < kNG; ++G) {
      const _Float16 hi = (_Float16)gs[G];
      const _Float16 lo = (_Float16)(gs[G] - (float)hi);
      xw[qb][G] = (g == 2) ? hi : (_Float16)0.0f;
      xw[qb][G + 4] = (g == 2) ? lo : (_Float16)0.0f;
    }
  }
  int cur_epoch = -2;
  auto set_epoch = [&](int ep) {
    if (ep == cur_epoch) return;
    cur_epoch = ep;
    if (g == 2) return;  // the group sums do not change
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int64_t qi = qw0 + 16 * qb + l16;
      if (ep >= 0 && qi < a.nq && a.r > 0) {
        // lane group 1 takes directions 8..15 (hi); groups 0 and 3 take 0..7 (hi, lo)
        const float* src = a.qU + (((int64_t)h * a.n_epoch_slots + ep) * a.nq + qi) * kRankPad + (g == 1 ? 8 : 0);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const float x = qsign * src[s2];
          const _Float16 hi = (_Float16)x;
          xw[qb][s2] = (g < 2) ? hi : (_Float16)(x - (float)hi);
        }
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) xw[qb][s2] = (_Float16)0.0f;
      }
    }
  };

  // logits S^T blocks [16 tokens x 16 Queries] of the tile in stage Ks, in
  // eight steps (32 channels x two 16-token blocks: the c and code*s
  // fragments, 4 reads) and the X step. Each step's operands are read while
  // earlier steps' MFMAs run (kAhead steps ahead: two where the registers
  // allow, in the kernel without a self segment), so a wait for LDS never
  // idles the wave behind a single MFMA; the c products come before the
  // code*s products of a step.
  constexpr int kAhead = SELF ? 1 : 2, kBufs = kAhead + 1;
  auto logits = [&](const _Float16* Ks, floatx4 (&S)[2][4]) {
    const _Float16* rb = Ks + l16 * kKRow + 8 * g;
    half8 A[kBufs][4];
    auto rd = [&](half8 (&buf)[4], int stp) {  // ks = stp / 2, blocks tb = 2 (stp % 2) ..
      const int ks = stp >> 1, tb0 = 2 * (stp & 1);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        buf[2 * j] = *reinterpret_cast<const half8*>(rb + 16 * (tb0 + j) * kKRow + 32 * ks);
        buf[2 * j + 1] = *reinterpret_cast<const half8*>(rb + 16 * (tb0 + j) * kKRow + 32 * ks + kCsOff);
      }
    };
    auto rdx = [&](half8 (&buf)[4]) {  // X operands of the four blocks (lane group g: X[8g .. 8g+7])
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) buf[tb] = *reinterpret_cast<const half8*>(rb + 16 * tb * kKRow + kXOff);
    };
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) S[qb][tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int stp = 0; stp < kAhead; ++stp) rd(A[stp], stp);
#pragma unroll
    for (int stp = 0; stp < 9; ++stp) {
      __builtin_amdgcn_sched_barrier(0);
      const int nx = stp + kAhead;  // the step whose operands are read now
      if (nx < 8)
        rd(A[nx % kBufs], nx);
      else if (nx == 8)
        rdx(A[8 % kBufs]);
      if (stp < 8) {
        const int ks = stp >> 1, tb0 = 2 * (stp & 1);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              S[qb][tb0 + j] = mfma16(A[stp % kBufs][2 * j + pass], qh[qb][ks], S[qb][tb0 + j]);
      } else {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) S[qb][tb] = mfma16(A[8 % kBufs][tb], xw[qb], S[qb][tb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  floatx4 O[2][kD / 16], Z[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    Z[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < kD / 16; ++cb) O[qb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  float lrow[2] = {0.0f, 0.0f};
  float mrow[2] = {-__builtin_inff(), -__builtin_inff()};
  const half2v one2 = {(_Float16)1.0f, (_Float16)1.0f};

  // Online softmax of tile ti's logits S (log2 domain) into the fp16 P
  // fragments. The running max is raised only when a row's new max exceeds
  // it by more than 8 (p <= 2^8 stays exact enough in fp16 and float32), so
  // the output rescale is rare.
  auto softmax = [&](const TileInfo& ti, floatx4 (&S)[2][4], half8 (&pf)[2][2]) {
    const bool full = (ti.tcount == kTileKV) && !(ti.ep < 0 && a.causal_self);
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
            if (ti.ep < 0 && a.causal_self) ok = ok && ((int64_t)(ti.tstart + j) <= qi);
            if (!ok) S[qb][tb][v] = -__builtin_inff();
          }
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int v = 0; v < 4; ++v) mx = fmaxf(mx, S[qb][tb][v]);
      // The row maximum is needed only where the running max rises, which
      // any of its four lanes sees from its own 16 logits; the lanes
      // exchange maxima only then (wave-uniform: rescale every lane, alpha
      // = 1 where unchanged).
      if (__ballot(mx * cl2 > mrow[qb] + 8.0f)) {
        mx = max_xor32(max_xor16(mx)) * cl2;
        const bool raise = mx > mrow[qb] + 8.0f;
        const float mnew = raise ? mx : mrow[qb];
        const float alpha = (mrow[qb] == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(mrow[qb] - mnew);
        mrow[qb] = mnew;
        lrow[qb] *= alpha;
        Z[qb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < kD / 16; ++cb) O[qb][cb] *= alpha;
      }
      // mrow is finite as soon as any logit of the row is: a row still at
      // -inf has only masked (-inf) logits, and exp2(-inf * c + 0) = 0
      const float nm = (mrow[qb] == -__builtin_inff()) ? 0.0f : -mrow[qb];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float pv[2][4];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int v = 0; v < 4; ++v) pv[t2][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][2 * ks + t2][v], cl2, nm));
        const half2v p0 = pk_f16(pv[0][0], pv[0][1]), p1 = pk_f16(pv[0][2], pv[0][3]);
        const half2v p2 = pk_f16(pv[1][0], pv[1][1]), p3 = pk_f16(pv[1][2], pv[1][3]);
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
  };

  // o^T += (code * s)^T P^T and the zero-point rows, in eight steps of two
  // channel blocks (the zero-point rows join the last step of each 32-token
  // half); each step's operands are read while the previous step's MFMAs run.
  auto pv = [&](const _Float16* Vs, const half8 (&pf)[2][2]) {
    const _Float16* rb = Vs + l16 * kVRow + 8 * g;
    half8 B[kBufs][3];
    auto rd = [&](half8 (&buf)[3], int stp) {  // ks = stp / 4, channel blocks 2 (stp % 4), +1
      const int ks = stp >> 2, cb0 = 2 * (stp & 3);
      buf[0] = *reinterpret_cast<const half8*>(rb + 16 * cb0 * kVRow + 32 * ks);
      buf[1] = *reinterpret_cast<const half8*>(rb + 16 * (cb0 + 1) * kVRow + 32 * ks);
      if ((stp & 3) == 3) buf[2] = *reinterpret_cast<const half8*>(rb + 128 * kVRow + 32 * ks);
    };
#pragma unroll
    for (int stp = 0; stp < kAhead; ++stp) rd(B[stp], stp);
#pragma unroll
    for (int stp = 0; stp < 8; ++stp) {
      __builtin_amdgcn_sched_barrier(0);
      if (stp + kAhead < 8) rd(B[(stp + kAhead) % kBufs], stp + kAhead);
      const int ks = stp >> 2, cb0 = 2 * (stp & 3);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) O[qb][cb0 + j] = mfma16(B[stp % kBufs][j], pf[qb][ks], O[qb][cb0 + j]);
      if ((stp & 3) == 3) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) Z[qb] = mfma16(B[stp % kBufs][2], pf[qb][ks], Z[qb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  _Float16* const Kst0 = lds;
  _Float16* const Vst0 = lds + kKStages * kKSt;
  auto clampt = [&](int t) { return t < thi ? t : thi - 1; };

  RawK rk;
  RawV rv;
  uint32_t id_next = 0;
  floatx4 S[2][4];

  if (tlo < thi) {
    // prologue: K(tlo), K(tlo+1) and V(tlo) staged, the raw words of K(tlo+2)
    // and V(tlo+1) and the id of tile tlo+3 in registers; the leading group
    // holds the logits of tile tlo
    const TileInfo t0 = tile_info(p, tlo);
    load_k(rk, t0, load_id(t0));
    load_v(rv, t0);
    store_k(rk, t0, Kst0);
    store_v(rv, t0, Vst0);
    const TileInfo t1 = tile_info(p, clampt(tlo + 1));
    load_k(rk, t1, load_id(t1));
    store_k(rk, t1, Kst0 + kKSt);
    const TileInfo t2 = tile_info(p, clampt(tlo + 2));
    load_k(rk, t2, load_id(t2));
    id_next = load_id(tile_info(p, clampt(tlo + 3)));
    load_v(rv, t1);
    __syncthreads();
    if (lead && wave_live) {
      set_epoch(t0.ep);
      logits(Kst0, S);
    }
    // Tile descriptors of tiles i .. i+4 (clamped to the last tile) in a
    // ring advanced once per step: a segment cursor moves by at most one
    // segment per tile (every segment holds a tile), so each step costs a
    // few scalar operations instead of a search of the plan.
    TileInfo tr[5] = {t0, t1, t2, tile_info(p, clampt(tlo + 3)), tile_info(p, clampt(tlo + 4))};
    int cur_t = clampt(tlo + 4);
    int sg = 0;
    while (p.tile_prefix[sg + 1] <= cur_t) ++sg;
    int seg_tp = p.tile_prefix[sg], seg_tp1 = p.tile_prefix[sg + 1];
    int seg_s = p.seg_start[sg], seg_e = p.seg_start[sg] + p.seg_len[sg], seg_ep = p.seg_epoch[sg];
    // Step i (stages: K(i) in ks0, K(i+1) in ks1, K(i+2) built into ks2;
    // V(i) in vs0, V(i+1) built into vs1)
    int ks0 = 0, vs0 = 0;
    for (int i = tlo; i < thi; ++i) {
      const int ks1 = ks0 == 2 ? 0 : ks0 + 1, ks2 = ks1 == 2 ? 0 : ks1 + 1;
      const TileInfo ti = tr[0];
      if (wave_live) {
        if (!lead) {
          set_epoch(ti.ep);
          logits(Kst0 + ks0 * kKSt, S);
        }
        half8 pf[2][2];
        softmax(ti, S, pf);
        pv(Vst0 + vs0 * kVSt, pf);
      }
      __builtin_amdgcn_sched_barrier(0);
      store_k(rk, tr[2], Kst0 + ks2 * kKSt);
      store_v(rv, tr[1], Vst0 + (vs0 ^ 1) * kVSt);
      load_k(rk, tr[3], id_next);
      // advance the ring to tiles i+1 .. i+5
      {
        const int nt = clampt(i + 5);
        if (nt != cur_t) {
          cur_t = nt;
          if (nt >= seg_tp1) {
            ++sg;
            seg_tp = seg_tp1;
            seg_tp1 = p.tile_prefix[sg + 1];
            seg_s = p.seg_start[sg];
            seg_e = seg_s + p.seg_len[sg];
            seg_ep = p.seg_epoch[sg];
          }
        }
        TileInfo tn;
        tn.ep = seg_ep;
        tn.tstart = seg_s + (cur_t - seg_tp) * kTileKV;
        tn.tcount = (seg_e - tn.tstart) < kTileKV ? (seg_e - tn.tstart) : kTileKV;
        tr[0] = tr[1];
        tr[1] = tr[2];
        tr[2] = tr[3];
        tr[3] = tr[4];
        tr[4] = tn;
      }
      id_next = load_id(tr[3]);  // tile i+4
      load_v(rv, tr[1]);         // tile i+2
      if (lead && wave_live && i + 1 < thi) {
        set_epoch(tr[0].ep);  // tile i+1
        logits(Kst0 + ks1 * kKSt, S);
      }
      __syncthreads();
      ks0 = ks1;
      vs0 ^= 1;
    }
  }

  if (!wave_live) return;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    // the zero-point term: group G of Query l16 sits in lane l16 (lane group
    // 0), element G
    float zg[kNG];
#pragma unroll
    for (int G = 0; G < kNG; ++G) zg[G] = __shfl(Z[qb][G], l16);
#pragma unroll
    for (int cb = 0; cb < kD / 16; ++cb) O[qb][cb] += zg[cb >> 1];
    float l = add_xor32(add_xor16(lrow[qb]));
    const int64_t qi = qw0 + 16 * qb + l16;
    if (qi >= a.nq) continue;
    if (a.splits == 1) {
      const float inv = 1.0f / l;
      float* dst = a.out + ((int64_t)h * a.nq + qi) * kD + 4 * g;
#pragma unroll
      for (int cb = 0; cb < kD / 16; ++cb) {
        const floatx4 o = O[qb][cb] * inv;
        *reinterpret_cast<float4*>(dst + 16 * cb) = make_float4(o[0], o[1], o[2], o[3]);
      }
    } else {
      const int64_t row = ((int64_t)split * a.H + h) * a.nq + qi;
      float* dst = a.part_o + row * kD + 4 * g;
#pragma unroll
      for (int cb = 0; cb < kD / 16; ++cb) {
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

}  // namespace

hipError_t launch_attend_bf16(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  const int64_t nwg = (a.nq + a.qpb - 1) / a.qpb * a.splits * a.H;
  if (nwg <= 0 || nwg > INT32_MAX) return hipErrorInvalidValue;
  const bool c16 = a.C16 != nullptr && a.n_epoch_slots > 0;
  if (c16) {
    const int64_t n = (int64_t)a.n_epoch_slots * a.epoch_C_stride / 16;  // uint4 units
    const int64_t nb = (n + 255) / 256;
    hipLaunchKernelGGL(c16_kernel, dim3((unsigned)(nb < 2048 ? nb : 2048)), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(a.Cbase), reinterpret_cast<uint4*>(a.C16), n);
  }
  dim3 grid((unsigned)nwg), block(kAttnThreads);
  if (a.nself > 0) {
    if (c16)
      hipLaunchKernelGGL((attend_bf16_kernel<true, true>), grid, block, 0, s, a, p);
    else
      hipLaunchKernelGGL((attend_bf16_kernel<true, false>), grid, block, 0, s, a, p);
  } else {
    if (c16)
      hipLaunchKernelGGL((attend_bf16_kernel<false, true>), grid, block, 0, s, a, p);
    else
      hipLaunchKernelGGL((attend_bf16_kernel<false, false>), grid, block, 0, s, a, p);
  }
  return hipGetLastError();
}

}  // namespace qwm
