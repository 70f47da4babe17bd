// Decode-shaped attention over the 2-bit QuantWM cache (gfx950): a few
// Queries per head (16 per workgroup) against a long cache, the regime
// where reading the packed cache from HBM should bound the time.
//
// Method (QuantWM; fugumt.com abstract and roboind.com "Step 1"/"Step 2"):
// for cached token t of epoch e(t), Key residual group G with zero-point zp_G
// and step s_G, centroid id(t) and PSAC coefficients coef_t,
//   l_qt = q . C_id(t) + sum_G s_G (q_G . code_G) + sum_G zp_G (sum of q over G)
//          + (q U_r^(e)) . coef_t,
// which is q . khat_t + (q U_r) . coef_t with khat = c + zp + code * s
// regrouped so that no Key is dequantized:
//  * q . C_m is one table per (head, epoch, Query) made by qc_kernel (bf16
//    products are exact, float32 sums), looked up by id;
//  * q_G . code_G runs on v_mfma_f32_16x16x32_f16 with the 2-bit codes as
//    the operand (small integers are exact in fp16; q is exact in fp16 for
//    bf16 inputs), one MFMA per group, and the group's step is applied to the
//    float32 result;
//  * zp . qsum and the PSAC term are one more pair of MFMAs ([qU_hi | qU_lo]
//    x [coef | coef], [qsum_hi | qsum_lo] x [zp | zp]);
//  * Values: o = P (code * s) + P zp. The codes times the group's step are
//    exact fp16 values (the step is chosen so that 3 s is one), staged per
//    tile in LDS (two passes of 64 channels); the zero-points of the four
//    groups form a 4-row operand of their own whose MFMA result is added to
//    the output per group at the end. P is fp16.
// Requires bf16 inputs, head_dim 128 and an even PSAC rank.
// Mapping: one workgroup = one wave = 16 Queries of one head and one
// split of the KV tiles; every wave streams its own 64-token tiles, so many
// tiles are in flight per CU. The packed words of the next tile are loaded
// while the current one is computed.
#include "qwm_codes.h"
#include "qwm_dev.h"
#include "qwm_internal.h"

namespace qwm {

namespace {

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx4 mfma_f16(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half2v pk_f16(float x, float y) { return __builtin_convertvector(float2v{x, y}, half2v); }

// DPP lane moves inside rows of 16 lanes (float bits).
template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// +inf in a VGPR, opaque to the compiler: max2 below would otherwise be
// folded back into a maximum.
__device__ __forceinline__ float opaque_inf() {
  float x;
  asm volatile("v_mov_b32 %0, 0x7f800000" : "=v"(x));
  return x;
}
// The larger of a and b as the median of (a, b, +inf): one v_med3_f32. A
// maximum (fmaxf) first quiets both inputs in IEEE mode, two more
// instructions where an input is not known to be canonical (a lane move, a
// sum); logits are never NaN.
__device__ __forceinline__ float max2(float a, float b, float inf) { return __builtin_amdgcn_fmed3f(a, b, inf); }
// Max / sum over the 16 lanes of a row; every lane of the row gets the result.
__device__ __forceinline__ float row16_max(float x, float inf) {
  x = max2(x, dpp_row<kDppQuadSwap1>(x), inf);
  x = max2(x, dpp_row<kDppQuadSwap2>(x), inf);
  x = max2(x, dpp_row<kDppRowHalfMirror>(x), inf);
  x = max2(x, dpp_row<kDppRowMirror>(x), inf);
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_row<kDppQuadSwap1>(x);
  x += dpp_row<kDppQuadSwap2>(x);
  x += dpp_row<kDppRowHalfMirror>(x);
  x += dpp_row<kDppRowMirror>(x);
  return x;
}

// The eight 2-bit codes of one 16-bit unit (code e in bits 2e .. 2e+1),
// spread by a byte permute so that codes 0..3 sit in byte 0 and codes 4..7
// in byte 2 (sel 0x0C010C00 for the low unit of a word, 0x0C030C02 for the
// high one).
__device__ __forceinline__ uint32_t spread_unit(uint32_t word, uint32_t sel) {
  return __builtin_amdgcn_perm(0u, word, sel);
}
// Spread codes -> eight fp16 values c * 2^-24 (the codes as fp16 subnormals:
// exact, no offset to remove), in the channel order 0, 4, 1, 5, 2, 6, 3, 7.
__device__ __forceinline__ half8 codes_to_f16_sub(uint32_t w) {
  uint32_t d[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) d[p] = (w >> (2 * p)) & 0x00030003u;
  return __builtin_bit_cast(half8, make_uint4(d[0], d[1], d[2], d[3]));
}

// ---------------------------------------------------------------- q . C table
// qc[h][e][c][j] = sign * q_j . C_c^(e) for Queries j < nqp (zero past nq),
// sign = the sign of the softmax scale. One wave per 16 centroids x 16
// Queries, K = 128 in four bf16 MFMAs.
__global__ __launch_bounds__(64) void qc_kernel(const uint16_t* q, int64_t nq, int nqp, const uint16_t* Cbase,
                                                int64_t epoch_C_stride, int H, int m, float sign, float* qc) {
  const int lane = threadIdx.x, i = lane & 15, kg = lane >> 4;
  const int qb = blockIdx.x, cb = blockIdx.y;
  const int h = blockIdx.z % H, e = blockIdx.z / H;
  const int c = 16 * cb + i;
  const uint16_t* Crow = Cbase + (size_t)e * epoch_C_stride + ((size_t)h * m + (c < m ? c : m - 1)) * 128;
  const int64_t qi = 16 * qb + i;
  const bool qv = qi < nq;
  const uint16_t* qrow = q + ((size_t)h * nq + (qv ? qi : 0)) * 128;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint4 aw = *reinterpret_cast<const uint4*>(Crow + 32 * ks + 8 * kg);
    uint4 bw = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * kg);
    if (!qv) bw = make_uint4(0u, 0u, 0u, 0u);
    acc = mfma_bf16(__builtin_bit_cast(bf16x8, aw), __builtin_bit_cast(bf16x8, bw), acc);
  }
  // D[row = centroid 4kg + v][col = Query i]
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int cr = 16 * cb + 4 * kg + v;
    if (cr < m) qc[(((size_t)h * (gridDim.z / H) + e) * m + cr) * nqp + 16 * qb + i] = sign * acc[v];
  }
}

struct TileInfo {
  int ep;      // epoch slot
  int tstart;  // first cache position of the tile
  int tcount;  // tokens in the tile (1..64)
};

// Tile `tile` of the plan; `sg` is a segment cursor at or before the tile's
// segment (tiles are visited in increasing order, so it only moves forward).
__device__ __forceinline__ TileInfo tile_info(const AttnPlan& p, int tile, int& sg) {
  while (p.tile_prefix[sg + 1] <= tile) ++sg;
  TileInfo ti;
  ti.ep = p.seg_epoch[sg];
  ti.tstart = p.seg_start[sg] + (tile - p.tile_prefix[sg]) * kTileKV;
  const int tend = p.seg_start[sg] + p.seg_len[sg];
  ti.tcount = (tend - ti.tstart) < kTileKV ? (tend - ti.tstart) : kTileKV;
  return ti;
}

// ---------------------------------------------------------------- decode kernel
// Raw words of one tile. Lane = token for the K words (staged in LDS); lane
// (kg, j) for the V words of tokens 16tb + j: in channel pass P (channels
// 64P .. 64P+63) the lane dequantizes channels 16(kg&1) .. +15 of group
// 2P + (kg>>1).
struct DecRaw {
  uint4 k0, k1, kp, c0, c1;
  uint32_t id;
  uint32_t vc[4][2];  // [tb][pass] 16 codes
  uint32_t vp[4][2];  // [tb][pass] zero-point | step << 16
};

// The workgroup is one wave: LDS accesses of a wave execute in program order,
// so a fence for the compiler is the only synchronization the tile stages
// need (no wait for the loads in flight).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int NQ>
__global__ __launch_bounds__(64, 2) void decode_kernel(const DecodeArgs a, const AttnPlan p) {
  static_assert(NQ == 16, "one 16-Query block per wave");
  constexpr int D = 128, NG = 4;
  // (code * s)^T of one 64-channel pass, one fp16 plane: [channel][token
  // slot], rows of 72 halves (16-byte aligned; 16 consecutive rows hit
  // distinct banks), every 16-channel block skewed by 64 bytes so the four
  // blocks written together hit different banks.
  constexpr int VROW = 72;
  constexpr int VPL = 64 * VROW + 4 * 32;  // halves of the code * s plane
  constexpr int PROW = 80;                 // P [Query][token slot] fp16
  constexpr int ZROW = 72;                 // zero-point plane: [16 rows: groups 0..3, then zeros][token slot]
  __shared__ __attribute__((aligned(16))) _Float16 vt[VPL];
  __shared__ __attribute__((aligned(16))) _Float16 zt[16 * ZROW];
  __shared__ __attribute__((aligned(16))) _Float16 pt[NQ * PROW];
  __shared__ __attribute__((aligned(16))) uint32_t kst[kTileKV * 8];  // K codes [token][kg][group] u16
  __shared__ __attribute__((aligned(16))) uint32_t kpr[kTileKV * 4];  // K params [token][group]
  __shared__ __attribute__((aligned(16))) float kst24[kTileKV * 4];   // K steps times 2^24 [token][group]
  __shared__ __attribute__((aligned(16))) uint32_t cst[kTileKV * 8];  // PSAC coefficients [token][16]
  auto vrow_off = [](int cl) { return cl * VROW + 32 * (cl >> 4); };  // local channel 0..63

  const int lane = threadIdx.x, j = lane & 15, kg = lane >> 4;
  // Workgroups go to the 8 XCDs in turn (dispatch id mod 8). Renumber them so
  // that each XCD receives one contiguous run of logical ids (Query blocks,
  // then splits, then heads): an XCD then serves a few heads, whose q . C
  // tables stay in its L2 (a bijection of the grid whatever the dispatch
  // order).
  int h, split, qblk;
  {
    const int nwg = (int)gridDim.x, bid = (int)blockIdx.x;
    const int per = nwg >> 3, rem = nwg & 7, xcd = bid & 7;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + (bid >> 3);
    const int nqb = (int)((a.nq + NQ - 1) / NQ);
    qblk = logical % nqb;
    const int hs = logical / nqb;
    split = hs % a.splits;
    h = hs / a.splits;
  }
  const int64_t q0 = (int64_t)qblk * NQ;
  // the softmax runs in the log2 domain with a positive factor; a negative
  // scale is carried by negated Queries (exact) and a negated q . C table
  const float qsign = (a.scale_log2 < 0.0f) ? -1.0f : 1.0f;
  const float cl2 = a.scale_log2 * qsign;

  const int T = p.tile_prefix[p.n_seg];
  const int tlo = (int)(((int64_t)T * split) / a.splits);
  const int thi = (int)(((int64_t)T * (split + 1)) / a.splits);

  // per-head bases; per-token offsets fit 32 bits (capacity <= 2^26)
  const uint8_t* kcode_h = a.cache.kcode + (size_t)h * a.cache.capP * (D / 4);
  const uint8_t* vcode_h = a.cache.vcode + (size_t)h * a.cache.capP * (D / 4);
  const uint32_t* kparam_h = a.cache.kparam + (size_t)h * a.cache.capP * NG;
  const uint32_t* vparam_h = a.cache.vparam + (size_t)h * a.cache.capP * NG;
  const uint8_t* ids_h = a.cache.ids + (size_t)h * a.cache.capP;
  const uint16_t* coef_h = a.cache.coef + (size_t)h * a.cache.capP * a.r;
  const float* qc_h = a.qc + (size_t)h * a.E * a.m * a.nqp;

  // ---- Query operands (fp16, exact for bf16 inputs): qa[G] holds Query
  // q0 + j, channels 32G + 8kg .. +7; qsum[G] = sum of the Query over group G
  half8 qa[NG];
  float qsum[NG];
  {
    const int64_t qi = q0 + j;
    const bool qv = qi < a.nq;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)h * a.nq + (qv ? qi : 0)) * D;
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      const uint4 w = *reinterpret_cast<const uint4*>(qrow + 32 * G + 8 * kg);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
      float s = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // channels 2k and 2k+1 of the octet go to the positions of the
        // spread code order (channel c at 2c for c < 4, at 2(c - 4) + 1)
        const float x0 = qv ? qsign * __uint_as_float(ww[k] << 16) : 0.0f;
        const float x1 = qv ? qsign * __uint_as_float(ww[k] & 0xFFFF0000u) : 0.0f;
        const int c0 = 2 * k, c1 = 2 * k + 1;
        qa[G][c0 < 4 ? 2 * c0 : 2 * (c0 - 4) + 1] = (_Float16)x0;
        qa[G][c1 < 4 ? 2 * c1 : 2 * (c1 - 4) + 1] = (_Float16)x1;
        s += x0;
        s += x1;
      }
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      qsum[G] = s;
    }
  }
  // [qsum_hi | qsum_lo] operand of the zero-point MFMA
  half8 ax2;
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    const _Float16 hi = (_Float16)qsum[G];
    const _Float16 lo = (_Float16)(qsum[G] - (float)hi);
    ax2[G] = (kg == 0) ? hi : (kg == 1) ? lo : (_Float16)0.0f;
    ax2[G + 4] = (_Float16)0.0f;
  }
  half8 ax1;  // [qU_hi | qU_lo] of the current epoch
  int cur_ep = -2;

  floatx4 O[D / 16];  // o[Query 4kg + v][channel 16cb + j]
  float mrow[4], lrow[4];
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) O[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  floatx4 Zs = {0.f, 0.f, 0.f, 0.f};  // zero-point term: [Query 4kg + v][group j], groups 0..3
  for (int e = lane; e < 12 * ZROW; e += 64) zt[4 * ZROW + e] = (_Float16)0.0f;  // rows 4..15 stay zero
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    mrow[v] = -__builtin_inff();
    lrow[v] = 0.0f;
  }
  const half2v one2 = {(_Float16)1.0f, (_Float16)1.0f};
  uint32_t cmask[8];  // wave-uniform: word s2 holds coefficients 2s2, 2s2+1
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) cmask[s2] = (2 * s2 < a.r) ? 0xFFFFFFFFu : 0u;

  // Token indices are clamped into the tile, so every load is unconditional.
  auto load_raw = [&](DecRaw& r, const TileInfo& ti) {
    const uint32_t t = (uint32_t)ti.tstart + (uint32_t)(lane < ti.tcount ? lane : ti.tcount - 1);
    r.id = ids_h[t];
    const uint4* kc = reinterpret_cast<const uint4*>(kcode_h) + t * 2u;
    r.k0 = kc[0];
    r.k1 = kc[1];
    r.kp = reinterpret_cast<const uint4*>(kparam_h)[t];
    // r is even: 4-byte aligned rows; halves past r are dropped when staged
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(coef_h) + t * ((uint32_t)a.r >> 1);
    r.c0 = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    r.c1 = make_uint4(cw[4], cw[5], cw[6], cw[7]);
    // (unsigned 32-bit element offsets from the uniform per-head bases: the
    // loads then take a VGPR offset against an SGPR base, no 64-bit adds)
    const uint32_t ukg = (uint32_t)kg;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int tt = 16 * tb + j;
      const uint32_t tv = (uint32_t)ti.tstart + (uint32_t)(tt < ti.tcount ? tt : ti.tcount - 1);
      // group 2P + kg / 2, channels 16 (kg & 1) .. : code word 4 kg + 16 P of
      // the token's 32-byte row, parameter word 4 tv + 2P + kg / 2
      const uint32_t* vrow = reinterpret_cast<const uint32_t*>(vcode_h) + (tv * (uint32_t)(D / 16) + ukg);
      const uint32_t* prow = vparam_h + (tv * (uint32_t)NG + (ukg >> 1));
#pragma unroll
      for (int P = 0; P < 2; ++P) {
        r.vc[tb][P] = vrow[4 * P];
        r.vp[tb][P] = prow[2 * P];
      }
    }
  };
  // q . C of the lane's 4 Queries (4kg .. +3) and token 16tb + j; -inf for
  // the token slots past the end of a segment's last tile, so that their
  // logits are -inf (the other terms are finite)
  auto load_qc = [&](floatx4 (&dst)[4], const TileInfo& ti, uint32_t id_lane) {
    const float* base = qc_h + (size_t)ti.ep * a.m * a.nqp + q0 + 4 * kg;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const uint32_t id = (uint32_t)__shfl((int)id_lane, 16 * tb + j);
      const float4 x = *reinterpret_cast<const float4*>(base + id * (uint32_t)a.nqp);
      dst[tb] = floatx4{x.x, x.y, x.z, x.w};
    }
    if (ti.tcount < kTileKV) {  // wave-uniform
      // (keeps this rare branch a branch: the selects would otherwise run
      // on every tile)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        if (16 * tb + j >= ti.tcount)
          dst[tb] = floatx4{-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
    }
  };
  // Values of one channel pass: 16 channels of 4 tokens (slots 4j + tb)
  // as code * s (exact fp16). The tokens go in pairs (tb 0, 1) and (2, 3):
  // one byte permute puts both tokens' codes of 8 channels into one word
  // (the first token's channel c in bits 2c, the second's in 16 + 2c), so
  // each channel's fp16 pair is already the two slots' values of its row.
  auto dequant_v = [&](const uint32_t (&vc)[4], const uint32_t (&vp)[4]) {
    const CodeScale cs01 = code_scale(__builtin_amdgcn_perm(vp[1], vp[0], 0x07060302u));
    const CodeScale cs23 = code_scale(__builtin_amdgcn_perm(vp[3], vp[2], 0x07060302u));
    const int clb = 32 * (kg >> 1) + 16 * (kg & 1);  // first local channel
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {  // channels clb + 8 hh .. +7
      const uint32_t sel = hh ? 0x07060302u : 0x05040100u;
      const uint32_t z01 = __builtin_amdgcn_perm(vc[1], vc[0], sel), z23 = __builtin_amdgcn_perm(vc[3], vc[2], sel);
      uint32_t x01[8], x23[8], w01[8], w23[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        x01[c] = z01 >> (2 * c);
        x23[c] = z23 >> (2 * c);
      }
      code_pairs(x01, cs01, w01);
      code_pairs(x23, cs23, w23);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<uint2*>(vt + vrow_off(clb + 8 * hh + c) + 4 * j) = make_uint2(w01[c], w23[c]);
    }
  };
  // Zero-points of the 4 tokens (slots 4j + tb) of the lane's group into row
  // `grow` of the zero-point plane (lanes of the first half of each group).
  auto store_zp = [&](const uint32_t (&vp)[4], int grow) {
    if ((kg & 1) == 0)
      *reinterpret_cast<uint2*>(zt + grow * ZROW + 4 * j) =
          make_uint2((vp[0] & 0xFFFFu) | (vp[1] << 16), (vp[2] & 0xFFFFu) | (vp[3] << 16));
  };
  // o += P (code * s) for the 64 channels of pass P; in pass 0 also the
  // zero-point term of all four groups
  auto pv_pass = [&](int P) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const half8 pa = *reinterpret_cast<const half8*>(pt + j * PROW + 32 * ks + 8 * kg);
#pragma unroll
      for (int cbl = 0; cbl < 4; ++cbl) {
        const int off = vrow_off(16 * cbl + j) + 32 * ks + 8 * kg;
        const half8 vv = *reinterpret_cast<const half8*>(vt + off);
        O[4 * P + cbl] = mfma_f16(pa, vv, O[4 * P + cbl]);
      }
      if (P == 0) {
        const half8 vz = *reinterpret_cast<const half8*>(zt + j * ZROW + 32 * ks + 8 * kg);
        Zs = mfma_f16(pa, vz, Zs);
      }
    }
  };

  // One tile: `cur` holds its raw words and qcc its q . C values. Once the
  // K words are staged and the V words copied out, `cur` is refilled with
  // the next tile's words; its q . C values are gathered at the end (their
  // ids have arrived by then).
  int sg = 0;  // segment cursor of the tiles visited
  auto process = [&](int tile, DecRaw& cur, floatx4 (&qcc)[4], TileInfo& tinfo) {
    const TileInfo ti = tinfo;
    // ---- stage the K words: codes permuted to [token][kg][group] so a lane
    // reads the 4 groups of its channel octet in one 8-byte read
    {
      const uint32_t ow[8] = {cur.k0.x, cur.k0.y, cur.k0.z, cur.k0.w, cur.k1.x, cur.k1.y, cur.k1.z, cur.k1.w};
      uint32_t nw[8];
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          // octet d of groups 2s and 2s+1 (u16 index 4G + d of the row)
          const uint32_t lo = ow[4 * s + d / 2], hi = ow[4 * s + 2 + d / 2];
          nw[2 * d + s] = __builtin_amdgcn_perm(hi, lo, (d & 1) ? 0x07060302u : 0x05040100u);
        }
      uint4* ks4 = reinterpret_cast<uint4*>(kst + lane * 8);
      ks4[0] = make_uint4(nw[0], nw[1], nw[2], nw[3]);
      ks4[1] = make_uint4(nw[4], nw[5], nw[6], nw[7]);
      *reinterpret_cast<uint4*>(kpr + lane * 4) = cur.kp;
      // the steps times 2^24 (exact in float32), once per token
      *reinterpret_cast<float4*>(kst24 + lane * 4) =
          make_float4(half_bits_to_float(cur.kp.x >> 16) * 16777216.0f, half_bits_to_float(cur.kp.y >> 16) * 16777216.0f,
                      half_bits_to_float(cur.kp.z >> 16) * 16777216.0f, half_bits_to_float(cur.kp.w >> 16) * 16777216.0f);
      uint4* cs4 = reinterpret_cast<uint4*>(cst + lane * 8);
      cs4[0] = make_uint4(cur.c0.x & cmask[0], cur.c0.y & cmask[1], cur.c0.z & cmask[2], cur.c0.w & cmask[3]);
      cs4[1] = make_uint4(cur.c1.x & cmask[4], cur.c1.y & cmask[5], cur.c1.z & cmask[6], cur.c1.w & cmask[7]);
    }
    uint32_t vc1[4], vp1[4];  // pass 1 words, kept while `cur` is refilled
    {
      uint32_t vc0[4], vp0[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        vc0[tb] = cur.vc[tb][0];
        vp0[tb] = cur.vp[tb][0];
        vc1[tb] = cur.vc[tb][1];
        vp1[tb] = cur.vp[tb][1];
      }
      dequant_v(vc0, vp0);
      store_zp(vp0, kg >> 1);      // groups 0, 1
      store_zp(vp1, 2 + (kg >> 1));  // groups 2, 3 (their codes are staged in pass 1)
    }
    // Prefetch without branches (indices clamped to the last tile): a load on
    // one path only would make the next wait cover every load in flight.
    const TileInfo tn = tile_info(p, tile + 1 < thi ? tile + 1 : thi - 1, sg);
    load_raw(cur, tn);
    wave_sync();

    // ---- PSAC Query operand of this epoch: lanes kg < 2 hold qU_hi, kg >= 2 qU_lo
    if (ti.ep != cur_ep) {
      cur_ep = ti.ep;
      const int64_t qi = q0 + j;
      if (qi < a.nq && a.r > 0) {
        const float* src = a.qU + (((int64_t)h * a.E + cur_ep) * a.nq + qi) * kRankPad + 8 * (kg & 1);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const float x = qsign * src[s2];
          const _Float16 hi = (_Float16)x;
          ax1[s2] = (kg < 2) ? hi : (_Float16)(x - (float)hi);
        }
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) ax1[s2] = (_Float16)0.0f;
      }
    }

    // ---- logits: D[Query 4kg + v][token 16tb + j]
    floatx4 S[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int tt = 16 * tb + j;
      const uint2 cw = *reinterpret_cast<const uint2*>(kst + tt * 8 + 2 * kg);
      const uint4 kp = *reinterpret_cast<const uint4*>(kpr + tt * 4);
      const float4 st4 = *reinterpret_cast<const float4*>(kst24 + tt * 4);
      const float st[4] = {st4.x, st4.y, st4.z, st4.w};
      const uint4 cf = *reinterpret_cast<const uint4*>(cst + tt * 8 + 4 * (kg & 1));
      // zero-points of groups 0..3 at k = 8kg + G; ax2 is zero for k = 8kg + 4..7
      // and for kg >= 2, where the (finite) repeats below meet zeros
      const uint32_t z01 = __builtin_amdgcn_perm(kp.y, kp.x, 0x05040100u);
      const uint32_t z23 = __builtin_amdgcn_perm(kp.w, kp.z, 0x05040100u);
      const half8 bzp = __builtin_bit_cast(half8, make_uint4(z01, z23, z01, z23));
      floatx4 acc = mfma_f16(ax1, __builtin_bit_cast(half8, cf), floatx4{0.f, 0.f, 0.f, 0.f});
      acc = mfma_f16(ax2, bzp, acc);
      const uint32_t cws[4] = {spread_unit(cw.x, 0x0C010C00u), spread_unit(cw.x, 0x0C030C02u),
                               spread_unit(cw.y, 0x0C010C00u), spread_unit(cw.y, 0x0C030C02u)};
      // q_G . (code_G * 2^-24), exact in float32; the step carries the 2^24.
      // The four MFMAs go first, so that each result has arrived when its
      // multiply-adds start.
      floatx4 dg[NG];
#pragma unroll
      for (int G = 0; G < NG; ++G) dg[G] = mfma_f16(qa[G], codes_to_f16_sub(cws[G]), floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int G = 0; G < NG; ++G)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(st[G], dg[G][v], acc[v]);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += qcc[tb][v];  // the table carries the sign (and the mask)
      S[tb] = acc;
    }

    // ---- online softmax (log2 domain); the running max is raised only when
    // a row's max exceeds it by more than 8, so the rescale of O is rare. A
    // lane sees from its own 4 logits whether its row rises; the 16 lanes of
    // a row exchange maxima only then (wave-uniform branch).
    bool raise_any = false;
    float lmx[4];
    const float inf = opaque_inf();
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      lmx[v] = max2(max2(S[0][v], S[1][v], inf), max2(S[2][v], S[3][v], inf), inf);
      raise_any |= lmx[v] * cl2 > mrow[v] + 8.0f;
    }
    if (__builtin_amdgcn_ballot_w64(raise_any)) {
      // (keeps the lane exchanges inside this rare branch)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float mx = row16_max(lmx[v], inf) * cl2;
        const float mnew = mx > mrow[v] + 8.0f ? mx : mrow[v];
        const float alpha = (mrow[v] == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(mrow[v] - mnew);
        mrow[v] = mnew;
        lrow[v] *= alpha;
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) O[cb][v] *= alpha;
        Zs[v] *= alpha;
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float nm = (mrow[v] == -__builtin_inff()) ? 0.0f : -mrow[v];
      float pv[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) pv[tb] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[tb][v], cl2, nm));
      const half2v p0 = pk_f16(pv[0], pv[1]), p1 = pk_f16(pv[2], pv[3]);
      float l = lrow[v];
      l = __builtin_amdgcn_fdot2(p0, one2, l, false);
      l = __builtin_amdgcn_fdot2(p1, one2, l, false);
      lrow[v] = l;
      *reinterpret_cast<half4*>(pt + (4 * kg + v) * PROW + 4 * j) = half4{p0[0], p0[1], p1[0], p1[1]};
    }
    wave_sync();
    pv_pass(0);
    wave_sync();
    dequant_v(vc1, vp1);
    wave_sync();
    pv_pass(1);
    wave_sync();
    load_qc(qcc, tn, cur.id);
    tinfo = tn;
  };

  DecRaw rw;
  floatx4 qcv[4];
  if (tlo < thi) {
    TileInfo ti = tile_info(p, tlo, sg);
    load_raw(rw, ti);
    load_qc(qcv, ti, rw.id);
    for (int tile = tlo; tile < thi; ++tile) process(tile, rw, qcv, ti);
  }

  // ---- epilogue: row sums over the 16 token lanes; normalized output or a
  // split partial (o, running max, row sum) for the merge
  // the zero-point term: group G of Query 4kg + v sits in lane (kg, G)
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float zg[4];
#pragma unroll
    for (int G = 0; G < 4; ++G) zg[G] = __shfl(Zs[v], 16 * kg + G);
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) O[cb][v] += zg[cb >> 1];
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float l = row16_sum(lrow[v]);
    const int64_t qi = q0 + 4 * kg + v;
    if (qi >= a.nq) continue;
    if (a.splits == 1) {
      const float inv = 1.0f / l;
      float* dst = a.out + ((int64_t)h * a.nq + qi) * D + j;
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) dst[16 * cb] = O[cb][v] * inv;
    } else {
      const int64_t row = ((int64_t)split * a.H + h) * a.nq + qi;
      float* dst = a.part_o + row * D + j;
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) dst[16 * cb] = O[cb][v];
      if (j == 0) {
        a.part_ml[row * 2] = mrow[v];
        a.part_ml[row * 2 + 1] = l;
      }
    }
  }
}

}  // namespace

hipError_t launch_qc(const void* q, int64_t nq, int nqp, const void* Cbase, int64_t epoch_C_stride, int H, int m,
                     int E, float sign, float* qc, hipStream_t s) {
  dim3 grid((unsigned)(nqp / 16), (unsigned)((m + 15) / 16), (unsigned)(H * E)), block(64);
  hipLaunchKernelGGL(qc_kernel, grid, block, 0, s, reinterpret_cast<const uint16_t*>(q), nq, nqp,
                     reinterpret_cast<const uint16_t*>(Cbase), epoch_C_stride, H, m, sign, qc);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, const AttnPlan& p, hipStream_t s) {
  const int64_t nwg = (a.nq + kDecodeQ - 1) / kDecodeQ * a.splits * a.H;
  if (nwg <= 0 || nwg > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)nwg), block(64);
  hipLaunchKernelGGL(decode_kernel<kDecodeQ>, grid, block, 0, s, a, p);
  return hipGetLastError();
}

}  // namespace qwm
