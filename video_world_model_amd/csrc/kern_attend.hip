// Attention over the 2-bit QuantWM cache with PSAC logit compensation (gfx950).
//
// Method (QuantWM; fugumt.com abstract: PSAC "restores the remaining Key
// errors along the dominant Query subspace ... to stabilize attention
// logits"; roboind.com "Step 2"): for cached token j of epoch e(j)
//   l_ij = (q_i . khat_j + (q_i U_r^(e(j))) . coef_j) * scale,
//   khat_j = c_id(j) + zp + code * step   (per 32-channel group),
// plus optional full-precision self tokens of the attending chunk; softmax
// over all visible tokens and o_i = sum_j p_ij vhat_j.
//
// Mapping to CDNA4:
//  * one workgroup = 8 waves = 256 Queries of one head, one split of the KV
//    sequence; the KV sequence is walked in 64-token tiles that never cross an
//    epoch boundary or the cache/self boundary;
//  * each tile is dequantized ONCE per workgroup into LDS (shared by the 8
//    waves; waves 0-3 build khat, waves 4-7 build vhat^T): khat as float16 hi + lo pairs (hi = fp16(x), lo = fp16(x - hi),
//    22 significant bits), the r PSAC coefficients next to them, and vhat^T
//    as hi + lo;
//  * logits come from v_mfma_f32_16x16x32_f16 with the contraction dimension
//    [khat_hi | khat_lo | coef] x [q | q | qU_hi, qU_lo]: one MFMA chain per
//    16x16 block computes q.khat and the PSAC term together;
//  * online softmax in float32 with cross-lane max/sum over the 4 lane groups
//    that share a Query (shuffles), P in fp16, o += vhat^T P^T by MFMA with
//    vhat hi and lo.
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
};

__device__ __forceinline__ floatx4 mfma16(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
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

__device__ __forceinline__ void split_hilo(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

template <int D, int DT, bool LOGITS>
__global__ __launch_bounds__(kAttnThreads) void attend_kernel(const AttnArgs a, const AttnPlan p) {
  using Sh = AttnShape<D>;
  constexpr int KS = Sh::KS, KROW = Sh::KROW, VROW = Sh::VROW, NG = Sh::NG;
  constexpr bool QLO = (DT == 1);  // float32 Queries also carry a lo part
  constexpr int VSZ = LOGITS ? 8 : D * VROW;
  constexpr int KITEMS = kTileKV * NG;               // (token, group) items of the khat tile
  constexpr int VITEMS = (kTileKV / 4) * (D / 8);    // (4-token quad, 8-channel octet) items
  constexpr int VBASE = kAttnThreads / 2;            // threads [VBASE, VBASE + VITEMS) dequantize V
  static_assert(KITEMS <= VBASE && VITEMS <= kAttnThreads - VBASE, "dequant items must fit one pass");
  __shared__ __attribute__((aligned(16))) _Float16 Ks[kTileKV * KROW];
  __shared__ __attribute__((aligned(16))) _Float16 Vh[VSZ];
  __shared__ __attribute__((aligned(16))) _Float16 Vl[VSZ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int h = LOGITS ? a.logit_head : (int)blockIdx.z;
  const int split = blockIdx.y;
  const int64_t qw0 = (int64_t)blockIdx.x * kTileQ + wave * 32;
  const bool wave_live = qw0 < a.nq;  // waves whose 32 Queries are all padding skip the math

  const int T = p.tile_prefix[p.n_seg];
  const int tlo = (int)(((int64_t)T * split) / a.splits);
  const int thi = (int)(((int64_t)T * (split + 1)) / a.splits);

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
      for (int s = 0; s < 8; ++s) {
        const float xv = qv ? x[s] : 0.0f;
        _Float16 hi, lo;
        split_hilo(xv, hi, lo);
        qh[qb][ks][s] = hi;
        if constexpr (QLO) ql[qb][ks][s] = lo;
      }
    }
  }
  half8 qu[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int s = 0; s < 8; ++s) qu[qb][s] = (_Float16)0.0f;
  int cur_epoch = -2;

  floatx4 O[2][D / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) O[qb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-__builtin_inff(), -__builtin_inff()};
  float lrow[2] = {0.0f, 0.0f};

  for (int tile = tlo; tile < thi; ++tile) {
    int sg = 0;
    while (p.tile_prefix[sg + 1] <= tile) ++sg;
    const int ep = p.seg_epoch[sg];
    const int tstart = p.seg_start[sg] + (tile - p.tile_prefix[sg]) * kTileKV;
    const int tend = p.seg_start[sg] + p.seg_len[sg];
    const int tcount = (tend - tstart) < kTileKV ? (tend - tstart) : kTileKV;

    __syncthreads();  // previous tile's LDS reads are complete
    if (tid < KITEMS) {
      // ---- khat row segment: item = (token t = it % 64, group G = it / 64); a wave
      // writes 64 consecutive rows of one group (row pitch 140 dwords spreads
      // 16 rows over all 64 banks).
      const int t = tid % kTileKV, G = tid / kTileKV;
      _Float16* row = Ks + t * KROW;
      half8 hv[4], lv[4];
      if (t < tcount) {
        float x[32];
        if (ep >= 0) {
          const int64_t slot = (int64_t)h * a.cache.capP + tstart + t;
          const uint2 cw = *reinterpret_cast<const uint2*>(a.cache.kcode + slot * (D / 4) + 8 * G);
          const uint32_t pr = a.cache.kparam[slot * NG + G];
          const float zpf = half_bits_to_float(pr & 0xFFFFu), scf = half_bits_to_float(pr >> 16);
          const int id = a.cache.ids[slot];
          const void* Cb = reinterpret_cast<const char*>(a.Cbase) + (int64_t)ep * a.epoch_C_stride;
          load_span<DT, 32>(Cb, ((int64_t)h * a.m + id) * D + 32 * G, x);
#pragma unroll
          for (int j = 0; j < 32; ++j) {
            const uint32_t w = j < 16 ? cw.x : cw.y;
            const float code = (float)((w >> (2 * (j & 15))) & 3u);
            x[j] = x[j] + __builtin_fmaf(code, scf, zpf);  // zp + code*step: the product is exact
          }
        } else {
          load_span<DT, 32>(a.kself, ((int64_t)h * a.nself + tstart + t) * D + 32 * G, x);
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          _Float16 hi, lo;
          split_hilo(x[j], hi, lo);
          hv[j >> 3][j & 7] = hi;
          lv[j >> 3][j & 7] = lo;
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            hv[u][s] = (_Float16)0.0f;
            lv[u][s] = (_Float16)0.0f;
          }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        *reinterpret_cast<half8*>(row + 32 * G + 8 * u) = hv[u];
        *reinterpret_cast<half8*>(row + D + 32 * G + 8 * u) = lv[u];
      }
      if (G == 0) {
        half8 c0, c1;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          c0[s] = (_Float16)0.0f;
          c1[s] = (_Float16)0.0f;
        }
        if (t < tcount && ep >= 0) {
          const int64_t slot = (int64_t)h * a.cache.capP + tstart + t;
          const uint16_t* cf = a.cache.coef + slot * a.r;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            if (s < a.r) c0[s] = (_Float16)half_bits_to_float(cf[s]);
            if (s + 8 < a.r) c1[s] = (_Float16)half_bits_to_float(cf[s + 8]);
          }
        }
        *reinterpret_cast<half8*>(row + 2 * D) = c0;
        *reinterpret_cast<half8*>(row + 2 * D + 8) = c1;
      }
    }
    if constexpr (!LOGITS) {
      if (tid >= VBASE && tid < VBASE + VITEMS) {
        // ---- vhat^T: item = (quad tq = it % 16, octet co = it / 16); the 16 quads
        // of a wave land on 16 different bank pairs of each row.
        const int it = tid - VBASE;
        const int tq = it % (kTileKV / 4), co = it / (kTileKV / 4);
        half4 vh4[8], vl4[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = 4 * tq + u;
          float x[8];
          if (t < tcount) {
            if (ep >= 0) {
              const int64_t slot = (int64_t)h * a.cache.capP + tstart + t;
              const uint32_t cw = *reinterpret_cast<const uint16_t*>(a.cache.vcode + slot * (D / 4) + 2 * co);
              const uint32_t pr = a.cache.vparam[slot * NG + (co >> 2)];
              const float zpf = half_bits_to_float(pr & 0xFFFFu), scf = half_bits_to_float(pr >> 16);
#pragma unroll
              for (int s = 0; s < 8; ++s) x[s] = __builtin_fmaf((float)((cw >> (2 * s)) & 3u), scf, zpf);
            } else {
              load_span<DT, 8>(a.vself, ((int64_t)h * a.nself + tstart + t) * D + 8 * co, x);
            }
          } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) x[s] = 0.0f;
          }
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            _Float16 hi, lo;
            split_hilo(x[s], hi, lo);
            vh4[s][u] = hi;
            vl4[s][u] = lo;
          }
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          *reinterpret_cast<half4*>(Vh + (8 * co + s) * VROW + 4 * tq) = vh4[s];
          *reinterpret_cast<half4*>(Vl + (8 * co + s) * VROW + 4 * tq) = vl4[s];
        }
      }
    }
    __syncthreads();
    if (!wave_live) continue;

    // ---- per-epoch PSAC Query fragment: lanes g<2 hold qU_hi, g>=2 qU_lo
    if (ep != cur_epoch) {
      cur_epoch = ep;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int64_t qi = qw0 + 16 * qb + l16;
        if (ep >= 0 && qi < a.nq) {
          const float* src = a.qU + (((int64_t)h * a.n_epoch_slots + ep) * a.nq + qi) * kRankPad + 8 * (g & 1);
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            _Float16 hi, lo;
            split_hilo(src[s], hi, lo);
            qu[qb][s] = (g < 2) ? hi : lo;
          }
        } else {
#pragma unroll
          for (int s = 0; s < 8; ++s) qu[qb][s] = (_Float16)0.0f;
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
    for (int ks = 0; ks < KS; ++ks)
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
        if (qi >= a.nq) continue;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int j = 16 * tb + 4 * g + v;
            if (j < tcount) a.logits[qi * a.logit_len + tstart + j] = S[qb][tb][v] * a.scale;
          }
      }
      continue;
    } else {
      // ---- online softmax (log2 domain). The running max is only raised when
      // a row's new max exceeds it by more than 8 (p <= 2^8 stays exact
      // enough in fp16 and float32), so the output rescale is rare.
      const bool full = (tcount == kTileKV) && !(ep < 0 && a.causal_self);
      half8 pf[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int64_t qi = qw0 + 16 * qb + l16;
        float sv[4][4];
        float mx = -__builtin_inff();
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float x = S[qb][tb][v] * a.scale_log2;
            if (!full) {
              const int j = 16 * tb + 4 * g + v;
              bool ok = j < tcount;
              if (ep < 0 && a.causal_self) ok = ok && ((int64_t)(tstart + j) <= qi);
              x = ok ? x : -__builtin_inff();
            }
            sv[tb][v] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool raise = mx > mrow[qb] + 8.0f;
        if (__ballot(raise)) {  // wave-uniform: rescale every lane (alpha = 1 where unchanged)
          const float mnew = raise ? mx : mrow[qb];
          const float alpha = (mrow[qb] == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(mrow[qb] - mnew);
          mrow[qb] = mnew;
          lrow[qb] *= alpha;
#pragma unroll
          for (int cb = 0; cb < D / 16; ++cb) O[qb][cb] *= alpha;
        }
        const float mcur = mrow[qb];
        const bool none = (mcur == -__builtin_inff());
        float ps = 0.0f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float pv = none ? 0.0f : __builtin_amdgcn_exp2f(sv[tb][v] - mcur);
            sv[tb][v] = pv;
            ps += pv;
          }
        lrow[qb] += ps;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            pf[qb][ks][v] = (_Float16)sv[2 * ks][v];
            pf[qb][ks][4 + v] = (_Float16)sv[2 * ks + 1][v];
          }
      }
      // ---- o^T += vhat^T P^T (tokens {4g..4g+3, 16+4g..16+4g+3} of each 32-token step)
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int off = (16 * cb + l16) * VROW + 32 * ks + 4 * g;
          const half4 h0 = *reinterpret_cast<const half4*>(Vh + off);
          const half4 h1 = *reinterpret_cast<const half4*>(Vh + off + 16);
          const half4 l0 = *reinterpret_cast<const half4*>(Vl + off);
          const half4 l1 = *reinterpret_cast<const half4*>(Vl + off + 16);
          const half8 ah = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
          const half8 al = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            O[qb][cb] = mfma16(ah, pf[qb][ks], O[qb][cb]);
            O[qb][cb] = mfma16(al, pf[qb][ks], O[qb][cb]);
          }
        }
    }
  }

  if constexpr (!LOGITS) {
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

// Log-sum-exp merge of the split-KV partials (log2 domain).
template <int D>
__global__ __launch_bounds__(D) void merge_kernel(const AttnArgs a) {
  const int64_t qi = blockIdx.x;
  const int h = blockIdx.y, c = threadIdx.x;
  float M = -__builtin_inff();
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.part_ml[(((int64_t)s * a.H + h) * a.nq + qi) * 2]);
  float L = 0.0f, o = 0.0f;
  for (int s = 0; s < a.splits; ++s) {
    const int64_t row = ((int64_t)s * a.H + h) * a.nq + qi;
    const float m = a.part_ml[row * 2];
    const float w = (m == -__builtin_inff()) ? 0.0f : exp2f(m - M);
    L += a.part_ml[row * 2 + 1] * w;
    o += a.part_o[row * D + c] * w;
  }
  a.out[((int64_t)h * a.nq + qi) * D + c] = o / L;
}

// q . U_r for every epoch slot: qU[h][e][i][k] (k < 16, zero for k >= r).
template <int D, int DT>
__global__ __launch_bounds__(256) void qu_kernel(const void* q, int64_t nq, int r, const float* Ubase,
                                                 int64_t ustride, int E, float* qU) {
  const int h = blockIdx.y, e = blockIdx.z;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t qi = idx / kRankPad;
  const int k = (int)(idx % kRankPad);
  if (qi >= nq) return;
  float acc = 0.0f;
  if (k < r) {
    const float* U = Ubase + (int64_t)e * ustride + (int64_t)h * D * r;
    const int64_t qb = ((int64_t)h * nq + qi) * D;
    for (int j = 0; j < D; ++j) acc = fmaf(load_in<DT>(q, qb + j), U[j * r + k], acc);
  }
  qU[(((int64_t)h * E + e) * nq + qi) * kRankPad + k] = acc;
}

}  // namespace

hipError_t launch_qu(int D, int dtype, const void* q, int64_t nq, int H, int r, const float* Ubase,
                     int64_t ustride, int E, float* qU, hipStream_t s) {
  dim3 grid((unsigned)((nq * kRankPad + 255) / 256), (unsigned)H, (unsigned)E), block(256);
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

template <bool LOGITS>
static hipError_t launch_attend_impl(int D, int dtype, const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  dim3 grid((unsigned)((a.nq + kTileQ - 1) / kTileQ), (unsigned)a.splits, LOGITS ? 1u : (unsigned)a.H);
  dim3 block(kAttnThreads);
  if (D == 128 && dtype == 0)
    hipLaunchKernelGGL((attend_kernel<128, 0, LOGITS>), grid, block, 0, s, a, p);
  else if (D == 128)
    hipLaunchKernelGGL((attend_kernel<128, 1, LOGITS>), grid, block, 0, s, a, p);
  else if (dtype == 0)
    hipLaunchKernelGGL((attend_kernel<64, 0, LOGITS>), grid, block, 0, s, a, p);
  else
    hipLaunchKernelGGL((attend_kernel<64, 1, LOGITS>), grid, block, 0, s, a, p);
  return hipGetLastError();
}

hipError_t launch_attend(int D, int dtype, const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  return launch_attend_impl<false>(D, dtype, a, p, s);
}
hipError_t launch_attend_logits(int D, int dtype, const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  return launch_attend_impl<true>(D, dtype, a, p, s);
}

hipError_t launch_merge(int D, const AttnArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.nq, (unsigned)a.H), block((unsigned)D);
  if (D == 128)
    hipLaunchKernelGGL((merge_kernel<128>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((merge_kernel<64>), grid, block, 0, s, a);
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
