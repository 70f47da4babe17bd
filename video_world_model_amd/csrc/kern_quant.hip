// QSAC quantize-on-insert, k-means centroid construction and epoch shadows
// for the QuantWM 2-bit KV cache (gfx950).
//
// Method (QuantWM, arXiv 2609.26425; roboind.com article "Step 1" and
// "Step 2", fugumt.com abstract): each Key is assigned the centroid that
// minimizes J = sum_G S_G (max_G r - min_G r)^2, r = k - c (or, for the QVG
// baseline of "Step 1", the squared distance |r|^2; or the weighted error the
// INT2 quantization of r actually leaves), the residual is
// stored as per-group asymmetric INT2 with fp16 zero-point/step, the Key's
// remaining error is projected on the PSAC basis (r fp16 coefficients), and
// the Value is stored as plain per-group INT2.
//
// Mapping to CDNA4: in the assignment one lane owns one token, so the
// objective and its running argmin run lane-sequentially in exactly the order
// of the definition. The centroid row being scored is the same for every lane
// of a wave; it is loaded through the scalar path (one copy per wave in
// SGPRs) and consumed as an SGPR operand of v_sub, so the candidate loop is
// pure VALU (sub, max3, min3). The four waves of a block split the candidate
// list of the same 64 tokens (see quantize_kernel). Builds use -ffp-contract=off so no multiply-add
// is fused: every float32 operation rounds exactly as in the definition.
#include "qwm_dev.h"
#include "qwm_internal.h"

namespace qwm {

namespace {

// QSAC objective of one candidate row (float32, fixed operation order):
// per group r = k - c, mx/mn, R = mx - mn, t = R*R, u = S_G*t, J = ((u0+u1)+u2)+...
// (R is unaffected by the sign of a zero max/min, so no folding is needed here.)
template <int D>
__device__ __forceinline__ float qsac_cost(const float (&kf)[D], const float* __restrict__ crow,
                                           const float (&SG)[D / kGroup]) {
  constexpr int NG = D / kGroup;
  float J = 0.0f;
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    const float r0 = kf[G * kGroup] - crow[G * kGroup];
    float mx = r0, mn = r0;
#pragma unroll
    for (int j = 1; j < kGroup; ++j) {
      const float r = kf[G * kGroup + j] - crow[G * kGroup + j];
      mx = fmaxf(mx, r);
      mn = fminf(mn, r);
    }
    const float R = mx - mn;
    const float t = R * R;
    const float u = SG[G] * t;
    J = (G == 0) ? u : J + u;
  }
  return J;
}

// QVG's nearest-centroid cost (float32, fixed order): per group the running
// sum p_G = t_0 + t_1 + ... of t_j = r_j * r_j over the channels in ascending
// order, then D = ((p_0 + p_1) + p_2) + ...
template <int D>
__device__ __forceinline__ float nearest_cost(const float (&kf)[D], const float* __restrict__ crow) {
  constexpr int NG = D / kGroup;
  float J = 0.0f;
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    const float r0 = kf[G * kGroup] - crow[G * kGroup];
    float p = r0 * r0;
#pragma unroll
    for (int j = 1; j < kGroup; ++j) {
      const float r = kf[G * kGroup + j] - crow[G * kGroup + j];
      const float t = r * r;
      p = p + t;
    }
    J = (G == 0) ? p : J + p;
  }
  return J;
}

// Smallest fp16 s >= x whose triple is an fp16 value too, so that every
// offset code * s (code 0..3) is exactly an fp16 value (the attention kernels
// contract the codes times the step in fp16): round up, then at most three
// one-ulp steps upward while 3 s (exact in float32) is not an fp16 value.
__device__ __forceinline__ uint32_t f16_step_up(float x) {
  uint32_t b = f16_round_up(x);
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const float t = 3.0f * half_bits_to_float(b);
    if (half_bits_to_float(half_bits(__float2half_rn(t))) == t) break;
    b = f16_next_up(b);
  }
  return b;
}

// Per-group INT2 parameters (signed zeros folded to +0):
// zp = largest fp16 <= min, step = smallest fp16 >= (max - zp) / 3 whose
// triple is an fp16 value.
__device__ __forceinline__ void int2_params(float mn, float mx, uint32_t& zpb, uint32_t& scb, float& zpf,
                                            float& scf) {
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  zpb = f16_round_down(mn);
  zpf = half_bits_to_float(zpb);
  const float step = (mx - zpf) / 3.0f;  // correctly rounded divide
  scb = f16_step_up(step);
  scf = half_bits_to_float(scb);
}

// code = clamp(rint((x - zp) / step), 0, 3); a zero step gives 0.
__device__ __forceinline__ uint32_t int2_code(float x, float zpf, float scf) {
  if (scf == 0.0f) return 0u;
  float y = (x - zpf) / scf;  // correctly rounded divide
  y = rintf(y);               // nearest, ties to even
  y = fminf(fmaxf(y, 0.0f), 3.0f);
  return (uint32_t)y;
}

// The same codes without a divide per value: rcs = v_rcp_f32(step) is within
// 1 ulp of 1/step, so for quotients below 4 the product (x - zp) * rcs lies
// within 1e-6 of the correctly rounded quotient, and both round to the same
// integer unless the product is within 4e-6 of a half-integer (0.5, 1.5, 2.5
// decide the code; quotients past 3.5 or below -0.5 clamp the same either
// way). Such values take the exact divide. A zero step has rcs = 0: the
// product is 0 and so is the code.
__device__ __forceinline__ float rcp_step(float scf) { return scf == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(scf); }
// The codes (as floats 0..3) of a whole group, with one wave-uniform check
// for the group instead of one per value (each check is a branch): only when
// some lane holds a value that close to a boundary are that lane's boundary
// values redone with the correctly rounded divide.
template <int N>
__device__ __forceinline__ void int2_codes_rcp(const float (&x)[N], float zpf, float scf, float (&code)[N]) {
  const float rcs = rcp_step(scf);
  bool anynear = false;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float qa = (x[j] - zpf) * rcs;
    const float rq = rintf(qa);
    anynear = anynear | (fabsf(qa - rq) > 0.5f - 4e-6f);
    code[j] = fminf(fmaxf(rq, 0.0f), 3.0f);
  }
  if (__builtin_expect(__any(anynear), 0)) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float qa = (x[j] - zpf) * rcs;
      if (fabsf(qa - rintf(qa)) > 0.5f - 4e-6f) code[j] = (float)int2_code(x[j], zpf, scf);
    }
  }
}

// Weighted error left by the INT2 quantization of r = k - c (float32, fixed
// order): per group the quantizer of the cache (zero-point, step, codes),
// e_j = r_j - (zp + code_j * step), E = t_0 + t_1 + ... of t_j = e_j * e_j,
// u = S_G * E, J = ((u0 + u1) + u2) + ...
template <int D>
__device__ __forceinline__ float postq_cost(const float (&kf)[D], const float* __restrict__ crow,
                                            const float (&SG)[D / kGroup]) {
  constexpr int NG = D / kGroup;
  float J = 0.0f;
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    float r[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) r[j] = kf[G * kGroup + j] - crow[G * kGroup + j];
    float mx = r[0], mn = r[0];
#pragma unroll
    for (int j = 1; j < kGroup; ++j) {
      mx = fmaxf(mx, r[j]);
      mn = fminf(mn, r[j]);
    }
    uint32_t zpb, scb;
    float zpf, scf;
    int2_params(mn, mx, zpb, scb, zpf, scf);
    float code[kGroup];
    int2_codes_rcp(r, zpf, scf, code);
    float E = 0.0f;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const float rhat = zpf + code[j] * scf;  // the product is exact
      const float e = r[j] - rhat;
      const float t = e * e;
      E = (j == 0) ? t : E + t;
    }
    const float u = SG[G] * E;
    J = (G == 0) ? u : J + u;
  }
  return J;
}

// Term of group G in the assignment cost of the chosen rule: the cost is
// ((u_0 + u_1) + u_2) + ... of these terms, all >= 0, so every partial sum is
// a lower bound of the full cost (float32 addition of non-negative numbers
// never decreases).
template <int OBJ, int D>
__device__ __forceinline__ float group_term(const float (&kf)[D], const float* __restrict__ crow, int G,
                                            const float (&SG)[D / kGroup]) {
  static_assert(OBJ != kObjPostq, "the post-rounding error is evaluated whole");
  const float r0 = kf[G * kGroup] - crow[G * kGroup];
  if constexpr (OBJ == kObjNearest) {
    float p = r0 * r0;
#pragma unroll
    for (int j = 1; j < kGroup; ++j) {
      const float r = kf[G * kGroup + j] - crow[G * kGroup + j];
      const float t = r * r;
      p = p + t;
    }
    return p;
  } else {
    float mx = r0, mn = r0;
#pragma unroll
    for (int j = 1; j < kGroup; ++j) {
      const float r = kf[G * kGroup + j] - crow[G * kGroup + j];
      mx = fmaxf(mx, r);
      mn = fminf(mn, r);
    }
    const float R = mx - mn;
    const float t = R * R;
    return SG[G] * t;
  }
}

// Assignment cost of the chosen rule: kObjQsac, kObjNearest or kObjPostq.
template <int OBJ, int D>
__device__ __forceinline__ float assign_cost(const float (&kf)[D], const float* __restrict__ crow,
                                             const float (&SG)[D / kGroup]) {
  if constexpr (OBJ == kObjNearest)
    return nearest_cost<D>(kf, crow);
  else if constexpr (OBJ == kObjPostq)
    return postq_cost<D>(kf, crow, SG);
  else
    return qsac_cost<D>(kf, crow, SG);
}

// N consecutive input elements (bf16 or float) -> float, 16-byte loads.
template <int N, int DT>
__device__ __forceinline__ void load_row_span(const void* base, int64_t off, float (&x)[N]) {
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

// Block = 4 waves, 64 tokens of one head.
//  phase 1: wave w scans candidates [w*mq, (w+1)*mq) for all 64 tokens (lane =
//           token), keeping its lexicographic (J, id) minimum;
//  phase 2: the four quarter minima are combined in candidate order (lower
//           quarter wins an exact tie), which equals the argmin over all
//           candidates with ties to the smallest id;
//  phase 3: one lane per (token, 32-channel group) quantizes the residual and
//           the Value group and forms the group's PSAC partial sums; the group
//           partials of a token are added in group order (lanes of a token are
//           adjacent), and all records are written with contiguous stores.
constexpr int kQTok = 64;

// PART 0: the whole kernel. For k-means passes over too few Keys to fill
// the device twice over, the centroid scan is split: PART 1 scans one half of the centroids
// (blockIdx.z) and writes each token's best (J, id) of that half to a.part;
// PART 2 takes the better of the two halves (the first on equal J, so the
// smallest id keeps a tie) and runs phases 3 and on.
template <int D, int DT, bool ASSIGN_ONLY, int OBJ, int PART>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  constexpr int NG = D / kGroup;
  __shared__ float bj[4][kQTok];
  __shared__ int bi[4][kQTok];
  // PSAC basis as [i][group][33]: the 4 group rows read together sit 2 banks apart
  constexpr int UGP = kGroup + 1;
  __shared__ double us[ASSIGN_ONLY ? 1 : kRankPad * NG * UGP];

  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: candidate rows load as scalars
  const int64_t t0 = (int64_t)blockIdx.x * kQTok;
  const int nt = (int)((a.n - t0) < kQTok ? (a.n - t0) : kQTok);

  // ---- phase 1: assignment cost over this wave's candidate quarter (of the
  // block's range). It runs before any barrier so that the wave-uniform
  // candidate rows are fetched with scalar loads (a barrier would make them
  // possibly clobbered).
  if constexpr (PART != 2) {
    float kf[D];
    load_row_span<D, DT>(a.k, ((int64_t)h * a.n + t0 + (lane < nt ? lane : 0)) * D, kf);
    float SG[NG];
#pragma unroll
    for (int G = 0; G < NG; ++G) SG[G] = a.S[h * NG + G];
    const int mh = (a.m + 1) / 2;  // PART 1: half 0 = [0, mh), half 1 = [mh, m)
    const int rb = (PART == 1 && blockIdx.z == 1) ? mh : 0;
    const int re = (PART == 1 && blockIdx.z == 0) ? mh : a.m;
    const int mq = (re - rb + 3) / 4;
    const int c0 = rb + wave * mq, c1 = (c0 + mq) < re ? (c0 + mq) : re;  // may be empty
    const float* __restrict__ Ch = a.C32 + (int64_t)h * a.m * D;
    float bestJ = __builtin_inff();
    int best = c0;
    for (int c = c0; c < c1; ++c) {
      const float J = assign_cost<OBJ, D>(kf, Ch + (int64_t)c * D, SG);
      if (J < bestJ) {  // strict: the smallest id keeps an exact tie
        bestJ = J;
        best = c;
      }
    }
    bj[wave][lane] = bestJ;
    bi[wave][lane] = best;
  }
  if constexpr (PART == 1) {
    __syncthreads();
    if (tid < nt) {
      float J = bj[0][tid];
      int id = bi[0][tid];
#pragma unroll
      for (int w = 1; w < 4; ++w)
        if (bj[w][tid] < J) {
          J = bj[w][tid];
          id = bi[w][tid];
        }
      a.part[((int64_t)blockIdx.z * a.H + h) * a.n + t0 + tid] = make_uint2(__float_as_uint(J), (uint32_t)id);
    }
    return;
  }
  if constexpr (!ASSIGN_ONLY) {
    const double* Uh = a.U64 + (int64_t)h * D * a.r;
    for (int i = tid; i < D * kRankPad; i += 256) {
      const int row = i / kRankPad, col = i % kRankPad;  // row = channel
      us[(col * NG + row / kGroup) * UGP + row % kGroup] = (col < a.r) ? Uh[row * a.r + col] : 0.0;
    }
  }
  __syncthreads();

  // ---- phase 2: combine the quarters (or the halves) in candidate order
  auto combined = [&](int t) {
    if constexpr (PART == 2) {
      // the scan wrote tokens below nt only: padding lanes of the last block
      // take the block's first token (their results are never stored)
      const int tc = t < nt ? t : 0;
      const uint2 p0 = a.part[(int64_t)h * a.n + t0 + tc];
      const uint2 p1 = a.part[((int64_t)a.H + h) * a.n + t0 + tc];
      return (int)((__uint_as_float(p1.x) < __uint_as_float(p0.x)) ? p1.y : p0.y);
    } else {
      float J = bj[0][t];
      int id = bi[0][t];
#pragma unroll
      for (int w = 1; w < 4; ++w)
        if (bj[w][t] < J) {
          J = bj[w][t];
          id = bi[w][t];
        }
      return id;
    }
  };
  if constexpr (ASSIGN_ONLY) {
    if (tid < nt) a.ids_out[(int64_t)h * a.n + t0 + tid] = (uint8_t)combined(tid);
    return;
  } else {
    // ---- phase 3: one lane per (token, group)
    if (tid >= kQTok * NG) return;  // no barrier below
    const int t = tid / NG, G = tid % NG;
    const bool valid = t < nt;
    const int best = combined(t);
    const int64_t slot = (int64_t)h * a.cache.capP + a.pos0 + t0 + t;
    const float* crow = a.C32 + ((int64_t)h * a.m + best) * D + G * kGroup;
    float c[kGroup], k[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; j += 4) {
      const float4 cv = *reinterpret_cast<const float4*>(crow + j);
      c[j] = cv.x;
      c[j + 1] = cv.y;
      c[j + 2] = cv.z;
      c[j + 3] = cv.w;
    }
    load_row_span<kGroup, DT>(a.k, ((int64_t)h * a.n + t0 + (valid ? t : 0)) * D + G * kGroup, k);
    float mx = k[0] - c[0], mn = mx;
#pragma unroll
    for (int j = 1; j < kGroup; ++j) {
      const float r = k[j] - c[j];
      mx = fmaxf(mx, r);
      mn = fminf(mn, r);
    }
    uint32_t zpb, scb;
    float zpf, scf;
    int2_params(mn, mx, zpb, scb, zpf, scf);
    float rr[kGroup], kc[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) rr[j] = k[j] - c[j];
    int2_codes_rcp(rr, zpf, scf, kc);
    uint32_t w0 = 0, w1 = 0;
    float e[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const uint32_t code = (uint32_t)kc[j];
      if (j < 16)
        w0 |= code << (2 * j);
      else
        w1 |= code << (2 * (j - 16));
      // PSAC error e = k - (c + rhat), rhat = zp + code*step (the product is exact).
      const float rhat = zpf + (float)code * scf;
      const float tsum = c[j] + rhat;
      e[j] = k[j] - tsum;
    }
    // coef_i = sum over the token's groups (in group order) of sum_j e_j U_ji,
    // each group's partial formed by its own lane in float64.
    uint16_t* cf = a.cache.coef + slot * a.r;
    for (int i = 0; i < a.r; ++i) {
      const double* urow = &us[(i * NG + G) * UGP];
      double part = 0.0;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) part = fma((double)e[j], urow[j], part);
      const double coef = group_ordered_sum<NG>(part);
      if (valid && (i % NG) == G) cf[i] = (uint16_t)f64_to_f16_bits(coef);
    }
    // Value group
    float v[kGroup];
    load_row_span<kGroup, DT>(a.v, ((int64_t)h * a.n + t0 + (valid ? t : 0)) * D + G * kGroup, v);
    float vmx = v[0], vmn = v[0];
#pragma unroll
    for (int j = 1; j < kGroup; ++j) {
      vmx = fmaxf(vmx, v[j]);
      vmn = fminf(vmn, v[j]);
    }
    uint32_t vzb, vsb;
    float vzf, vsf;
    int2_params(vmn, vmx, vzb, vsb, vzf, vsf);
    float vc[kGroup];
    int2_codes_rcp(v, vzf, vsf, vc);
    uint32_t u0 = 0, u1 = 0;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const uint32_t code = (uint32_t)vc[j];
      if (j < 16)
        u0 |= code << (2 * j);
      else
        u1 |= code << (2 * (j - 16));
    }
    if (!valid) return;
    *reinterpret_cast<uint2*>(a.cache.kcode + slot * (D / 4) + 8 * G) = make_uint2(w0, w1);
    *reinterpret_cast<uint2*>(a.cache.vcode + slot * (D / 4) + 8 * G) = make_uint2(u0, u1);
    a.cache.kparam[slot * NG + G] = zpb | (scb << 16);
    a.cache.vparam[slot * NG + G] = vzb | (vsb << 16);
    if (G == 0) a.cache.ids[slot] = (uint8_t)best;
  }
}

// k-means seeding: centroid i = key floor(i * n / m).
template <int D, int DT>
__global__ void seed_kernel(const void* keys, int64_t n, int m, void* C, float* C32) {
  const int i = blockIdx.x, h = blockIdx.y, j = threadIdx.x;
  const int64_t src = (int64_t)i * n / m;
  const int64_t si = ((int64_t)h * n + src) * D + j;
  const int64_t di = ((int64_t)h * m + i) * D + j;
  if constexpr (DT == 0)
    reinterpret_cast<uint16_t*>(C)[di] = reinterpret_cast<const uint16_t*>(keys)[si];
  else
    reinterpret_cast<float*>(C)[di] = reinterpret_cast<const float*>(keys)[si];
  C32[di] = load_in<DT>(keys, si);
}

// k-means update: one block of NW waves per (centroid, head) (8 for long
// builds, 2 for short ones, where many centroids each have few members and
// the block count, not the scan, sets the time). The head's ids are read as
// 16-byte blocks aligned in memory (the first block may begin before the
// head's first id and the last may end after its last; those bytes are
// masked). Wave w owns the block range [w*bs, (w+1)*bs), one block per lane
// and round; a wave prefix sum over the per-lane match counts lists the
// centroid's members in token order in LDS. Member Key rows are fetched
// kUpdRows at a time (each row by the whole wave, every load issued before
// the first is used) and added into float64 lane accumulators; the NW wave
// sums are then added in wave order. The mean is rounded once to the cache
// dtype; a centroid without members keeps its value. The order of every
// addition is fixed, so repeated runs give the same bits.
constexpr int kUpdRows = 8;  // member rows in flight per wave

template <int D, int DT, int NW>
__global__ __launch_bounds__(NW * 64) void update_kernel(const void* keys, const uint8_t* ids, int64_t n64, int m,
                                                         void* C, float* C32) {
  constexpr int PER = D / 64;  // channels per lane
  static_assert(NW * 64 >= D, "one thread per channel in the final sum");
  __shared__ uint16_t list[NW][64 * 16];
  __shared__ double red[NW][D];
  __shared__ int cnt[NW];
  const int n = (int)n64;  // n <= 2^22
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = blockIdx.x, h = blockIdx.y;
  uint16_t* lst = list[wave];
  // per-head bases (uniform); row offsets fit 32 bits
  const uint16_t* kh16 = reinterpret_cast<const uint16_t*>(keys) + (size_t)h * n * D;
  const float* kh32 = reinterpret_cast<const float*>(keys) + (size_t)h * n * D;
  const uint8_t* idh = ids + (size_t)h * n;
  const int sh = (int)(reinterpret_cast<uintptr_t>(idh) & 15u);  // id 0 sits at byte sh of block 0
  const uint4* blk = reinterpret_cast<const uint4*>(idh - sh);
  const int nb = (sh + n + 15) >> 4;
  const int bs = (nb + NW - 1) / NW;
  const int b0 = wave * bs, b1 = (b0 + bs < nb) ? b0 + bs : nb;

  double acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.0;
  int count = 0;
  for (int rb = b0; rb < b1; rb += 64) {  // wave-uniform
    const int bi = rb + lane;
    const uint4 w = blk[bi < b1 ? bi : rb];  // every lane loads; lanes past the range are masked below
    const int tb = 16 * rb - sh;             // token of byte 0 of the round's first block
    const int t0 = tb + 16 * lane;           // token of byte 0 of this lane's block
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    uint32_t match = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) match |= (uint32_t)(((ww[q] >> (8 * k)) & 0xFFu) == (uint32_t)c) << (4 * q + k);
    // bytes b with 0 <= t0 + b < n of a block inside the wave's range
    const int lo = t0 < 0 ? -t0 : 0;
    const int hi = (n - t0) < 16 ? (n - t0) : 16;
    const uint32_t keep = (bi < b1 && hi > lo) ? (((1u << hi) - 1u) & ~((1u << lo) - 1u)) : 0u;
    match &= keep;
    const int mc = __popc(match);
    int incl = mc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int total = __shfl(incl, 63);
    int pos = incl - mc;
    while (match) {
      const int b = __ffs(match) - 1;
      match &= match - 1;
      lst[pos++] = (uint16_t)(16 * lane + b);  // token tb + entry
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int u0 = 0; u0 < total; u0 += kUpdRows) {
      uint32_t row[kUpdRows];
#pragma unroll
      for (int u = 0; u < kUpdRows; ++u) {
        const int uu = (u0 + u < total) ? u0 + u : total - 1;
        row[u] = (uint32_t)(tb + lst[uu]) * (uint32_t)D + PER * lane;
      }
      float x[kUpdRows][PER];
#pragma unroll
      for (int u = 0; u < kUpdRows; ++u) {
        if constexpr (DT == 0) {
          if constexpr (PER == 2) {
            const uint32_t v = *reinterpret_cast<const uint32_t*>(kh16 + row[u]);
            x[u][0] = __uint_as_float(v << 16);
            x[u][1] = __uint_as_float(v & 0xFFFF0000u);
          } else {
            x[u][0] = __uint_as_float((uint32_t)kh16[row[u]] << 16);
          }
        } else {
          if constexpr (PER == 2) {
            const float2 v = *reinterpret_cast<const float2*>(kh32 + row[u]);
            x[u][0] = v.x;
            x[u][1] = v.y;
          } else {
            x[u][0] = kh32[row[u]];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kUpdRows; ++u)
        if (u0 + u < total) {
#pragma unroll
          for (int k = 0; k < PER; ++k) acc[k] += (double)x[u][k];
        }
    }
    count += total;
    // the list is rewritten next round: every lane must be done reading it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) red[wave][PER * lane + k] = acc[k];
  if (lane == 0) cnt[wave] = count;
  __syncthreads();
  if (threadIdx.x >= D) return;
  const int j = threadIdx.x;
  int total = 0;
  double sum = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    total += cnt[w];
    sum += red[w][j];
  }
  if (total == 0) return;
  const double mean = sum / (double)total;
  const int64_t di = ((int64_t)h * m + c) * D + j;
  if constexpr (DT == 0) {
    const uint32_t bb = f64_to_bf16_bits(mean);
    reinterpret_cast<uint16_t*>(C)[di] = (uint16_t)bb;
    C32[di] = bf16_bits_to_float(bb);
  } else {
    const float f = (float)mean;  // nearest-even
    reinterpret_cast<float*>(C)[di] = f;
    C32[di] = f;
  }
}

// ---- pruned k-means assignment (iterations after the first)
//
// sqrt(J) is a seminorm of r = k - c: each group range R_G is one (it is
// subadditive and absolutely homogeneous) and sqrt(sum_G S_G R_G^2) is a
// weighted 2-norm of them; the square root of the nearest-centroid cost is
// the Euclidean norm. Hence, for a token x last assigned to centroid b,
// N(x - c) >= N(c - b) - N(x - b), and every candidate with
// N(c - b) > 2 N(x - b) has J(x, c) > J(x, b) strictly: it can neither win
// nor tie. Tokens are grouped by their previous centroid, 64 to a wave; a
// candidate is skipped by the whole wave when its distance to b exceeds
// twice the largest N(x - b) of the wave, with a 1e-3 relative margin for the
// float32 evaluation. All other candidates are scored exactly as in the full
// assignment, so the ids are the same bits as an assignment over all
// candidates.

// Tokens grouped by centroid id: perm[h][off[c] .. off[c+1]) are the tokens of
// centroid c (any order), woff[c] = sum over c' < c of ceil(count(c') / 64).
__global__ __launch_bounds__(1024) void bucket_kernel(const uint8_t* ids, int64_t n, int m, int32_t* perm,
                                                      int32_t* off, int32_t* woff) {
  __shared__ int cnt[256], cur[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const uint8_t* idh = ids + (int64_t)h * n;
  if (tid < 256) cnt[tid] = 0;
  __syncthreads();
  for (int64_t i = tid; i < n; i += 1024) atomicAdd(&cnt[idh[i]], 1);
  __syncthreads();
  if (tid < 64) {
    // exclusive scans of the counts and of the per-centroid wave counts, 4
    // centroids per lane
    int c4[4], w4[4], cs = 0, ws = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 4 * tid + k;
      c4[k] = (c < m) ? cnt[c] : 0;
      w4[k] = (c4[k] + 63) / 64;
      cs += c4[k];
      ws += w4[k];
    }
    int ci = cs, wi = ws;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int yc = __shfl_up(ci, o), yw = __shfl_up(wi, o);
      if (tid >= o) {
        ci += yc;
        wi += yw;
      }
    }
    int co = ci - cs, wo = wi - ws;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 4 * tid + k;
      if (c <= m) {
        off[h * 257 + c] = co;
        woff[h * 257 + c] = wo;
      }
      if (c < 256) cur[c] = co;
      co += c4[k];
      wo += w4[k];
    }
    if (tid == 63 && m == 256) {  // the end of the last centroid's range
      off[h * 257 + 256] = co;
      woff[h * 257 + 256] = wo;
    }
  }
  __syncthreads();
  for (int64_t i = tid; i < n; i += 1024) {
    const int p = atomicAdd(&cur[idh[i]], 1);
    perm[(int64_t)h * n + p] = (int32_t)i;
  }
}

// Distances N(C_c - C_b) = sqrt(J) between every two centroids of a head,
// row b of the table = [h][b][0 .. m): the bound the pruned assignment
// compares with, computed once per iteration instead of in every wave that
// needs a row. Lane c holds centroid c in registers (as a Key in the
// assignment) and the wave walks its share of the rows b with scalar loads;
// the same function of the same rows as the assignment's own cost.
constexpr int kCcdSplit = 16;  // b ranges per (64 rows, head)

template <int D, int OBJ>
__global__ __launch_bounds__(64) void ccd_kernel(int m, const float* __restrict__ C32, const float* __restrict__ S,
                                                 float* __restrict__ ccd) {
  constexpr int NG = D / kGroup;
  const int lane = threadIdx.x, h = blockIdx.y;
  const int c = blockIdx.x * 64 + lane;
  const int nb = (m + kCcdSplit - 1) / kCcdSplit;
  const int b0 = blockIdx.z * nb, b1 = (b0 + nb) < m ? (b0 + nb) : m;
  const float* __restrict__ Ch = C32 + (int64_t)h * m * D;
  float SG[NG];
#pragma unroll
  for (int G = 0; G < NG; ++G) SG[G] = S[h * NG + G];
  float x[D];
  load_row_span<D, 1>(Ch, (int64_t)(c < m ? c : 0) * D, x);
  for (int b = b0; b < b1; ++b) {
    const float v = sqrtf(assign_cost<OBJ, D>(x, Ch + (int64_t)b * D, SG));
    if (c < m) ccd[((int64_t)h * m + b) * m + c] = v;
  }
}

// One block of NWB waves per (previous centroid b, chunk of 64 of its
// tokens). Every wave scores b first (that gives the bound of the keep mask
// and a starting minimum (J_b, b) per token), forms the same keep mask and
// takes every NWB-th kept candidate; the NWB (J, id) minima are combined
// lexicographically, which is the argmin over all candidates with ties to the
// smallest id. A candidate's cost is built group by group; once every token
// of the wave has a partial sum that already loses to its current minimum
// (larger, or equal with a larger id), the remaining groups are skipped: the
// full cost is at least the partial sum, so the candidate cannot win or tie
// to a smaller id. The candidate rows are wave-uniform scalar loads, so
// nothing before them may look like a memory clobber (no barrier): the
// centroid distances N(C_c - C_b) come from the table ccd_kernel fills
// before the launch.
template <int D, int DT, int OBJ, int NWB>
__global__ __launch_bounds__(NWB * 64) void assign_pruned_kernel(const void* keys, int64_t n, int m,
                                                                 const float* C32, const float* S,
                                                                 const int32_t* perm, const int32_t* off,
                                                                 const int32_t* woff, const float* ccdtab,
                                                                 uint8_t* ids_out, unsigned long long* work) {
  constexpr int NG = D / kGroup;
  __shared__ float bj[NWB][64];
  __shared__ int bi[NWB][64];
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = blockIdx.x;
  const int32_t* wo = woff + h * 257;
  const int32_t* of = off + h * 257;
  if (w >= wo[m]) return;  // the whole block: no barrier is reached
  // centroid b with wo[b] <= w < wo[b+1]
  int lo = 0, hi = m - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (wo[mid] <= w)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int b = __builtin_amdgcn_readfirstlane(lo);
  const int start = of[b] + 64 * (w - wo[b]);
  const int cnt = (of[b + 1] - start) < 64 ? (of[b + 1] - start) : 64;
  const float* __restrict__ Ch = C32 + (int64_t)h * m * D;
  const float* __restrict__ Cb = Ch + (int64_t)b * D;
  float SG[NG];
#pragma unroll
  for (int G = 0; G < NG; ++G) SG[G] = S[h * NG + G];

  // N(C_c - C_b) for c = 64*round + lane, from the table of this iteration
  const float* __restrict__ ccd_b = ccdtab + ((int64_t)h * m + b) * m;
  float ccd[4];
#pragma unroll
  for (int rd = 0; rd < 4; ++rd) {
    const int c = 64 * rd + lane;
    ccd[rd] = (64 * rd < m) ? ccd_b[c < m ? c : 0] : 0.0f;
  }

  const int tok = perm[(int64_t)h * n + start + (lane < cnt ? lane : cnt - 1)];
  float kf[D];
  load_row_span<D, DT>(keys, ((int64_t)h * n + tok) * D, kf);
  const float Jb = assign_cost<OBJ, D>(kf, Cb, SG);
  // group terms computed for each Key of this wave (wave-uniform); the cost of
  // the previous centroid, which every wave repeats, counts in wave 0 only
  int terms = (NWB == 1 || wave == 0) ? NG : 0;
  float d = (lane < cnt) ? sqrtf(Jb) : 0.0f;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) d = fmaxf(d, __shfl_xor(d, o));
  const float bound = 2.0f * d * 1.001f;

  float bestJ = Jb;
  int best = b;
  const bool idle = lane >= cnt;  // copies of the last token: never hold a candidate back
  int rank = 0;  // position in the kept list, to deal the candidates to the waves
#pragma unroll
  for (int rd = 0; rd < 4; ++rd) {
    if (64 * rd >= m) break;
    const int cl = 64 * rd + lane;
    uint64_t keep = __ballot(cl < m && cl != b && !(ccd[rd] > bound));
    while (keep) {
      const int c = 64 * rd + __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(keep));
      keep &= keep - 1;
      if (NWB > 1 && (rank++ % NWB) != wave) continue;
      const float* __restrict__ crow = Ch + (int64_t)c * D;
      float J = 0.0f;
      bool lost = false;
#pragma unroll
      for (int G = 0; G < NG; ++G) {
        const float u = group_term<OBJ, D>(kf, crow, G, SG);
        ++terms;
        J = (G == 0) ? u : J + u;
        if (G < NG - 1 && __all(idle || J > bestJ || (J == bestJ && c > best))) {
          lost = true;
          break;
        }
      }
      if (!lost && (J < bestJ || (J == bestJ && c < best))) {
        bestJ = J;
        best = c;
      }
    }
  }
  // channel evaluations of this wave: its group terms times the Keys it holds
  if (work != nullptr && lane == 0) atomicAdd(work, (unsigned long long)terms * kGroup * (unsigned long long)cnt);
  if constexpr (NWB == 1) {
    if (lane < cnt) ids_out[(int64_t)h * n + tok] = (uint8_t)best;
  } else {
    bj[wave][lane] = bestJ;
    bi[wave][lane] = best;
    __syncthreads();
    if (tid < cnt) {
      float J = bj[0][tid];
      int id = bi[0][tid];
#pragma unroll
      for (int v = 1; v < NWB; ++v)
        if (bj[v][tid] < J || (bj[v][tid] == J && bi[v][tid] < id)) {
          J = bj[v][tid];
          id = bi[v][tid];
        }
      const int t2 = perm[(int64_t)h * n + start + tid];
      ids_out[(int64_t)h * n + t2] = (uint8_t)id;
    }
  }
}

// Commit of a staged calibration: copy C, S, U from the staging slot to the
// epoch slot and write the float / float64 shadows quantize reads, in one pass.
template <int DT>
__global__ void commit_kernel(const void* Cs, const float* Ss, const float* Us, void* Cd, float* Sd, float* Ud,
                              int64_t nC, int64_t nS, int64_t nU, float* C32, double* U64) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nC) {
    if constexpr (DT == 0)
      reinterpret_cast<uint16_t*>(Cd)[i] = reinterpret_cast<const uint16_t*>(Cs)[i];
    else
      reinterpret_cast<float*>(Cd)[i] = reinterpret_cast<const float*>(Cs)[i];
    C32[i] = load_in<DT>(Cs, i);
  }
  if (i < nS) Sd[i] = Ss[i];
  if (i < nU) {
    Ud[i] = Us[i];
    U64[i] = (double)Us[i];
  }
}

__global__ void fill_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <int DT>
__global__ void shadow_kernel(const void* C, const float* U, int64_t nC, int64_t nU, float* C32, double* U64) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nC) C32[i] = load_in<DT>(C, i);
  if (i < nU) U64[i] = (double)U[i];
}

}  // namespace

hipError_t launch_quantize(int D, int dtype, const QuantArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  dim3 grid((unsigned)((a.n + kQTok - 1) / kQTok), (unsigned)a.H);
  dim3 grid2(grid.x, grid.y, 2);
  dim3 block(256);
  const bool assign = (a.v == nullptr);
  if (a.part != nullptr && a.n > kQuantSplitMaxTokens) return hipErrorInvalidValue;
#define QWM_QLAUNCH(DD, TT, OO)                                                                \
  if (a.part != nullptr) {                                                                     \
    hipLaunchKernelGGL((quantize_kernel<DD, TT, true, OO, 1>), grid2, block, 0, s, a);         \
    if (assign)                                                                                \
      hipLaunchKernelGGL((quantize_kernel<DD, TT, true, OO, 2>), grid, block, 0, s, a);        \
    else                                                                                       \
      hipLaunchKernelGGL((quantize_kernel<DD, TT, false, OO, 2>), grid, block, 0, s, a);       \
  } else if (assign) {                                                                         \
    hipLaunchKernelGGL((quantize_kernel<DD, TT, true, OO, 0>), grid, block, 0, s, a);          \
  } else {                                                                                     \
    hipLaunchKernelGGL((quantize_kernel<DD, TT, false, OO, 0>), grid, block, 0, s, a);         \
  }
#define QWM_QOBJ(DD, TT)                  \
  if (a.obj == kObjNearest) {             \
    QWM_QLAUNCH(DD, TT, kObjNearest)      \
  } else if (a.obj == kObjPostq) {        \
    QWM_QLAUNCH(DD, TT, kObjPostq)        \
  } else {                                \
    QWM_QLAUNCH(DD, TT, kObjQsac)         \
  }
  if (a.obj != kObjQsac && a.obj != kObjNearest && a.obj != kObjPostq) return hipErrorInvalidValue;
  if (D == 128 && dtype == 0) {
    QWM_QOBJ(128, 0)
  } else if (D == 128 && dtype == 1) {
    QWM_QOBJ(128, 1)
  } else if (D == 64 && dtype == 0) {
    QWM_QOBJ(64, 0)
  } else if (D == 64 && dtype == 1) {
    QWM_QOBJ(64, 1)
  } else {
    return hipErrorInvalidValue;
  }
#undef QWM_QOBJ
#undef QWM_QLAUNCH
  return hipGetLastError();
}

hipError_t launch_kmeans_seed(int D, int dtype, const void* keys, int64_t n, int H, int m, void* C, float* C32,
                              hipStream_t s) {
  dim3 grid((unsigned)m, (unsigned)H), block((unsigned)D);
  if (dtype == 0)
    hipLaunchKernelGGL((D == 128 ? seed_kernel<128, 0> : seed_kernel<64, 0>), grid, block, 0, s, keys, n, m, C,
                       C32);
  else
    hipLaunchKernelGGL((D == 128 ? seed_kernel<128, 1> : seed_kernel<64, 1>), grid, block, 0, s, keys, n, m, C,
                       C32);
  return hipGetLastError();
}

hipError_t launch_kmeans_bucket(const uint8_t* ids, int64_t n, int H, int m, int32_t* perm, int32_t* off,
                                int32_t* woff, hipStream_t s) {
  hipLaunchKernelGGL(bucket_kernel, dim3((unsigned)H), dim3(1024), 0, s, ids, n, m, perm, off, woff);
  return hipGetLastError();
}

// Waves per block of the pruned assignment (the waves of a block share its
// 64 Keys and deal the kept candidates among themselves). At 256 centroids,
// with the centroid distances read from the table, one wave per block does
// best: 0.85 ms per wm_layer launch against 0.86 with 2 waves and 0.97
// with 4. Below 128 centroids the host takes the full pass; 2 waves measured
// best there.
static int pruned_waves(int m) { return m < 128 ? 2 : 1; }

hipError_t launch_kmeans_ccd(int D, int obj, int H, int m, const float* C32, const float* S, float* ccd,
                             hipStream_t s) {
  if (m < 1 || m > 256) return hipErrorInvalidValue;
  dim3 grid((unsigned)((m + 63) / 64), (unsigned)H, (unsigned)kCcdSplit), block(64);
  if (obj == kObjQsac && D == 128)
    hipLaunchKernelGGL((ccd_kernel<128, kObjQsac>), grid, block, 0, s, m, C32, S, ccd);
  else if (obj == kObjQsac && D == 64)
    hipLaunchKernelGGL((ccd_kernel<64, kObjQsac>), grid, block, 0, s, m, C32, S, ccd);
  else if (obj == kObjNearest && D == 128)
    hipLaunchKernelGGL((ccd_kernel<128, kObjNearest>), grid, block, 0, s, m, C32, S, ccd);
  else if (obj == kObjNearest && D == 64)
    hipLaunchKernelGGL((ccd_kernel<64, kObjNearest>), grid, block, 0, s, m, C32, S, ccd);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_kmeans_assign_pruned(int D, int dtype, int obj, const void* keys, int64_t n, int H, int m,
                                       const float* C32, const float* S, const int32_t* perm, const int32_t* off,
                                       const int32_t* woff, const float* ccd, uint8_t* ids_out,
                                       unsigned long long* work, hipStream_t s) {
  dim3 grid((unsigned)((n + 63) / 64 + m), (unsigned)H);
  if (obj != kObjQsac && obj != kObjNearest) return hipErrorInvalidValue;
  const int nwb = pruned_waves(m);
#define QWM_PLAUNCH(DD, TT, OO)                                                                                      \
  if (nwb == 1)                                                                                                      \
    hipLaunchKernelGGL((assign_pruned_kernel<DD, TT, OO, 1>), grid, dim3(64), 0, s, keys, n, m, C32, S, perm, off,   \
                       woff, ccd, ids_out, work);                                                                               \
  else if (nwb == 2)                                                                                                 \
    hipLaunchKernelGGL((assign_pruned_kernel<DD, TT, OO, 2>), grid, dim3(128), 0, s, keys, n, m, C32, S, perm, off,  \
                       woff, ccd, ids_out, work);                                                                               \
  else                                                                                                               \
    hipLaunchKernelGGL((assign_pruned_kernel<DD, TT, OO, 4>), grid, dim3(256), 0, s, keys, n, m, C32, S, perm, off,  \
                       woff, ccd, ids_out, work);
#define QWM_POBJ(DD, TT)                \
  if (obj == kObjNearest) {             \
    QWM_PLAUNCH(DD, TT, kObjNearest)    \
  } else {                              \
    QWM_PLAUNCH(DD, TT, kObjQsac)       \
  }
  if (D == 128 && dtype == 0) {
    QWM_POBJ(128, 0)
  } else if (D == 128) {
    QWM_POBJ(128, 1)
  } else if (dtype == 0) {
    QWM_POBJ(64, 0)
  } else {
    QWM_POBJ(64, 1)
  }
#undef QWM_POBJ
#undef QWM_PLAUNCH
  return hipGetLastError();
}

hipError_t launch_kmeans_update(int D, int dtype, const void* keys, const uint8_t* ids, int64_t n, int H, int m,
                                void* C, float* C32, hipStream_t s) {
  dim3 grid((unsigned)m, (unsigned)H);
  const bool small = n <= 4096;  // 2 waves per block
#define QWM_ULAUNCH(DD, TT)                                                                               \
  if (small)                                                                                              \
    hipLaunchKernelGGL((update_kernel<DD, TT, 2>), grid, dim3(128), 0, s, keys, ids, n, m, C, C32);       \
  else                                                                                                    \
    hipLaunchKernelGGL((update_kernel<DD, TT, 8>), grid, dim3(512), 0, s, keys, ids, n, m, C, C32);
  if (D == 128 && dtype == 0) {
    QWM_ULAUNCH(128, 0)
  } else if (D == 128) {
    QWM_ULAUNCH(128, 1)
  } else if (dtype == 0) {
    QWM_ULAUNCH(64, 0)
  } else {
    QWM_ULAUNCH(64, 1)
  }
#undef QWM_ULAUNCH
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_commit(int D, int dtype, const void* Cs, const float* Ss, const float* Us, void* Cd, float* Sd,
                         float* Ud, int H, int m, int r, float* C32, double* U64, hipStream_t s) {
  const int64_t nC = (int64_t)H * m * D, nS = (int64_t)H * (D / kGroup), nU = (int64_t)H * D * r;
  int64_t n = nC > nU ? nC : nU;
  if (nS > n) n = nS;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(commit_kernel<0>, grid, block, 0, s, Cs, Ss, Us, Cd, Sd, Ud, nC, nS, nU, C32, U64);
  else
    hipLaunchKernelGGL(commit_kernel<1>, grid, block, 0, s, Cs, Ss, Us, Cd, Sd, Ud, nC, nS, nU, C32, U64);
  return hipGetLastError();
}

hipError_t launch_shadow(int D, int dtype, const void* C, const float* U, int H, int m, int r, float* C32,
                         double* U64, hipStream_t s) {
  const int64_t nC = (int64_t)H * m * D, nU = (int64_t)H * D * r;
  const int64_t n = nC > nU ? nC : nU;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(shadow_kernel<0>, grid, block, 0, s, C, U, nC, nU, C32, U64);
  else
    hipLaunchKernelGGL(shadow_kernel<1>, grid, block, 0, s, C, U, nC, nU, C32, U64);
  return hipGetLastError();
}

}  // namespace qwm
