// QSAC quantize-on-insert, k-means centroid construction and epoch shadows
// for the QuantWM 2-bit KV cache (gfx950).
//
// Method (QuantWM, arXiv 2609.26425; roboind.com article "Step 1" and
// "Step 2", fugumt.com abstract): each Key is assigned the centroid that
// minimizes J = sum_G S_G (max_G r - min_G r)^2, r = k - c, the residual is
// stored as per-group asymmetric INT2 with fp16 zero-point/step, the Key's
// remaining error is projected on the PSAC basis (r fp16 coefficients), and
// the Value is stored as plain per-group INT2.
//
// Mapping to CDNA4: one lane owns one token (64 tokens per wave), so the
// objective, the argmin and the group min/max all run lane-sequentially in
// exactly the order of the definition, with no cross-lane reduction. The
// centroid row being scored is the same for every lane of the wave; it is
// loaded through the scalar path (one copy per wave in SGPRs) and consumed as
// an SGPR operand of v_sub, so the candidate loop is pure VALU (sub, max3,
// min3) with no LDS traffic. Builds use -ffp-contract=off so no multiply-add
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

// Per-group INT2 parameters (signed zeros folded to +0):
// zp = largest fp16 <= min, step = smallest fp16 >= (max - zp) / 3.
__device__ __forceinline__ void int2_params(float mn, float mx, uint32_t& zpb, uint32_t& scb, float& zpf,
                                            float& scf) {
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  zpb = f16_round_down(mn);
  zpf = half_bits_to_float(zpb);
  const float step = (mx - zpf) / 3.0f;  // correctly rounded divide
  scb = f16_round_up(step);
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

template <int D, int DT>
__device__ __forceinline__ void load_row(const void* base, int64_t off, float (&x)[D]) {
  if constexpr (DT == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
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
    for (int i = 0; i < D / 4; ++i) {
      const float4 w = p[i];
      x[4 * i] = w.x;
      x[4 * i + 1] = w.y;
      x[4 * i + 2] = w.z;
      x[4 * i + 3] = w.w;
    }
  }
}

// Plain per-group INT2 of one row x (Values): codes into words, params.
template <int D>
__device__ __forceinline__ void int2_row(const float (&x)[D], uint32_t (&words)[D / 16],
                                         uint32_t (&params)[D / kGroup]) {
  constexpr int NG = D / kGroup;
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    float mx = x[G * kGroup], mn = x[G * kGroup];
#pragma unroll
    for (int j = 1; j < kGroup; ++j) {
      mx = fmaxf(mx, x[G * kGroup + j]);
      mn = fminf(mn, x[G * kGroup + j]);
    }
    uint32_t zpb, scb;
    float zpf, scf;
    int2_params(mn, mx, zpb, scb, zpf, scf);
    params[G] = zpb | (scb << 16);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const uint32_t code = int2_code(x[G * kGroup + j], zpf, scf);
      if (j < 16)
        w0 |= code << (2 * j);
      else
        w1 |= code << (2 * (j - 16));
    }
    words[2 * G] = w0;
    words[2 * G + 1] = w1;
  }
}

template <int D, int DT, bool ASSIGN_ONLY>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  constexpr int NG = D / kGroup;
  const int h = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * kQuantTokensPerBlock + threadIdx.x;
  if (t >= a.n) return;  // the kernel has no barrier

  float kf[D];
  load_row<D, DT>(a.k, ((int64_t)h * a.n + t) * D, kf);

  float SG[NG];
#pragma unroll
  for (int G = 0; G < NG; ++G) SG[G] = a.S[h * NG + G];

  // QSAC assignment: ascending candidates; strict < keeps the smallest id on ties.
  const float* __restrict__ Ch = a.C32 + (int64_t)h * a.m * D;
  float bestJ = __builtin_inff();
  int best = 0;
  for (int c = 0; c < a.m; ++c) {
    const float J = qsac_cost<D>(kf, Ch + (int64_t)c * D, SG);
    if (J < bestJ) {
      bestJ = J;
      best = c;
    }
  }
  if constexpr (ASSIGN_ONLY) {
    a.ids_out[(int64_t)h * a.n + t] = (uint8_t)best;
  } else {
    const int64_t slot = (int64_t)h * a.cache.capP + a.pos0 + t;
    const float* crow = Ch + (int64_t)best * D;
    const double* __restrict__ Uh = a.U64 + (int64_t)h * D * a.r;
    double acc[kRankPad];
#pragma unroll
    for (int i = 0; i < kRankPad; ++i) acc[i] = 0.0;

    uint32_t kparam[NG];
    uint32_t kwords[D / 16];  // 16 channels (2 bits each) per 32-bit word
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      float mx, mn;
      {
        const float r0 = kf[G * kGroup] - crow[G * kGroup];
        mx = r0;
        mn = r0;
      }
#pragma unroll
      for (int j = 1; j < kGroup; ++j) {
        const float r = kf[G * kGroup + j] - crow[G * kGroup + j];
        mx = fmaxf(mx, r);
        mn = fminf(mn, r);
      }
      uint32_t zpb, scb;
      float zpf, scf;
      int2_params(mn, mx, zpb, scb, zpf, scf);
      kparam[G] = zpb | (scb << 16);
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const int ch = G * kGroup + j;
        const float c = crow[ch];
        const float r = kf[ch] - c;
        const uint32_t code = int2_code(r, zpf, scf);
        if (j < 16)
          w0 |= code << (2 * j);
        else
          w1 |= code << (2 * (j - 16));
        // PSAC error e = k - (c + rhat), rhat = zp + code*step (the product is exact).
        const float rhat = zpf + (float)code * scf;
        const float tsum = c + rhat;
        const float e = kf[ch] - tsum;
        const double ed = (double)e;
        const double* urow = Uh + (int64_t)ch * a.r;
#pragma unroll
        for (int i = 0; i < kRankPad; ++i)
          if (i < a.r) acc[i] = fma(ed, urow[i], acc[i]);
      }
      kwords[2 * G] = w0;
      kwords[2 * G + 1] = w1;
    }
    uint32_t* kc = reinterpret_cast<uint32_t*>(a.cache.kcode + slot * (D / 4));
#pragma unroll
    for (int i = 0; i < D / 16; ++i) kc[i] = kwords[i];
    uint32_t* kp = a.cache.kparam + slot * NG;
#pragma unroll
    for (int G = 0; G < NG; ++G) kp[G] = kparam[G];
    a.cache.ids[slot] = (uint8_t)best;
    uint16_t* cf = a.cache.coef + slot * a.r;
#pragma unroll
    for (int i = 0; i < kRankPad; ++i)
      if (i < a.r) cf[i] = (uint16_t)f64_to_f16_bits(acc[i]);

    // Value: plain per-group INT2.
    float vf[D];
    load_row<D, DT>(a.v, ((int64_t)h * a.n + t) * D, vf);
    uint32_t vwords[D / 16];
    uint32_t vparam[NG];
    int2_row<D>(vf, vwords, vparam);
    uint32_t* vc = reinterpret_cast<uint32_t*>(a.cache.vcode + slot * (D / 4));
#pragma unroll
    for (int i = 0; i < D / 16; ++i) vc[i] = vwords[i];
    uint32_t* vp = a.cache.vparam + slot * NG;
#pragma unroll
    for (int G = 0; G < NG; ++G) vp[G] = vparam[G];
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

// k-means update: one wave per (centroid, head). The wave walks the ids in
// token order (ballot of 64 at a time) and adds each member Key into float64
// lane accumulators (D / 64 channels per lane), so the sum is formed in the
// same token order on every run. The mean is rounded once to the cache dtype;
// a centroid without members keeps its value.
template <int D, int DT>
__global__ __launch_bounds__(64) void update_kernel(const void* keys, const uint8_t* ids, int64_t n, int m,
                                                    void* C, float* C32) {
  constexpr int PER = D / 64;
  const int c = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const uint8_t* idh = ids + (int64_t)h * n;
  double acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.0;
  int64_t count = 0;
  for (int64_t base = 0; base < n; base += 64) {
    const int64_t t = base + lane;
    const bool hit = (t < n) && (idh[t] == (uint8_t)c);
    uint64_t mask = __ballot(hit);
    while (mask) {
      const int b = __ffsll((unsigned long long)mask) - 1;
      mask &= mask - 1;
      const int64_t row = ((int64_t)h * n + base + b) * D;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] += (double)load_in<DT>(keys, row + lane + 64 * k);
      ++count;
    }
  }
  if (count == 0) return;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const double mean = acc[k] / (double)count;
    const int64_t di = ((int64_t)h * m + c) * D + lane + 64 * k;
    if constexpr (DT == 0) {
      const uint32_t b = f64_to_bf16_bits(mean);
      reinterpret_cast<uint16_t*>(C)[di] = (uint16_t)b;
      C32[di] = bf16_bits_to_float(b);
    } else {
      const float f = (float)mean;  // nearest-even
      reinterpret_cast<float*>(C)[di] = f;
      C32[di] = f;
    }
  }
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
  dim3 grid((unsigned)((a.n + kQuantTokensPerBlock - 1) / kQuantTokensPerBlock), (unsigned)a.H);
  dim3 block(kQuantTokensPerBlock);
  const bool assign = (a.v == nullptr);
#define QWM_QLAUNCH(DD, TT)                                                   \
  if (assign)                                                                 \
    hipLaunchKernelGGL((quantize_kernel<DD, TT, true>), grid, block, 0, s, a); \
  else                                                                        \
    hipLaunchKernelGGL((quantize_kernel<DD, TT, false>), grid, block, 0, s, a);
  if (D == 128 && dtype == 0) {
    QWM_QLAUNCH(128, 0)
  } else if (D == 128 && dtype == 1) {
    QWM_QLAUNCH(128, 1)
  } else if (D == 64 && dtype == 0) {
    QWM_QLAUNCH(64, 0)
  } else if (D == 64 && dtype == 1) {
    QWM_QLAUNCH(64, 1)
  } else {
    return hipErrorInvalidValue;
  }
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

hipError_t launch_kmeans_update(int D, int dtype, const void* keys, const uint8_t* ids, int64_t n, int H, int m,
                                void* C, float* C32, hipStream_t s) {
  dim3 grid((unsigned)m, (unsigned)H), block(64);
  if (dtype == 0)
    hipLaunchKernelGGL((D == 128 ? update_kernel<128, 0> : update_kernel<64, 0>), grid, block, 0, s, keys, ids, n,
                       m, C, C32);
  else
    hipLaunchKernelGGL((D == 128 ? update_kernel<128, 1> : update_kernel<64, 1>), grid, block, 0, s, keys, ids, n,
                       m, C, C32);
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
