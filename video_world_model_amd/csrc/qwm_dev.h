// Device helpers for the QuantWM kernels (gfx950). Every helper states the
// rounding it performs; the quantizer's bit-exact steps depend on them.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qwm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Input element -> float. DT 0: bfloat16 bit pattern (exact widening), DT 1: float.
template <int DT>
__device__ __forceinline__ float load_in(const void* p, int64_t i) {
  if constexpr (DT == 0) {
    uint32_t b = reinterpret_cast<const uint16_t*>(p)[i];
    return __uint_as_float(b << 16);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t half_bits(__half h) { return (uint32_t)__half_as_ushort(h); }
__device__ __forceinline__ float half_bits_to_float(uint32_t b) {
  return __half2float(__ushort_as_half((unsigned short)b));
}

// Next float16 toward +inf / -inf of a finite value, on the bit pattern.
__device__ __forceinline__ uint32_t f16_next_up(uint32_t b) {
  if (b == 0x8000u) return 0x0001u;       // -0 -> smallest positive subnormal
  return (b & 0x8000u) ? b - 1u : b + 1u;  // negative: magnitude down; positive: up
}
__device__ __forceinline__ uint32_t f16_next_down(uint32_t b) {
  if (b == 0x0000u) return 0x8001u;       // +0 -> smallest negative subnormal
  return (b & 0x8000u) ? b + 1u : b - 1u;
}

// Largest float16 <= x: nearest-even conversion, then one step down if it
// landed above x.
__device__ __forceinline__ uint32_t f16_round_down(float x) {
  uint32_t b = half_bits(__float2half_rn(x));
  if (half_bits_to_float(b) > x) b = f16_next_down(b);
  return b;
}
// Smallest float16 >= x.
__device__ __forceinline__ uint32_t f16_round_up(float x) {
  uint32_t b = half_bits(__float2half_rn(x));
  if (half_bits_to_float(b) < x) b = f16_next_up(b);
  return b;
}

// float64 -> float rounded toward zero with a sticky low bit ("round to
// odd"). A later nearest-even rounding to any format with at least two fewer
// significand bits (fp16, bf16) then equals one direct rounding of x.
__device__ __forceinline__ float f64_to_f32_odd(double x) {
  float f = (float)x;  // nearest-even
  double fd = (double)f;
  if (fd != x) {
    uint32_t b = __float_as_uint(f);
    if (fabs(fd) > fabs(x)) b -= 1u;  // step toward zero (f != 0 here)
    b |= 1u;
    f = __uint_as_float(b);
  }
  return f;
}
__device__ __forceinline__ uint32_t f64_to_f16_bits(double x) {
  return half_bits(__float2half_rn(f64_to_f32_odd(x)));
}
// float -> bfloat16 nearest-even (bits).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  b = b + 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) { return f32_to_bf16_bits(f64_to_f32_odd(x)); }

// ---- wave64 reductions with DPP (VALU lane moves; no LDS round trip) ----
// update_dpp(old, src, ctrl, row_mask, bank_mask, bound_ctrl): lanes outside
// row_mask, or whose source lane is invalid, receive `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double x, double old) {
  const int lo = __builtin_amdgcn_update_dpp(__double2loint(old), __double2loint(x), CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(__double2hiint(old), __double2hiint(x), CTRL, ROW_MASK, 0xF, false);
  return __hiloint2double(hi, lo);
}
constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// Sum over each aligned group of 8 lanes; every lane of the group gets it.
__device__ __forceinline__ double group8_sum(double x) {
  x += dpp_f64<kDppQuadSwap1, 0xF>(x, 0.0);
  x += dpp_f64<kDppQuadSwap2, 0xF>(x, 0.0);
  x += dpp_f64<kDppRowHalfMirror, 0xF>(x, 0.0);
  return x;
}
// Sum over the 64 lanes, returned to every lane (wave-uniform).
__device__ __forceinline__ double wave_sum(double x) {
  x = group8_sum(x);
  x += dpp_f64<kDppRowMirror, 0xF>(x, 0.0);
  x += dpp_f64<kDppRowBcast15, 0xA>(x, 0.0);
  x += dpp_f64<kDppRowBcast31, 0xC>(x, 0.0);
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), 63);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), 63);
  return __hiloint2double(hi, lo);
}
// Maximum over the 64 lanes, returned to every lane.
__device__ __forceinline__ double wave_max(double x) {
  x = fmax(x, dpp_f64<kDppQuadSwap1, 0xF>(x, x));
  x = fmax(x, dpp_f64<kDppQuadSwap2, 0xF>(x, x));
  x = fmax(x, dpp_f64<kDppRowHalfMirror, 0xF>(x, x));
  x = fmax(x, dpp_f64<kDppRowMirror, 0xF>(x, x));
  x = fmax(x, dpp_f64<kDppRowBcast15, 0xA>(x, x));
  x = fmax(x, dpp_f64<kDppRowBcast31, 0xC>(x, x));
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), 63);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), 63);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_min(double x) { return -wave_max(-x); }

// Sum of the values of the NG (2 or 4) adjacent lanes of an aligned lane
// group, added in lane order ((x0 + x1) + x2) + x3; every lane of the group
// gets the same bits.
template <int NG>
__device__ __forceinline__ double group_ordered_sum(double x) {
  if constexpr (NG == 4) {
    const double x0 = dpp_f64<0x00, 0xF>(x, 0.0);  // quad_perm [0,0,0,0]
    const double x1 = dpp_f64<0x55, 0xF>(x, 0.0);  // quad_perm [1,1,1,1]
    const double x2 = dpp_f64<0xAA, 0xF>(x, 0.0);  // quad_perm [2,2,2,2]
    const double x3 = dpp_f64<0xFF, 0xF>(x, 0.0);  // quad_perm [3,3,3,3]
    return ((x0 + x1) + x2) + x3;
  } else {
    static_assert(NG == 2, "groups of 2 or 4 lanes");
    const double x0 = dpp_f64<0xA0, 0xF>(x, 0.0);  // quad_perm [0,0,2,2]
    const double x1 = dpp_f64<0xF5, 0xF>(x, 0.0);  // quad_perm [1,1,3,3]
    return x0 + x1;
  }
}

}  // namespace qwm
