// 2-bit codes times their group's step as fp16 pairs, for the attention
// kernels' Value (and Key) operands (gfx950).
//
// QuantWM stores every Key residual and Value group as 2-bit codes c with a
// zero-point and a step s per 32-channel group (roboind.com article, "Step
// 1"); the dequantized value is zp + c * s. The step is chosen so that 3 s
// is an fp16 value, so every c * s (c = 0..3) is one, and the operand
// c * s can be built without rounding:
//  * a code pair c0, c1 (bits 0-1 and 16-17 of a word, the rest cleared) is
//    or-ed into the fp16 pair 1024 + c (exact: ulp 1 in [1024, 2048));
//  * then c * s is either (b - 1024) * s, two exact operations, or, when
//    every lane's steps are below 64, one fused b * s - 1024 s: -1024 s is
//    exact there and the single rounding of the fused result returns the
//    exact c * s.
// The choice is wave-uniform (a ballot), so each wave takes one branch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qwm {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// 0x64006400 (fp16 1024, 1024) in a VGPR: with the mask in an SGPR the
// compiler can then fuse "(x & mask) | magic" into one v_and_or_b32 (a VOP3
// reads at most one scalar operand here).
__device__ __forceinline__ uint32_t magic_1024_vgpr() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

struct CodeScale {
  half2v s2, nb;  // steps (two fp16); -1024 * steps (used when `small`)
  uint32_t magic;
  bool small;  // every lane's steps are below 64 (wave-uniform)
};

// s2_bits: two fp16 steps (>= 0), one per half.
__device__ __forceinline__ CodeScale code_scale(uint32_t s2_bits) {
  CodeScale cs;
  cs.s2 = __builtin_bit_cast(half2v, s2_bits);
  cs.nb = cs.s2 * (half2v){(_Float16)-1024.0f, (_Float16)-1024.0f};
  cs.magic = magic_1024_vgpr();
  // fp16 bits below 0x5400 (64.0) in both halves
  const bool ok = (s2_bits & 0x7FFFu) < 0x5400u && ((s2_bits >> 16) & 0x7FFFu) < 0x5400u;
  cs.small = __builtin_amdgcn_ballot_w64(!ok) == 0;
  return cs;
}

// out[i] = the code pair in bits 0-1 and 16-17 of x[i] (other bits are
// masked off) times the steps, for N pairs; the branch on `small` is taken
// once for all of them.
template <int N>
__device__ __forceinline__ void code_pairs(const uint32_t (&x)[N], const CodeScale& cs, uint32_t (&out)[N]) {
  if (cs.small) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const half2v b = __builtin_bit_cast(half2v, (x[i] & 0x00030003u) | cs.magic);
      out[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(b, cs.s2, cs.nb));
    }
  } else {
    const half2v k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const half2v b = __builtin_bit_cast(half2v, (x[i] & 0x00030003u) | cs.magic);
      out[i] = __builtin_bit_cast(uint32_t, (b - k1024) * cs.s2);
    }
  }
}

}  // namespace qwm
