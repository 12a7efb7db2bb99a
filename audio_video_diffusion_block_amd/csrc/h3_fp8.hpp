// MX-scaled e4m3 helpers shared by the FP8 attention and the FP8 GEMMs.
//
// Block format: 32 consecutive elements share one E8M0 byte e + 127 (the
// scale 2^e) and are stored as OCP e4m3 (1 sign, 4 exponent bits with bias
// 7, 3 mantissa bits; largest finite 448).  e is the smallest exponent with
// amax <= 448 * 2^e, so the block's largest magnitude lands in e4m3's top
// binade, and elements are rounded to nearest, ties to even.
//
// gfx950 v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, fp32 accumulation):
// A lane (row + 32 h) byte e pairs with B lane (col + 32 h) byte e; bytes 0-15
// of both lane halves form the first 32-element block of the contraction
// (E8M0 scale taken from the row's lane), bytes 16-31 the second (scale from
// lane row + 32).  The logical contraction index of (h, e) is therefore
// 32 (e / 16) + 16 h + e % 16, and a 64-deep step covers two scale blocks.
#pragma once

#include "h3_common.hpp"

namespace h3 {
namespace fp8 {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// smallest e in [-127, 127] with amax <= 448 * 2^e (0 for an all-zero block):
// amax = 1.f * 2^E needs e = E - 8, or E - 7 when 1.f > 1.75
__device__ __forceinline__ int e8m0_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)(b >> 23) - 127;
  if (E == -127) return -127;
  const int e = E - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// four values times the power of two s -> four e4m3 bytes (nearest, ties to even)
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d, float s) {
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a * s, b * s, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c * s, d * s, (int)w, true);
}

// 32 floats -> 32 e4m3 bytes (8 words) and their E8M0 byte
__device__ __forceinline__ uint32_t quant32(const float* v, uint32_t* w) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = e8m0_exp(amax);
  const float s = __builtin_ldexpf(1.0f, -e);
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = pack4_e4m3(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], s);
  return (uint32_t)(e + 127);
}

// 32 wait states: VALU code that reads or rewrites the accumulators of a
// v_mfma_scale_f32_32x32x64_f8f6f4 issued just before (the compiler's own
// padding after this instruction has been measured to be too short: the
// last result registers were read stale)
__device__ __forceinline__ void scaled_mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// scaled e4m3 x e4m3 MFMA whose operands' scale bytes sit at byte SEL of the scale registers
template <int SEL>
__device__ __forceinline__ f32x16_t mfma_e4m3(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c,
                                             uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SEL, (int)sa, SEL, (int)sb);
}

}  // namespace fp8
}  // namespace h3
