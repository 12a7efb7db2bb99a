// Shared device helpers for the gfx950 kernels: storage types, 16-byte vector
// loads/stores, wave reductions through DPP, and the internal launcher API that
// h3_api.cpp calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3 {

typedef uint16_t bf16_t;  // bfloat16 storage bits

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bfloat16, round to nearest even (hardware conversion on gfx950)
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// ---- 8-element loads/stores of a storage type into/from fp32 registers ----

template <typename T>
struct Vec8;

template <>
struct Vec8<float> {
  __device__ __forceinline__ static void load(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  // streaming forms: non-temporal hint, for data touched once per pass
  __device__ __forceinline__ static void load_nt(const float* p, float (&v)[8]) {
    const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
  __device__ __forceinline__ static void store_nt(float* p, const float (&v)[8]) {
    const f32x4_t a = {v[0], v[1], v[2], v[3]};
    const f32x4_t b = {v[4], v[5], v[6], v[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t*>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4_t*>(p + 4));
  }
};

template <>
struct Vec8<bf16_t> {
  __device__ __forceinline__ static void load(const bf16_t* p, float (&v)[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static void store(bf16_t* p, const float (&v)[8]) {
    uint4 a;
    a.x = pack_bf16x2(v[0], v[1]);
    a.y = pack_bf16x2(v[2], v[3]);
    a.z = pack_bf16x2(v[4], v[5]);
    a.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = a;
  }
  __device__ __forceinline__ static void load_nt(const bf16_t* p, float (&v)[8]) {
    const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static void store_nt(bf16_t* p, const float (&v)[8]) {
    const u32x4_t a = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7])};
    __builtin_nontemporal_store(a, reinterpret_cast<u32x4_t*>(p));
  }
};

// ---- DPP reductions inside rows of 16 lanes (every lane gets the result) ----

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// sum over groups of N lanes (N in {2, 4, 8, 16}), aligned to N
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);                      // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);  // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x); // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror
  return x;
}

// full 64-lane sum, result valid in every lane
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Column of key 0 of segment s in the transposed-V scratch: 64-aligned, with a
// gap so that every segment can be read in whole 64-key tiles.
__host__ __device__ __forceinline__ int64_t vt_segment_base(int64_t slot_begin, int s) {
  return round_up(slot_begin, 64) + 128 * (int64_t)s;
}
__host__ __device__ constexpr int64_t vt_columns(int64_t n_buf, int n_seg) {
  return round_up(n_buf, 64) + 128 * (int64_t)(n_seg + 1);
}

}  // namespace h3
