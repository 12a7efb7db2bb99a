// Measurement aids (not steps of the method).
//
// mfma_rate_kernel: the bf16 matrix-core rate the chip sustains, with no memory
// traffic, at the occupancy of the attention kernel (8 waves per work-group,
// one work-group per CU).  Each wave runs `iters` rounds of four independent
// 32x32x16 bf16 MFMAs.  The operands are fixed per lane: pseudo-random values
// in [-2, 2) or all zeros; the rate differs between the two because the chip
// lowers its clock with the switching activity of the operands.
#include "h3_common.hpp"
#include "h3_kernels.hpp"

namespace h3 {

__global__ __launch_bounds__(512, 1) void mfma_rate_kernel(float* __restrict__ out, int iters,
                                                           int zero) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t h = (lane * 2654435761u) ^ (i * 40503u) ^ (blockIdx.x * 97u) ^ (threadIdx.x >> 6);
    h ^= h >> 13;
    h *= 0x5bd1e995u;
    h ^= h >> 15;
    const float fa = zero ? 0.f : ((int)(h & 0xffff) - 32768) / 16384.f;
    const float fb = zero ? 0.f : ((int)(h >> 16) - 32768) / 16384.f;
    a[i] = (__bf16)fa;
    b[i] = (__bf16)fb;
  }
  f32x16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

hipError_t launch_mfma_rate(int blocks, int iters, int zero, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(512), 0, s, out, iters, zero);
  return hipGetLastError();
}

// HBM rates of the two access patterns the elementwise passes use, each in the
// fastest plain form measured on gfx950: one 16-byte chunk per thread and a
// large grid.  Copy (src -> dst, non-temporal loads and stores) is the pattern
// of the out-of-place passes; read-modify-write in place over the first
// `touch` chunks of rows of `row` chunks (plain loads and stores, which beat
// the non-temporal ones for this pattern) is that of the Q/K norm + RoPE pass
// on the q and k thirds of a QKV buffer.
__global__ __launch_bounds__(256) void hbm_copy_kernel(const u32x4_t* __restrict__ src,
                                                       u32x4_t* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void hbm_rmw_kernel(u32x4_t* __restrict__ buf, int64_t rows,
                                                      int64_t row, int64_t touch) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;  // index among touched chunks
  const int64_t r = t / touch;
  if (r >= rows) return;
  u32x4_t* p = buf + r * row + (t - r * touch);
  u32x4_t v = *p;
  v[0] += 1u;
  *p = v;
}

hipError_t launch_hbm_rate(int mode, const void* src, void* dst, int64_t rows, int64_t row,
                           int64_t touch, hipStream_t s) {
  const int64_t n = rows * touch;
  const dim3 grid((unsigned)ceil_div(n, 256));
  if (mode == 0)
    hipLaunchKernelGGL(hbm_copy_kernel, grid, dim3(256), 0, s, (const u32x4_t*)src,
                       (u32x4_t*)dst, n);
  else
    hipLaunchKernelGGL(hbm_rmw_kernel, grid, dim3(256), 0, s, (u32x4_t*)dst, rows, row, touch);
  return hipGetLastError();
}

}  // namespace h3
