// Small kernels around the block: head-slice copies that stand at the two ends
// of the sequence-parallel exchange, the Euler update and the timestep
// modulation of the four-forward student.
//
// Why Real-Time MiniMax H3 Serving Requires More Than a Faster DiT, "Key
// takeaways": an all-to-all moves rows around attention; MiniMax H3 通过
// vLLM-Omni 实现 FastH3 实时推理, "FastH3：四步学生模型": four forwards over five
// sigma positions.
#include "h3_common.hpp"
#include "h3_kernels.hpp"

#include <algorithm>

namespace h3 {

// Copy a [rows, groups, width] block of 16-byte chunks between two strided
// layouts: dst[r * ld_dst + g * gstride_dst + c] = src[r * ld_src + g * gstride_src + c].
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint4* __restrict__ src,
                                                        int64_t ld_src, int64_t gs_src,
                                                        uint4* __restrict__ dst, int64_t ld_dst,
                                                        int64_t gs_dst, int64_t rows, int groups,
                                                        int chunks) {
  const int64_t per_row = (int64_t)groups * chunks;
  const int64_t total = rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / per_row;
    const int rem = (int)(i - r * per_row);
    const int g = rem / chunks, c = rem % chunks;
    dst[r * ld_dst + g * gs_dst + c] = src[r * ld_src + g * gs_src + c];
  }
}

hipError_t launch_copy_rows(const void* src, int64_t ld_src, int64_t gs_src, void* dst,
                            int64_t ld_dst, int64_t gs_dst, int64_t rows, int groups,
                            int64_t bytes_per_group, hipStream_t s) {
  // strides in bytes, all multiples of 16
  const int chunks = (int)(bytes_per_group / 16);
  const int64_t total = rows * groups * chunks;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(total, 256), 65536);
  hipLaunchKernelGGL(copy_rows_kernel, dim3(blocks), dim3(256), 0, s, (const uint4*)src,
                     ld_src / 16, gs_src / 16, (uint4*)dst, ld_dst / 16, gs_dst / 16, rows, groups,
                     chunks);
  return hipGetLastError();
}

// z <- z + dsig * u ; x_next <- z (optional)
template <typename T>
__global__ __launch_bounds__(256) void euler_kernel(T* z, const T* u, T* x_next, int64_t n8,
                                                    float dsig) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * 256) {
    float zv[8], uv[8];
    Vec8<T>::load(z + 8 * i, zv);
    Vec8<T>::load(u + 8 * i, uv);
#pragma unroll
    for (int e = 0; e < 8; ++e) zv[e] += dsig * uv[e];
    Vec8<T>::store(z + 8 * i, zv);
    if (x_next) Vec8<T>::store(x_next + 8 * i, zv);
  }
}

hipError_t launch_euler(bool bf16, void* z, const void* u, void* x_next, int64_t n, float dsig,
                        hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(n8, 256), 65536);
  if (bf16)
    hipLaunchKernelGGL(euler_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, (bf16_t*)z,
                       (const bf16_t*)u, (bf16_t*)x_next, n8, dsig);
  else
    hipLaunchKernelGGL(euler_kernel<float>, dim3(blocks), dim3(256), 0, s, (float*)z,
                       (const float*)u, (float*)x_next, n8, dsig);
  return hipGetLastError();
}

// ---- timestep modulation: e(sigma) -> hid = silu(W_t1 e) -> t = W_t2 hid -> + table[b]

// hid[c] = silu(sum_j W_t1[c, j] e_j); one wave per output row c
template <typename T>
__global__ __launch_bounds__(256) void temb_hidden_kernel(const T* __restrict__ w1,
                                                          float* __restrict__ hid, int dim,
                                                          int emb, float sigma) {
  __shared__ float e[1024];
  const int half = emb / 2;
  for (int j = threadIdx.x; j < half; j += 256) {
    const double om = exp2(-(double)j / half * log2(10000.0));
    const double a = 1000.0 * (double)sigma * om;
    e[j] = (float)cos(a);
    e[half + j] = (float)sin(a);
  }
  __syncthreads();
  const int c = blockIdx.x * 4 + threadIdx.x / 64;
  if (c >= dim) return;
  const int lane = threadIdx.x % 64;
  float acc = 0.f;
  for (int j0 = lane * 8; j0 < emb; j0 += 512) {
    float wv[8];
    Vec8<T>::load(w1 + (int64_t)c * emb + j0, wv);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc += wv[t] * e[j0 + t];
  }
  acc = wave_sum(acc);
  if (lane == 0) hid[c] = acc / (1.0f + __expf(-acc));
}

// t[i] = sum_c W_t2[i, c] hid[c]; mod_out[b, i] = t[i] + table[b, i]; one wave per row i
template <typename T>
__global__ __launch_bounds__(256) void temb_out_kernel(const T* __restrict__ w2,
                                                       const float* __restrict__ hid,
                                                       const T* __restrict__ table,
                                                       T* __restrict__ mod_out, int dim,
                                                       int n_blocks) {
  const int64_t rows = 6 * (int64_t)dim;
  const int64_t i = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  if (i >= rows) return;
  const int lane = threadIdx.x % 64;
  float acc = 0.f;
  for (int c0 = lane * 8; c0 < dim; c0 += 512) {
    float wv[8];
    Vec8<T>::load(w2 + i * dim + c0, wv);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc += wv[t] * hid[c0 + t];
  }
  acc = wave_sum(acc);
  for (int b = lane; b < n_blocks; b += 64) {
    float tv;
    if constexpr (sizeof(T) == 2) tv = bf2f(table[b * rows + i]); else tv = table[b * rows + i];
    const float r = acc + tv;
    if constexpr (sizeof(T) == 2) mod_out[b * rows + i] = f2bf(r); else mod_out[b * rows + i] = r;
  }
}

hipError_t launch_timestep(bool bf16, float sigma, const void* w1, const void* w2,
                           const void* table, void* mod_out, int n_blocks, int dim, int emb,
                           void* ws, hipStream_t s) {
  float* hid = (float*)ws;
  const unsigned b1 = (unsigned)ceil_div(dim, 4);
  const unsigned b2 = (unsigned)ceil_div(6 * (int64_t)dim, 4);
  if (bf16) {
    hipLaunchKernelGGL(temb_hidden_kernel<bf16_t>, dim3(b1), dim3(256), 0, s, (const bf16_t*)w1,
                       hid, dim, emb, sigma);
    hipLaunchKernelGGL(temb_out_kernel<bf16_t>, dim3(b2), dim3(256), 0, s, (const bf16_t*)w2,
                       hid, (const bf16_t*)table, (bf16_t*)mod_out, dim, n_blocks);
  } else {
    hipLaunchKernelGGL(temb_hidden_kernel<float>, dim3(b1), dim3(256), 0, s, (const float*)w1,
                       hid, dim, emb, sigma);
    hipLaunchKernelGGL(temb_out_kernel<float>, dim3(b2), dim3(256), 0, s, (const float*)w2, hid,
                       (const float*)table, (float*)mod_out, dim, n_blocks);
  }
  return hipGetLastError();
}

}  // namespace h3
