// Fused gated residual + modulated normalisation over rows of the residual stream:
//   x <- x + gate * y            (optional)
//   h <- norm(x) * (1 + scale) + shift   (optional; LayerNorm or RMSNorm)
//
// Why Real-Time MiniMax H3 Serving Requires More Than a Faster DiT, "Key
// takeaways": modulation, normalisation and residual updates are fused.
//
// HBM-bound, one work-group per row.  Each thread owns CPT chunks of 8 values
// (16 bytes of bf16), chunk c at c = tid + i*blockDim so a wave's accesses are
// contiguous.  All loads of a row are issued before any arithmetic; the row
// stays in registers for the exact two-pass mean/variance, so x is read once.
// Every access carries the non-temporal hint: each byte is touched once per
// pass, and the hint lifts the pass from ~5.5 to ~6.0 TB/s at 30,776 x 5120.
#include "h3_common.hpp"
#include "h3_fp8.hpp"
#include "h3_kernels.hpp"

namespace h3 {
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  constexpr int NW = NT / 64;
  v = wave_sum(v);
  if constexpr (NW == 1) {
    return v;
  } else {
    const int w = threadIdx.x / 64;
    __syncthreads();  // red[] may still be read by a previous reduction
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += red[i];
    return t;
  }
}

// MX: h is not stored; instead its bf16 values are quantized in place of a
// separate pass into an MX operand (mq: e4m3 bytes, row stride ld_mq; ms: one
// E8M0 byte per 32 columns, row stride ld_ms).  A 32-column block is 4 chunks
// held by 4 adjacent lanes (NT is a multiple of 4), whose amax is one DPP
// exchange.  Needs dim % 32 == 0; the bytes equal those of quantizing the
// stored bf16 h.
template <typename T, int NT, int CPT, bool MX = false>
__global__ __launch_bounds__(NT) void modres_kernel(
    T* __restrict__ x, int64_t ld_x, const T* __restrict__ y, int64_t ld_y,
    const T* __restrict__ gate, const T* __restrict__ shift, const T* __restrict__ scale,
    int64_t ld_mod, T* __restrict__ h, int64_t ld_h, int dim, int norm_kind, float eps,
    uint8_t* __restrict__ mq = nullptr, int64_t ld_mq = 0, uint8_t* __restrict__ ms = nullptr,
    int64_t ld_ms = 0) {
  __shared__ float red[NT / 64];
  const int64_t row = blockIdx.x;
  const int chunks = dim / 8;
  T* xr = x + row * ld_x;
  const int64_t mrow = row * ld_mod;

  float xv[CPT][8];
  float yv[CPT][8];
  float gv[CPT][8];
  float sh[CPT][8];
  float sc[CPT][8];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < chunks) {
      Vec8<T>::load_nt(xr + 8 * c, xv[i]);
      if (y) {
        Vec8<T>::load_nt(y + row * ld_y + 8 * c, yv[i]);
        Vec8<T>::load_nt(gate + mrow + 8 * c, gv[i]);
      }
      if (MX || h) {
        Vec8<T>::load_nt(shift + mrow + 8 * c, sh[i]);
        Vec8<T>::load_nt(scale + mrow + 8 * c, sc[i]);
      }
    }
  }
  if (y) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * NT;
      if (c < chunks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[i][e] += gv[i][e] * yv[i][e];
        Vec8<T>::store_nt(xr + 8 * c, xv[i]);
      }
    }
  }
  if (!MX && !h) return;

  const float inv_dim = 1.0f / (float)dim;
  float mean = 0.f;
  if (norm_kind == 0) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (threadIdx.x + i * NT < chunks)
#pragma unroll
        for (int e = 0; e < 8; ++e) s += xv[i][e];
    mean = block_sum<NT>(s, red) * inv_dim;
  }
  float s2 = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    if (threadIdx.x + i * NT < chunks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = xv[i][e] - mean;
        s2 += d * d;
      }
  const float var = block_sum<NT>(s2, red) * inv_dim;
  const float rstd = rsqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < chunks) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = (xv[i][e] - mean) * rstd * (1.0f + sc[i][e]) + sh[i][e];
      if constexpr (MX) {
        float am = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = bf2f(f2bf(o[e]));  // the bf16 value the stored h would hold
          am = fmaxf(am, fabsf(o[e]));
        }
        am = fmaxf(am, dpp<0xB1>(am));  // quad_perm [1,0,3,2]
        am = fmaxf(am, dpp<0x4E>(am));  // quad_perm [2,3,0,1]: the block's amax
        const int ex = fp8::e8m0_exp(am);
        const float s = __builtin_ldexpf(1.0f, -ex);
        uint2 wq;
        wq.x = fp8::pack4_e4m3(o[0], o[1], o[2], o[3], s);
        wq.y = fp8::pack4_e4m3(o[4], o[5], o[6], o[7], s);
        __builtin_nontemporal_store(u32x2_t{wq.x, wq.y}, reinterpret_cast<u32x2_t*>(mq + row * ld_mq + 8 * c));
        if ((threadIdx.x & 3) == 0) ms[row * ld_ms + c / 4] = (uint8_t)(ex + 127);
      } else {
        Vec8<T>::store_nt(h + row * ld_h + 8 * c, o);
      }
    }
  }
}

template <typename T, int NT, int CPT>
static hipError_t launch_mr(void* x, int64_t ld_x, const void* y, int64_t ld_y, const void* gate,
                            const void* shift, const void* scale, int64_t ld_mod, void* h,
                            int64_t ld_h, int64_t n_tok, int dim, int norm_kind, float eps,
                            hipStream_t s) {
  hipLaunchKernelGGL((modres_kernel<T, NT, CPT>), dim3((unsigned)n_tok), dim3(NT), 0, s, (T*)x,
                     ld_x, (const T*)y, ld_y, (const T*)gate, (const T*)shift, (const T*)scale,
                     ld_mod, (T*)h, ld_h, dim, norm_kind, eps);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_mr(void* x, int64_t ld_x, const void* y, int64_t ld_y,
                              const void* gate, const void* shift, const void* scale,
                              int64_t ld_mod, void* h, int64_t ld_h, int64_t n_tok, int dim,
                              int norm_kind, float eps, hipStream_t s) {
  const int chunks = dim / 8;
#define H3_MR(NT, CPT)                                                                      \
  return launch_mr<T, NT, CPT>(x, ld_x, y, ld_y, gate, shift, scale, ld_mod, h, ld_h, n_tok, \
                               dim, norm_kind, eps, s)
  if (chunks <= 64) H3_MR(64, 1);
  if (chunks <= 128) H3_MR(128, 1);
  if (chunks <= 256) H3_MR(256, 1);
  if (chunks <= 512) H3_MR(128, 4);
  if (chunks <= 640) H3_MR(128, 5);
  if (chunks <= 1024) H3_MR(256, 4);
  H3_MR(256, 8);  // dim <= 16384 (checked by the caller)
#undef H3_MR
}

template <int NT, int CPT>
static hipError_t launch_mr_mx(void* x, int64_t ld_x, const void* shift, const void* scale,
                               int64_t ld_mod, void* q, int64_t ld_q, void* qs, int64_t ld_s,
                               int64_t n_tok, int dim, int norm_kind, float eps, hipStream_t s) {
  hipLaunchKernelGGL((modres_kernel<bf16_t, NT, CPT, true>), dim3((unsigned)n_tok), dim3(NT), 0,
                     s, (bf16_t*)x, ld_x, nullptr, 0, nullptr, (const bf16_t*)shift,
                     (const bf16_t*)scale, ld_mod, nullptr, 0, dim, norm_kind, eps, (uint8_t*)q,
                     ld_q, (uint8_t*)qs, ld_s);
  return hipGetLastError();
}

hipError_t launch_modulate_mx(const void* x, int64_t ld_x, const void* shift, const void* scale,
                              int64_t ld_mod, void* q, int64_t ld_q, void* qs, int64_t ld_s,
                              int64_t n_tok, int dim, int norm_kind, float eps, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  if (dim % 32 != 0) return hipErrorInvalidValue;
  void* xm = const_cast<void*>(x);  // read only: the residual half of the kernel is compiled out
  const int chunks = dim / 8;
#define H3_MRX(NT, CPT) \
  return launch_mr_mx<NT, CPT>(xm, ld_x, shift, scale, ld_mod, q, ld_q, qs, ld_s, n_tok, dim, norm_kind, eps, s)
  if (chunks <= 64) H3_MRX(64, 1);
  if (chunks <= 128) H3_MRX(128, 1);
  if (chunks <= 256) H3_MRX(256, 1);
  if (chunks <= 512) H3_MRX(128, 4);
  if (chunks <= 640) H3_MRX(128, 5);
  if (chunks <= 1024) H3_MRX(256, 4);
  H3_MRX(256, 8);  // dim <= 16384 (checked by the caller)
#undef H3_MRX
}

hipError_t launch_modulate_residual(bool bf16, void* x, int64_t ld_x, const void* y,
                                    int64_t ld_y, const void* gate, const void* shift,
                                    const void* scale, int64_t ld_mod, void* h, int64_t ld_h,
                                    int64_t n_tok, int dim, int norm_kind, float eps,
                                    hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  if (bf16)
    return dispatch_mr<bf16_t>(x, ld_x, y, ld_y, gate, shift, scale, ld_mod, h, ld_h, n_tok, dim,
                               norm_kind, eps, s);
  return dispatch_mr<float>(x, ld_x, y, ld_y, gate, shift, scale, ld_mod, h, ld_h, n_tok, dim,
                            norm_kind, eps, s);
}

}  // namespace h3
