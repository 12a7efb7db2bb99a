// Output-frame conversion: decoded fp32 video -> compact uint8.
//
// Why Real-Time MiniMax H3 Serving Requires More Than a Faster DiT, "Key
// takeaways" (decoding and media output): decoded frames are converted on the
// GPU, once, into contiguous uint8 BTHWC data, and the encoder is fed through
// planar paths without building another interleaved buffer.
//
// Value rule (fp32, in this order): v = x * 0.5 + 0.5; v = clamp(v, 0, 1) with
// NaN -> 0; u = round_half_even(v * 255).
// Input [B][3][T][H][W] fp32 (channel-first decoder output).  Output layout 0:
// [B][T][H][W][3] (interleaved RGB); layout 1: [B][T][3][H][W] (one plane per
// channel and frame).
//
// One thread converts 16 consecutive pixels of one image row: three 64-byte
// channel reads and 48 (interleaved) or 3 x 16 (planar) output bytes, so a
// wave reads 3 x 4 KB and writes 3 KB contiguously.  Rows whose width is not
// a multiple of 16 take an element-wise path.
#include "h3_common.hpp"
#include "h3_kernels.hpp"

namespace h3 {

namespace {

__device__ __forceinline__ uint32_t to_u8(float x) {
  float v = fmaf(x, 0.5f, 0.5f);     // x * 0.5 is exact: one rounding, as x * 0.5 + 0.5
  v = fminf(fmaxf(v, 0.0f), 1.0f);   // max(NaN, 0) = 0
  return (uint32_t)__builtin_rintf(v * 255.0f);
}

template <int LAYOUT, bool VEC>
__global__ __launch_bounds__(256) void frames_u8_kernel(const float* __restrict__ in,
                                                         uint8_t* __restrict__ out, int64_t T,
                                                         int64_t H, int64_t W, int64_t rows,
                                                         int64_t cpr) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = g / cpr;  // (b, t, h)
  if (row >= rows) return;
  const int64_t w0 = (g - row * cpr) * 16;
  const int64_t th = T * H, hw = H * W;
  const int64_t b = row / th, rem = row - b * th;
  const int64_t t = rem / H, h = rem - t * H;
  const int64_t plane = T * hw;  // one channel of one video
  const float* src = in + b * 3 * plane + t * hw + h * W + w0;
  if constexpr (VEC) {
    uint32_t q[3][16];
#pragma unroll
    for (int ch = 0; ch < 3; ++ch) {
      const float4* p = reinterpret_cast<const float4*>(src + ch * plane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = p[i];
        q[ch][4 * i + 0] = to_u8(v.x);
        q[ch][4 * i + 1] = to_u8(v.y);
        q[ch][4 * i + 2] = to_u8(v.z);
        q[ch][4 * i + 3] = to_u8(v.w);
      }
    }
    if constexpr (LAYOUT == 0) {
      // 16 pixels x RGB = 48 bytes = 12 words, byte k = pixel k/3, channel k%3
      uint32_t w[12];
#pragma unroll
      for (int k = 0; k < 12; ++k) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int byte = 4 * k + j;
          word |= q[byte % 3][byte / 3] << (8 * j);
        }
        w[k] = word;
      }
      uint4* dst = reinterpret_cast<uint4*>(out + (row * W + w0) * 3);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      dst[2] = make_uint4(w[8], w[9], w[10], w[11]);
    } else {
      uint8_t* base = out + (b * T + t) * 3 * hw + h * W + w0;
#pragma unroll
      for (int ch = 0; ch < 3; ++ch) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[k] = q[ch][4 * k] | (q[ch][4 * k + 1] << 8) | (q[ch][4 * k + 2] << 16) |
                 (q[ch][4 * k + 3] << 24);
        *reinterpret_cast<uint4*>(base + ch * hw) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  } else {
    const int n = (int)min((int64_t)16, W - w0);
    for (int i = 0; i < n; ++i) {
#pragma unroll
      for (int ch = 0; ch < 3; ++ch) {
        const uint8_t u = (uint8_t)to_u8(src[ch * plane + i]);
        if constexpr (LAYOUT == 0) out[(row * W + w0 + i) * 3 + ch] = u;
        else out[(b * T + t) * 3 * hw + ch * hw + h * W + w0 + i] = u;
      }
    }
  }
}

}  // namespace

hipError_t launch_frames_u8(const float* in, uint8_t* out, int64_t B, int64_t T, int64_t H,
                            int64_t W, int layout, hipStream_t s) {
  const int64_t rows = B * T * H;
  if (rows == 0 || W == 0) return hipSuccess;
  const int64_t cpr = (W + 15) / 16;
  const int64_t threads = rows * cpr;
  const dim3 grid((unsigned)((threads + 255) / 256));
  const bool vec = W % 16 == 0;
#define H3_F(L, V) \
  hipLaunchKernelGGL((frames_u8_kernel<L, V>), grid, dim3(256), 0, s, in, out, T, H, W, rows, cpr)
  if (layout == 0) {
    if (vec) H3_F(0, true); else H3_F(0, false);
  } else {
    if (vec) H3_F(1, true); else H3_F(1, false);
  }
#undef H3_F
  return hipGetLastError();
}

}  // namespace h3
