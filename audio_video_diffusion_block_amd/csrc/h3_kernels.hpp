// Internal launcher API between the C ABI (h3_api.cpp) and the kernel files.
// Every launcher enqueues on `s` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "h3_rope.hpp"

namespace h3 {

enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_RESIDUAL = 2 };

hipError_t launch_qk_norm_rope(bool bf16, int head_dim, void* q, int64_t ld_q, void* k,
                               int64_t ld_k, int64_t n_tok, int n_heads, const void* g_q,
                               const void* g_k, const void* pos, int sec_t, int sec_h,
                               float theta, float eps, hipStream_t s);

hipError_t launch_modulate_residual(bool bf16, void* x, int64_t ld_x, const void* y,
                                    int64_t ld_y, const void* gate, const void* shift,
                                    const void* scale, int64_t ld_mod, void* h, int64_t ld_h,
                                    int64_t n_tok, int dim, int norm_kind, float eps,
                                    hipStream_t s);
// modulated norm of x written as an MX e4m3 operand instead of bf16 (dim % 32 == 0)
hipError_t launch_modulate_mx(const void* x, int64_t ld_x, const void* shift, const void* scale,
                              int64_t ld_mod, void* q, int64_t ld_q, void* qs, int64_t ld_s,
                              int64_t n_tok, int dim, int norm_kind, float eps, hipStream_t s);

// Optional operand layouts of the bf16 K % 64 == 0 GEMM (sequence-parallel
// exchange buffers).  All zero: plain row-major A and C.
struct GemmMap {
  // A is grouped along K: columns [g*a_kgroup, (g+1)*a_kgroup) of row m sit at
  // A + g*a_gstride + m*lda (lda == a_kgroup); a_kgroup % 64 == 0
  int a_kgroup = 0;
  int64_t a_gstride = 0;
  // EPI_STORE scatter: output column n = (which*H + h)*D + d of row m goes to
  // C + ((p*M + m)*3 + which)*hc*D + j*D + d with h = p*hc + j (peer-major)
  int peer_H = 0, peer_hc = 0, peer_D = 0;
  // EPI_SWIGLU (N % 32 == 0): the bf16 output is also written as an MX e4m3
  // operand (mx_q bytes, row stride mx_ld; one E8M0 byte per 32 columns at mx_s,
  // row stride mx_lds), the same bytes as quantizing the stored bf16 output
  uint8_t* mx_q = nullptr;
  int64_t mx_ld = 0;
  uint8_t* mx_s = nullptr;
  int64_t mx_lds = 0;
  // with mx_q: only the MX operand is written (C is not touched and may be NULL)
  bool mx_only = false;
  // EPI_STORE of a QKV projection (N = 3*qk_H*qk_D, qk_D in {64, 128}): the q
  // and k head columns (n < 2*qk_H*qk_D) of rows whose qk_pos kind is video or
  // audio get Q/K RMSNorm (gains qk_gq, qk_gk) and RoPE before they are
  // stored, from their bf16-rounded values, exactly as the standalone pass
  // would; other rows and the v columns are stored as computed
  const int4* qk_pos = nullptr;
  const bf16_t* qk_gq = nullptr;
  const bf16_t* qk_gk = nullptr;
  int qk_H = 0, qk_D = 0;
  float qk_eps = 0.f;
  RopeTab qk_tab{};
  bool empty() const {
    return a_kgroup == 0 && peer_hc == 0 && mx_q == nullptr && !mx_only && qk_pos == nullptr;
  }
};

// out = A @ B^T with epilogue; for EPI_SWIGLU, B = W1, B3 = W3 and N = features
hipError_t launch_gemm(bool bf16, int epi, const void* A, int64_t lda, const void* B,
                       const void* B3, int64_t ldb, void* C, int64_t ldc, const void* gate,
                       int64_t ld_gate, int64_t M, int N, int K, hipStream_t s,
                       const GemmMap& map = GemmMap{});

// MX-scaled e4m3 operand (layout in k_gemm_fp8.hip): e4m3 data [rows][ld]
// bytes with round_up(K, 128) columns, zeros past K, and E8M0 scale bytes
// [rows][ld_scale], one per 32 columns
struct MxOperand {
  const void* data = nullptr;
  int64_t ld = 0;
  const void* scale = nullptr;
  int64_t ld_scale = 0;
};

// bf16 x [rows][cols] (cols % 32 == 0) -> MX operand (q, scale); kgroup > 0:
// columns [g*kgroup, (g+1)*kgroup) of row r at x + g*gstride + r*ld_x (elements)
hipError_t launch_mx_quantize(const void* x, int64_t ld_x, int64_t rows, int cols, void* q,
                              int64_t ld_q, void* scale, int64_t ld_s, hipStream_t s,
                              int kgroup = 0, int64_t gstride = 0);
// bf16 out = A @ B^T over MX operands (K the logical contraction length); for
// EPI_SWIGLU, b = W1, b3 = W3 (same ld and ld_scale) and N = features
hipError_t launch_gemm_mx8(int epi, const MxOperand& a, const MxOperand& b, const MxOperand& b3,
                           void* C, int64_t ldc, const void* gate, int64_t ld_gate, int64_t M,
                           int N, int K, hipStream_t s, const GemmMap& map = GemmMap{});

size_t attn_workspace_bytes(bool bf16, int64_t n_buf, int n_heads, int head_dim, int n_seg);
hipError_t launch_varlen_attn(bool bf16, int head_dim, const void* q, int64_t ld_q,
                              const void* k, int64_t ld_k, const void* v, int64_t ld_v, void* o,
                              int64_t ld_o, int64_t n_buf, int n_heads, const int* cu,
                              const int* valid, int n_seg, int max_len, float scale, void* ws,
                              hipStream_t s);

// bf16 attention with Skip-Softmax (skip_log2 < 0; -inf never skips); same
// workspace as launch_varlen_attn
hipError_t launch_varlen_attn_skip(int head_dim, const void* q, int64_t ld_q, const void* k,
                                   int64_t ld_k, const void* v, int64_t ld_v, void* o,
                                   int64_t ld_o, int64_t n_buf, int n_heads, const int* cu,
                                   const int* valid, int n_seg, int max_len, float scale,
                                   float skip_log2, void* ws, hipStream_t s);

// FP8 (MX-scaled e4m3) attention: bf16 q, k, v, o as above; workspace holds
// the quantized operands and their block scales.  skip_log2 < 0: with the
// Skip-Softmax rule at that threshold; 0: without it
size_t attn_fp8_workspace_bytes(int64_t n_buf, int n_heads, int head_dim, int n_seg);
hipError_t launch_varlen_attn_fp8(int head_dim, const void* q, int64_t ld_q, const void* k,
                                  int64_t ld_k, const void* v, int64_t ld_v, void* o,
                                  int64_t ld_o, int64_t n_buf, int n_heads, const int* cu,
                                  const int* valid, int n_seg, int max_len, float scale,
                                  float skip_log2, void* ws, hipStream_t s);

// strides and group sizes in BYTES (multiples of 16)
hipError_t launch_copy_rows(const void* src, int64_t ld_src, int64_t gs_src, void* dst,
                            int64_t ld_dst, int64_t gs_dst, int64_t rows, int groups,
                            int64_t bytes_per_group, hipStream_t s);

hipError_t launch_euler(bool bf16, void* z, const void* u, void* x_next, int64_t n, float dsig,
                        hipStream_t s);

hipError_t launch_timestep(bool bf16, float sigma, const void* w1, const void* w2,
                           const void* table, void* mod_out, int n_blocks, int dim, int emb,
                           void* ws, hipStream_t s);

// decoded frames [B][3][T][H][W] fp32 -> uint8, layout 0 [B][T][H][W][3], 1 [B][T][3][H][W]
hipError_t launch_frames_u8(const float* in, uint8_t* out, int64_t B, int64_t T, int64_t H,
                            int64_t W, int layout, hipStream_t s);

}  // namespace h3
