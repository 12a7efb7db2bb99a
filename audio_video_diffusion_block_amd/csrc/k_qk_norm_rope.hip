// Fused Q/K RMSNorm + RoPE, in place on the q and k regions of a QKV buffer.
//
// Why Real-Time MiniMax H3 Serving Requires More Than a Faster DiT, "Key
// takeaways": Q/K RMSNorm and RoPE are one fused operation, and a rank computes
// RoPE only for its own rows.
//
// HBM-bound pass.  A head row (D values) is owned by D/8 adjacent lanes, 8
// values (16 bytes of bf16) per lane, so four consecutive head rows of a token
// are one contiguous 1 KiB wave access.  The sum of squares is reduced across
// the D/8 lanes with DPP.  A lane always owns the same 4 RoPE pairs, whose
// per-position rotations come from the host-computed table (h3_rope.hpp), and
// recomputes cos/sin only when its token changes (each work-group walks a
// contiguous run of rows, so that happens every 2H/(256/(D/8)) rows).  The
// arithmetic is the one the QKV projection's fused epilogue uses, so both
// give the same bits.  A lane
// takes U rows per step (SLOTS rows apart) and issues their loads before
// processing the first; loads and stores carry the non-temporal hint.  On a
// [n, 3, H, D] bf16 buffer this runs at the rate of a plain in-place
// read-modify-write of the same q and k regions.
#include "h3_common.hpp"
#include "h3_kernels.hpp"
#include "h3_rope.hpp"

namespace h3 {

template <typename T, int D, int U>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(
    T* __restrict__ q, int64_t ld_q, T* __restrict__ k, int64_t ld_k, int64_t n_tok, int n_heads,
    const T* __restrict__ g_q, const T* __restrict__ g_k, const int4* __restrict__ pos,
    RopeTab tab, float eps, int64_t rows_per_block) {
  constexpr int L = D / 8;          // lanes per head row
  constexpr int SLOTS = 256 / L;    // head rows in flight per work-group
  const int lane = threadIdx.x % L;
  const int slot = threadIdx.x / L;
  const RopeLane rl = rope_lane(tab, lane);

  float gq[8], gk[8];
  Vec8<T>::load(g_q + 8 * lane, gq);
  Vec8<T>::load(g_k + 8 * lane, gk);

  const int64_t rows_per_tok = 2 * (int64_t)n_heads;
  const int64_t total = n_tok * rows_per_tok;
  const int64_t begin = (int64_t)blockIdx.x * rows_per_block;
  const int64_t end = min(total, begin + rows_per_block);

  int64_t cur_tok = -1;
  int kind = 2;
  float cs[4], sn[4];
  // U rows per step, SLOTS rows apart: all U loads are issued before the first
  // row is processed, and its stores follow
  for (int64_t r0 = begin + slot; r0 < end; r0 += U * SLOTS) {
    T* ptr[U];
    int64_t tok[U];
    bool is_k[U];
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + u * SLOTS;
      const int64_t rc = r < end ? r : r0;  // past the end: a harmless re-read of row r0
      tok[u] = rc / rows_per_tok;
      const int rr = (int)(rc - tok[u] * rows_per_tok);
      is_k[u] = rr >= n_heads;
      const int head = is_k[u] ? rr - n_heads : rr;
      ptr[u] = (is_k[u] ? k + tok[u] * ld_k : q + tok[u] * ld_q) + (int64_t)head * D + 8 * lane;
      Vec8<T>::load_nt(ptr[u], v[u]);  // pad rows are read too (in the buffer), never written
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (r0 + u * SLOTS >= end) break;
      if (tok[u] != cur_tok) {
        cur_tok = tok[u];
        const int4 p = pos[cur_tok];
        kind = p.x;
        rope_cos_sin(rl, p, cs, sn);
      }
      if (kind != 0 && kind != 1) continue;  // pad row: untouched
      qk_norm_rope_lane<L>(v[u], is_k[u] ? gk : gq, cs, sn, eps);
      Vec8<T>::store_nt(ptr[u], v[u]);
    }
  }
}

// One work-group per token, for tokens of 256 or more 16-byte chunks (2H x D/8):
// every chunk of the token's q and k rows is loaded before any arithmetic, CPT
// per thread (thread t holds chunks t, t + 256, ...; 256 is a multiple of D/8,
// so a thread's chunks all sit at the same place in their head rows and need
// the same 4 rotation pairs).  Measured ~2.5% faster than the row walk above
// at 40 heads of 128.
template <typename T, int D, int CPT>
__global__ __launch_bounds__(256) void qk_norm_rope_tok_kernel(
    T* __restrict__ q, int64_t ld_q, T* __restrict__ k, int64_t ld_k, int n_heads,
    const T* __restrict__ g_q, const T* __restrict__ g_k, const int4* __restrict__ pos,
    RopeTab tab, float eps) {
  constexpr int L = D / 8;  // lanes per head row
  const int64_t tok = blockIdx.x;
  const int lane = threadIdx.x % L;
  const int chunks = 2 * n_heads * L;
  const int4 ps = pos[tok];
  if (ps.x != 0 && ps.x != 1) return;  // pad row: untouched
  float v[CPT][8];
  T* ptr[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * 256;
    if (c < chunks) {  // whole head rows are in or out (chunks and 256 are multiples of L)
      const int row = c / L;
      const bool is_k = row >= n_heads;
      ptr[i] = (is_k ? k + tok * ld_k + (int64_t)(row - n_heads) * D
                     : q + tok * ld_q + (int64_t)row * D) + 8 * lane;
      Vec8<T>::load_nt(ptr[i], v[i]);
    }
  }
  // this thread's 4 pairs
  float cs[4], sn[4];
  rope_cos_sin(rope_lane(tab, lane), ps, cs, sn);
  float gq[8], gk[8];
  Vec8<T>::load(g_q + 8 * lane, gq);
  Vec8<T>::load(g_k + 8 * lane, gk);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * 256;
    if (c < chunks) {
      const bool is_k = c / L >= n_heads;
      qk_norm_rope_lane<L>(v[i], is_k ? gk : gq, cs, sn, eps);
      Vec8<T>::store_nt(ptr[i], v[i]);
    }
  }
}

template <typename T, int D>
static hipError_t launch_qk(void* q, int64_t ld_q, void* k, int64_t ld_k, int64_t n_tok,
                            int n_heads, const void* g_q, const void* g_k, const void* pos,
                            int sec_t, int sec_h, float theta, float eps, hipStream_t s) {
  constexpr int L = D / 8;
  constexpr int SLOTS = 256 / L;
  const int64_t total = n_tok * 2 * (int64_t)n_heads;
  const int64_t rows_per_block = (int64_t)SLOTS * 8;  // two steps of four rows per lane
  const int64_t blocks = ceil_div(total, rows_per_block);
  const int64_t chunks = 2 * (int64_t)n_heads * L;
  const RopeTab tab = make_rope_tab(D, sec_t, sec_h, theta);
  if (chunks >= 256 && chunks <= 8 * 256 && n_tok <= 0x7fffffff) {
#define H3_QKT(CPT)                                                                             \
  hipLaunchKernelGGL((qk_norm_rope_tok_kernel<T, D, CPT>), dim3((unsigned)n_tok), dim3(256), 0, s, \
                     (T*)q, ld_q, (T*)k, ld_k, n_heads, (const T*)g_q, (const T*)g_k,            \
                     (const int4*)pos, tab, eps);                                                \
  return hipGetLastError()
    switch ((int)ceil_div(chunks, 256)) {
      case 1: H3_QKT(1);
      case 2: H3_QKT(2);
      case 3: H3_QKT(3);
      case 4: H3_QKT(4);
      case 5: H3_QKT(5);
      case 6: H3_QKT(6);
      case 7: H3_QKT(7);
      default: H3_QKT(8);
    }
#undef H3_QKT
  }
  hipLaunchKernelGGL((qk_norm_rope_kernel<T, D, 4>), dim3((unsigned)blocks), dim3(256), 0, s,
                     (T*)q, ld_q, (T*)k, ld_k, n_tok, n_heads, (const T*)g_q, (const T*)g_k,
                     (const int4*)pos, tab, eps, rows_per_block);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(bool bf16, int head_dim, void* q, int64_t ld_q, void* k,
                               int64_t ld_k, int64_t n_tok, int n_heads, const void* g_q,
                               const void* g_k, const void* pos, int sec_t, int sec_h,
                               float theta, float eps, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  if (bf16) {
    if (head_dim == 128)
      return launch_qk<bf16_t, 128>(q, ld_q, k, ld_k, n_tok, n_heads, g_q, g_k, pos, sec_t, sec_h,
                                    theta, eps, s);
    return launch_qk<bf16_t, 64>(q, ld_q, k, ld_k, n_tok, n_heads, g_q, g_k, pos, sec_t, sec_h,
                                 theta, eps, s);
  }
  if (head_dim == 128)
    return launch_qk<float, 128>(q, ld_q, k, ld_k, n_tok, n_heads, g_q, g_k, pos, sec_t, sec_h,
                                 theta, eps, s);
  return launch_qk<float, 64>(q, ld_q, k, ld_k, n_tok, n_heads, g_q, g_k, pos, sec_t, sec_h,
                              theta, eps, s);
}

}  // namespace h3
