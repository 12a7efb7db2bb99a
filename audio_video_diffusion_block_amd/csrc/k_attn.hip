// Variable-length attention over a packed buffer of segments.
//
// Why Real-Time MiniMax H3 Serving Requires More Than a Faster DiT, "Key
// takeaways": attention on the packed audio-video sequence runs over valid
// sequence lengths with the structural suffix padding removed.
//
// bf16 path (gfx950 MFMA flash attention, forward):
//  * One work-group = NW waves = one (segment, head, 32*NW-row query tile).
//    Each wave owns 32 query rows for the whole key loop; its Q fragments stay
//    in registers.
//  * Keys stream in tiles of 64 through LDS, double buffered: K as [64][D]
//    (d contiguous) and V pre-transposed to [D][64] (keys contiguous) by a
//    separate pass into scratch, so both MFMA operands are plain 16-byte LDS
//    reads.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16, A =
//    K from LDS, B = Q^T from registers).  Each lane then holds 32 scores of ONE
//    query row (q = lane % 32): the row max/sum need only lane-local work plus
//    one exchange with lane ^ 32.  The K rows are read in a permuted order so
//    that the accumulator's key order matches, register for register, the
//    B-operand order of the P.V product; P is converted to bf16 in registers
//    and feeds O^T += V^T P^T directly (no LDS round trip).
//  * Online softmax in the log2 domain (scale*log2(e) folded into one FMA).
//    The running max is raised only when a row max exceeds it by more than 8
//    (2^8 bound on unnormalised weights), so the O rescale is skipped on most
//    tiles; the final 1/l uses the same stale max, so the result is exact.
//  * Keys beyond the valid length are zero-filled in LDS (K) / scratch (V^T)
//    and their scores masked to -inf, so NaN/Inf pad rows never reach a product.
//  * No atomics, no split over keys: the result is deterministic.
//
// fp32 path: one thread per (query row, head), plain online softmax.
#include "h3_common.hpp"
#include "h3_kernels.hpp"

namespace h3 {

// --------------------------------------------------------------- helpers

// segment of buffer row r: largest s with cu[s] <= r, or -1 (n_seg is small)
__device__ __forceinline__ int find_segment(const int* cu, int n_seg, int64_t r) {
  int lo = 0, hi = n_seg;  // cu[lo] <= r < cu[hi] invariant when in range
  if (r < cu[0] || r >= cu[n_seg]) return -1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int seg_valid(const int* cu, const int* valid, int s) {
  return valid ? valid[s] : cu[s + 1] - cu[s];
}

// Write 0 to every row of o that is not a valid row of some segment.
template <typename T>
__global__ __launch_bounds__(256) void zero_pad_rows_kernel(T* o, int64_t ld_o, int64_t n_buf,
                                                            int width, const int* cu,
                                                            const int* valid, int n_seg) {
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  if (r >= n_buf) return;
  const int s = find_segment(cu, n_seg, r);
  if (s >= 0 && r - cu[s] < seg_valid(cu, valid, s)) return;
  T* row = o + r * ld_o;
  for (int c = threadIdx.x % 64; c < width; c += 64) row[c] = T(0);
}

// V [rows, H*D] (row stride ld_v) -> V^T scratch [H][D][cols]: for segment s,
// key j (< round_up(valid, 64)) lands at column vt_segment_base(cu[s], s) + j;
// keys >= valid are written as zeros.  One work-group transposes 64 keys x D
// dims of one head through LDS.
template <int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(const bf16_t* __restrict__ v,
                                                          int64_t ld_v, bf16_t* __restrict__ vt,
                                                          int64_t cols, const int* cu,
                                                          const int* valid) {
  __shared__ bf16_t tile[64][D + 8];
  const int s = blockIdx.y;
  const int head = blockIdx.z;
  const int lo = cu[s];
  const int len = seg_valid(cu, valid, s);
  const int j0 = blockIdx.x * 64;
  if (j0 >= len) return;
  // load 64 rows x D (16-byte chunks)
  constexpr int CPR = D / 8;
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int r = i / CPR, c = i % CPR;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (j0 + r < len)
      val = *reinterpret_cast<const uint4*>(v + (int64_t)(lo + j0 + r) * ld_v + head * D + c * 8);
    const bf16_t* e = reinterpret_cast<const bf16_t*>(&val);
#pragma unroll
    for (int t = 0; t < 8; ++t) tile[r][c * 8 + t] = e[t];
  }
  __syncthreads();
  // write D rows x 64 keys (8 chunks of 8 keys per row)
  const int64_t base = vt_segment_base(lo, s) + j0;
  bf16_t* dst = vt + (int64_t)head * D * cols + base;
  for (int i = threadIdx.x; i < D * 8; i += 256) {
    const int d = i / 8, c = i % 8;
    uint4 val;
    bf16_t* e = reinterpret_cast<bf16_t*>(&val);
#pragma unroll
    for (int t = 0; t < 8; ++t) e[t] = tile[c * 8 + t][d];
    *reinterpret_cast<uint4*>(dst + (int64_t)d * cols + c * 8) = val;
  }
}

// ------------------------------------------------------------ MFMA kernel

namespace {
constexpr int KT = 64;  // keys per tile

// K tile in LDS: [64 keys][D], the D/8 16-byte chunks of a row swizzled by the row
template <int D>
__device__ __forceinline__ int k_off(int row, int chunk) {
  return row * D + ((chunk ^ (row & (D / 8 - 1))) << 3);
}
// V^T tile in LDS: [D][64 keys], 8 chunks per row swizzled by (row & 7)
__device__ __forceinline__ int vt_off(int row, int chunk) {
  return row * KT + ((chunk ^ (row & 7)) << 3);
}

// Accumulator row i of a 32x32 MFMA tile (lane half h, register r) is
// i = (r/4)*8 + h*4 + r%4.  Reading K row sigma(i) into A-operand row i makes
// register r of lane half h hold key (r/8)*16 + h*8 + r%8, i.e. registers
// 0..7 are keys h*8..h*8+7 and registers 8..15 keys 16+h*8.., which is the
// B-operand order of the P.V MFMA over keys 0..15 and 16..31.
__device__ __forceinline__ int sigma_row(int i) {
  const int a = i >> 3;
  return (a >> 1) * 16 + ((i >> 2) & 1) * 8 + (a & 1) * 4 + (i & 3);
}
}  // namespace

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_bf16_kernel(
    const bf16_t* __restrict__ q, int64_t ld_q, const bf16_t* __restrict__ k, int64_t ld_k,
    const bf16_t* __restrict__ vt, int64_t vt_cols, bf16_t* __restrict__ o, int64_t ld_o,
    const int* __restrict__ cu, const int* __restrict__ valid, float scale_log2) {
  constexpr int BMQ = NW * 32;
  constexpr int NTH = NW * 64;
  constexpr int KCH = D / 8;  // 16-byte chunks per K row
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][KT * D];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][D * KT];

  const int s = blockIdx.y;
  const int head = blockIdx.z;
  const int seg_lo = cu[s];
  const int len = seg_valid(cu, valid, s);
  const int q0 = blockIdx.x * BMQ;
  if (q0 >= len) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qi = lane & 31;   // this lane's query row within the wave
  const int hf = lane >> 5;   // lane half
  const int qrow = q0 + wave * 32 + qi;
  const bool q_ok = qrow < len;

  // ---- Q fragments: B operand of S^T = K Q^T, k-block kk covers d = kk*16 + hf*8 .. +8
  bf16x8_t qf[D / 16];
  {
    const bf16_t* qp = q + (int64_t)(seg_lo + (q_ok ? qrow : 0)) * ld_q + head * D + hf * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 val = q_ok ? *reinterpret_cast<const uint4*>(qp + kk * 16) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8_t, val);
    }
  }

  // ---- tile loaders: K 64 x D and V^T D x 64, 16-byte chunks
  constexpr int K_CHUNKS = KT * KCH;   // 1024 for D=128
  constexpr int V_CHUNKS = D * 8;      // 1024 for D=128
  constexpr int KPT = K_CHUNKS / NTH;  // per thread
  constexpr int VPT = V_CHUNKS / NTH;
  static_assert(K_CHUNKS % NTH == 0 && V_CHUNKS % NTH == 0, "tile split");
  const bf16_t* kbase = k + (int64_t)seg_lo * ld_k + head * D;
  const bf16_t* vbase = vt + (int64_t)head * D * vt_cols + vt_segment_base(seg_lo, s);
  uint4 rk[KPT], rv[VPT];
  auto load_tile = [&](int jt) {
    const int j0 = jt * KT;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NTH;
      const int r = c / KCH, ch = c % KCH;
      rk[i] = (j0 + r < len) ? *reinterpret_cast<const uint4*>(kbase + (int64_t)(j0 + r) * ld_k + ch * 8)
                             : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NTH;
      const int r = c / 8, ch = c % 8;
      rv[i] = *reinterpret_cast<const uint4*>(vbase + (int64_t)r * vt_cols + j0 + ch * 8);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NTH;
      *reinterpret_cast<uint4*>(&Ks[buf][k_off<D>(c / KCH, c % KCH)]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NTH;
      *reinterpret_cast<uint4*>(&Vs[buf][vt_off(c / 8, c % 8)]) = rv[i];
    }
  };

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY;  // running max of scaled scores (log2 domain)
  float l_run = 0.f;        // this lane's partial row sum

  const int n_tiles = (len + KT - 1) / KT;
  const int krow = sigma_row(qi);  // permuted K row read by this lane
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int jt = 0; jt < n_tiles; ++jt) {
    const int buf = jt & 1;
    if (jt + 1 < n_tiles) load_tile(jt + 1);

    // S^T for keys [0,32) and [32,64) of the tile
    f32x16_t sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            &Ks[buf][k_off<D>(kb * 32 + krow, kk * 2 + hf)]);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sc[kb], 0, 0, 0);
      }
    }
    // mask keys >= len (only the last tile can hold them)
    if ((jt + 1) * KT > len) {
      const int base = jt * KT;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = base + kb * 32 + (r >> 3) * 16 + hf * 8 + (r & 7);
          if (key >= len) sc[kb][r] = -INFINITY;
        }
    }
    // row max over the tile: lane-local, then with the partner lane (same query)
    float mx = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mx_s = mx * scale_log2;
    // raise the running max only when it is exceeded by more than 8 (log2 units)
    const bool raise = mx_s > m_run + 8.0f;
    if (__any(raise)) {
      const float m_new = raise ? mx_s : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // exp2(-inf) = 0 on the first tile
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    // P = exp2(s*scale_log2 - m), partial row sums, bf16 B operands
    bf16x8_t pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kb][half * 8 + 2 * t], scale_log2, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kb][half * 8 + 2 * t + 1], scale_log2, -m_run));
          l_run += p0 + p1;
          w[t] = pack_bf16x2(p0, p1);
        }
        pb[kb][half] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      }
    }
    // O^T += V^T P^T : d blocks of 32, keys in 4 blocks of 16
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int chunk = kb * 4 + half * 2 + hf;  // keys kb*32 + half*16 + hf*8 .. +8
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&Vs[buf][vt_off(db * 32 + qi, chunk)]);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][half], oacc[db], 0, 0, 0);
        }
      }
    }
    if (jt + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: lane holds query qi, d = db*32 + (r/4)*8 + hf*4 + r%4
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!q_ok) return;
  const float inv = 1.0f / l_tot;
  bf16_t* op = o + (int64_t)(seg_lo + qrow) * ld_o + head * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + hf * 4;
      uint2 val;
      val.x = pack_bf16x2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
      val.y = pack_bf16x2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d) = val;
    }
  }
}

// ------------------------------------------------------------ fp32 path

template <int D>
__global__ __launch_bounds__(128) void attn_fwd_f32_kernel(
    const float* __restrict__ q, int64_t ld_q, const float* __restrict__ k, int64_t ld_k,
    const float* __restrict__ v, int64_t ld_v, float* __restrict__ o, int64_t ld_o,
    const int* __restrict__ cu, const int* __restrict__ valid, float scale) {
  const int s = blockIdx.y, head = blockIdx.z;
  const int seg_lo = cu[s];
  const int len = seg_valid(cu, valid, s);
  const int i = blockIdx.x * 128 + threadIdx.x;
  if (i >= len) return;
  float qv[D], acc[D];
  const float* qp = q + (int64_t)(seg_lo + i) * ld_q + head * D;
  for (int d = 0; d < D; ++d) { qv[d] = qp[d]; acc[d] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < len; ++j) {
    const float* kp = k + (int64_t)(seg_lo + j) * ld_k + head * D;
    float sdot = 0.f;
    for (int d = 0; d < D; ++d) sdot += qv[d] * kp[d];
    sdot *= scale;
    const float m_new = fmaxf(m, sdot);
    const float alpha = expf(m - m_new);
    const float p = expf(sdot - m_new);
    const float* vp = v + (int64_t)(seg_lo + j) * ld_v + head * D;
    l = l * alpha + p;
    for (int d = 0; d < D; ++d) acc[d] = acc[d] * alpha + p * vp[d];
    m = m_new;
  }
  float* op = o + (int64_t)(seg_lo + i) * ld_o + head * D;
  for (int d = 0; d < D; ++d) op[d] = acc[d] / l;
}

// ------------------------------------------------------------ launcher

template <int D>
static hipError_t launch_attn_d(bool bf16, const void* q, int64_t ld_q, const void* k,
                                int64_t ld_k, const void* v, int64_t ld_v, void* o,
                                int64_t ld_o, int64_t n_buf, int n_heads, const int* cu,
                                const int* valid, int n_seg, int max_len, float scale, void* ws,
                                hipStream_t s) {
  if (n_buf == 0) return hipSuccess;
  // rows that are not valid rows of any segment get zeros
  const unsigned zblocks = (unsigned)ceil_div(n_buf, 4);
  if (bf16) {
    hipLaunchKernelGGL((zero_pad_rows_kernel<bf16_t>), dim3(zblocks), dim3(256), 0, s,
                       (bf16_t*)o, ld_o, n_buf, n_heads * D, cu, valid, n_seg);
  } else {
    hipLaunchKernelGGL((zero_pad_rows_kernel<float>), dim3(zblocks), dim3(256), 0, s, (float*)o,
                       ld_o, n_buf, n_heads * D, cu, valid, n_seg);
  }
  if (max_len == 0) return hipGetLastError();
  if (bf16) {
    const int64_t cols = vt_columns(n_buf, n_seg);
    hipLaunchKernelGGL((transpose_v_kernel<D>), dim3((unsigned)ceil_div(max_len, 64), n_seg, n_heads),
                       dim3(256), 0, s, (const bf16_t*)v, ld_v, (bf16_t*)ws, cols, cu, valid);
    constexpr int NW = 4;
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW>),
                       dim3((unsigned)ceil_div(max_len, NW * 32), n_seg, n_heads), dim3(NW * 64), 0,
                       s, (const bf16_t*)q, ld_q, (const bf16_t*)k, ld_k, (const bf16_t*)ws, cols,
                       (bf16_t*)o, ld_o, cu, valid, scale_log2);
  } else {
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D>), dim3((unsigned)ceil_div(max_len, 128), n_seg, n_heads),
                       dim3(128), 0, s, (const float*)q, ld_q, (const float*)k, ld_k,
                       (const float*)v, ld_v, (float*)o, ld_o, cu, valid, scale);
  }
  return hipGetLastError();
}

size_t attn_workspace_bytes(bool bf16, int64_t n_buf, int n_heads, int head_dim, int n_seg) {
  if (!bf16) return 0;
  return (size_t)n_heads * head_dim * vt_columns(n_buf, n_seg) * sizeof(bf16_t);
}

hipError_t launch_varlen_attn(bool bf16, int head_dim, const void* q, int64_t ld_q,
                              const void* k, int64_t ld_k, const void* v, int64_t ld_v, void* o,
                              int64_t ld_o, int64_t n_buf, int n_heads, const int* cu,
                              const int* valid, int n_seg, int max_len, float scale, void* ws,
                              hipStream_t s) {
  if (head_dim == 128)
    return launch_attn_d<128>(bf16, q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, cu, valid,
                              n_seg, max_len, scale, ws, s);
  return launch_attn_d<64>(bf16, q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, cu, valid,
                           n_seg, max_len, scale, ws, s);
}

}  // namespace h3
