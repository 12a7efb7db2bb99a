// GEMMs of the block: out = A @ B^T with A [M, K] activations and B [N, K]
// weights (torch Linear layout, both operands K-contiguous), fp32 accumulation,
// and three epilogues:
//   EPI_STORE     out = acc
//   EPI_SWIGLU    out = silu(acc_w1) * acc_w3   (W1 and W3 columns of the same
//                 output feature computed by the same wave)
//   EPI_RESIDUAL  out = out + gate * acc        (gated residual, in place)
//
// Why Real-Time MiniMax H3 Serving Requires More Than a Faster DiT, "Key
// takeaways": SwiGLU and residual updates are fused into neighbouring work.
//
// bf16 path (MFMA, gfx950): 256x256 output tile (256x128 for SwiGLU), K step
// 64.  Two kernels: the general one (any K multiple of 8: 512 threads = 8
// waves as 2 (M) x 4 (N), each wave 128x64 from 4x2 v_mfma_f32_32x32x16_bf16
// tiles, A and B staged through registers into LDS with the 16-byte chunk
// index XOR-swizzled by the row) and the K % 64 == 0 one (every shape of the
// block), described where it is defined.  The general kernel addresses in 64
// bits and also takes K % 64 == 0 calls whose row strides exceed 2^22 elements.
// The next K tile is fetched into registers while the current one is
// multiplied.  Work-group ids are remapped so that the tiles one XCD runs at
// a time form a compact 4 (M) x 8 (N) patch: their A and B panels are then
// shared in that XCD's L2.
//
// fp32 path: a plain LDS-tiled FMA kernel (small problems, parity runs).
#include "h3_common.hpp"
#include "h3_kernels.hpp"
#include "h3_gemm_tile.hpp"

namespace h3 {

using gemm_tile::silu_f;
using gemm_tile::tile_of;

namespace {

constexpr int BM = 256;
constexpr int BN = 256;  // rows of the B tile
constexpr int BK = 64;
constexpr int NTHREADS = 512;

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

}  // namespace

template <int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ B,
    const bf16_t* __restrict__ B3, int64_t ldb, bf16_t* C, int64_t ldc,
    const bf16_t* __restrict__ gate, int64_t ld_gate, int M, int N, int K, int tiles_m,
    int tiles_n) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * BK];

  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;   // 2 waves along M
  const int wn = wave >> 1;  // 4 waves along N

  // ---- global load assignment: 4 chunks of A and 4 of B per thread ----
  const int lchunk = tid & 7;
  const int lrow = tid >> 3;  // 0..63, +64*i
  const bf16_t* a_src[4];
  const bf16_t* b_src[4];
  bool a_ok[4], b_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lrow + 64 * i;
    const int gm = m0 + r;
    a_ok[i] = gm < M;
    a_src[i] = A + (int64_t)(a_ok[i] ? gm : 0) * lda + lchunk * 8;
    int gn;
    const bf16_t* base;
    if constexpr (EPI == EPI_SWIGLU) {
      // B tile rows [w*64, w*64+32) = W1 features, [w*64+32, w*64+64) = W3 features
      const int w = r >> 6, within = r & 63;
      gn = tn * 128 + w * 32 + (within & 31);
      base = within < 32 ? B : B3;
    } else {
      gn = tn * BN + r;
      base = B;
    }
    b_ok[i] = gn < N;
    b_src[i] = base + (int64_t)(b_ok[i] ? gn : 0) * ldb + lchunk * 8;
  }

  uint4 ra[4], rb[4];
  auto load_tile = [&](int kt) {
    const int k0 = kt * BK + lchunk * 8;
    const bool kin = k0 < K;  // K % 8 == 0: a chunk is wholly in or out
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = (a_ok[i] && kin) ? *reinterpret_cast<const uint4*>(a_src[i] + kt * BK)
                               : make_uint4(0, 0, 0, 0);
      rb[i] = (b_ok[i] && kin) ? *reinterpret_cast<const uint4*>(b_src[i] + kt * BK)
                               : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lrow + 64 * i;
      *reinterpret_cast<uint4*>(&As[buf][lds_off(r, lchunk)]) = ra[i];
      *reinterpret_cast<uint4*>(&Bs[buf][lds_off(r, lchunk)]) = rb[i];
    }
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int nk = (K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int chunk = kk * 2 + frag_half;
      bf16x8_t af[4], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8_t*>(
            &As[buf][lds_off(wm * 128 + mi * 32 + frag_row, chunk)]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bfr[ni] = *reinterpret_cast<const bf16x8_t*>(
            &Bs[buf][lds_off(wn * 64 + ni * 32 + frag_row, chunk)]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column (lane & 31), rows (r/4)*8 + (lane/32)*4 + r%4 ----
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 128 + mi * 32 + (r >> 2) * 8 + frag_half * 4 + (r & 3);
      if (row >= M) continue;
      if constexpr (EPI == EPI_SWIGLU) {
        const int col = tn * 128 + wn * 32 + frag_row;
        if (col < N) {
          const float a = acc[mi][0][r], b = acc[mi][1][r];
          C[(int64_t)row * ldc + col] = f2bf(silu_f(a) * b);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = tn * BN + wn * 64 + ni * 32 + frag_row;
          if (col < N) {
            bf16_t* p = C + (int64_t)row * ldc + col;
            if constexpr (EPI == EPI_RESIDUAL) {
              const float g = bf2f(gate[(int64_t)row * ld_gate + col]);
              *p = f2bf(bf2f(*p) + g * acc[mi][ni][r]);
            } else {
              *p = f2bf(acc[mi][ni][r]);
            }
          }
        }
      }
    }
  }
}

// --------------------------------------- bf16 path, K % 64 == 0, one wave/SIMD
//
// 256 x 256 output tile (256 x 128 for SwiGLU), K step 64, 256 threads = 4
// waves as 2 (M) x 2 (N), each wave 128 x 128 from 4 x 4 MFMA tiles whose
// accumulators (256 floats per lane) live in the accumulation registers.  Per
// 16-wide k-slice a wave reads 8 fragments for 16 MFMAs, half the LDS traffic
// per MFMA of a 128 x 64 wave tile.
//  * Tiles go from global memory straight into LDS (global_load_lds_dwordx4:
//    no staging registers, no LDS stores).  One such instruction writes 1 KB,
//    i.e. 8 rows of 64 bf16; lane l writes 16-byte slot l % 8 of row l / 8 and
//    fetches the global chunk that the swizzle puts there.
//  * LDS rows are unpadded, 16-byte chunk c of row r at slot c ^ ((r / 2) % 8):
//    the 16 rows one 16-lane group of a fragment read touches then cover all
//    16 slot positions of a 256-byte bank line.
//  * Rows past M (or N) are clamped to the last row: every load is in bounds
//    and those accumulator rows are never stored.
//  * Two LDS stages (128 KB): tile k+1 is in flight while tile k is multiplied;
//    one barrier per K step.
namespace {
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
constexpr int W4_THREADS = 256;
constexpr int W4_STAGE = 32768;  // bytes of one 256 x 64 bf16 tile
constexpr int64_t W4_MAX_LD = (int64_t)1 << 22;  // 255 rows * 2^23 bytes < 2^31
}  // namespace

// One output tile of 64 MI rows (MI = 4: 256 rows, the usual tile; MI = 2:
// 128 rows, for the rows of a last partial round) starting at row m0, in
// tile column tn.  Each wave computes MI x 4 MFMA tiles; the k-order of every
// output element's MFMAs is the same for both heights.
template <int EPI, int MI>
__device__ __forceinline__ void w4_tile(
    char* smem, const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ B,
    const bf16_t* __restrict__ B3, int64_t ldb, bf16_t* C, int64_t ldc,
    const bf16_t* __restrict__ gate, int64_t ld_gate, int M, int N, int K, int m0, int tn,
    const GemmMap& map) {
  static_assert(MI == 4 || MI == 2, "tile of 256 or 128 rows");
  constexpr int RA = 16 * MI;  // A rows each wave loads into LDS
  constexpr int NAI = 2 * MI;  // ... in NAI instructions of 8 rows
  constexpr int NI = NAI + 8;  // load instructions per K tile (B: 8 per wave)
  constexpr int NF = 4 + MI;   // fragments per 16-wide k-slice
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int row_a = (int)(lda * 2), row_b = (int)(ldb * 2);

  // ---- DMA assignment: wave w fills LDS rows 64 w .. 64 w + 63 of each tile,
  // 8 rows per instruction j.  Byte offsets are relative to the tile's first row.
  const char* a_base = reinterpret_cast<const char*>(A + (int64_t)m0 * lda);
  const char* b_base;
  const char* b3_base = nullptr;
  int b_row0;  // first B row of the tile
  if constexpr (EPI == EPI_SWIGLU) {
    b_row0 = tn * 128;
    b3_base = reinterpret_cast<const char*>(B3 + (int64_t)b_row0 * ldb);
  } else {
    b_row0 = tn * BN;
  }
  b_base = reinterpret_cast<const char*>(B + (int64_t)b_row0 * ldb);
  int a_off[NAI], b_off[8];
#pragma unroll
  for (int j = 0; j < NAI; ++j) {
    const int r = wave * RA + j * 8 + (lane >> 3);  // LDS row of the A tile
    const int c = (lane & 7) ^ ((r >> 1) & 7);       // global chunk for this slot
    a_off[j] = (min(m0 + r, M - 1) - m0) * row_a + c * 16;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wave * 64 + j * 8 + (lane >> 3);  // LDS row of the B tile
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    int br;
    if constexpr (EPI == EPI_SWIGLU) {
      // tile rows 64 w .. 64 w + 31 are W1 rows, the next 32 the W3 rows of
      // the same 32 output features (j < 4: W1, j >= 4: W3)
      br = b_row0 + wave * 32 + ((j * 8 + (lane >> 3)) & 31);
    } else {
      br = b_row0 + r;
    }
    b_off[j] = (min(br, N - 1) - b_row0) * row_b + c * 16;
  }
  // DMA instruction t (0..15) of tile kt: t < 8 fills A rows, t >= 8 B rows.
  // Issued as inline assembly: the compiler would otherwise count these loads
  // as pending LDS operations and make every later fragment read wait for
  // them (lgkmcnt(0)).  Their completion is tracked by vmcnt alone; the K loop
  // waits for vmcnt(0) before the barrier that publishes the tile.  The
  // global address is an SGPR base (the tile's row block and K offset) plus
  // the lane's fixed 32-bit offset; the LDS address goes to M0.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)smem;
  auto dma16 = [&](const char* base, int voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds_addr) : "memory", "m0");
  };
  // byte offset of K tile kt in A (grouped-K layouts jump between column groups)
  auto a_koff = [&](int kt) -> int64_t {
    const int k0 = kt * BK;
    if (map.a_kgroup == 0) return (int64_t)k0 * 2;
    const int g = k0 / map.a_kgroup;
    return (g * map.a_gstride + (k0 - g * map.a_kgroup)) * 2;
  };
  auto issue_dma = [&](int kt, int stage, int t) {
    const int koff = kt * BK * 2;
    if (t < NAI) {
      dma16(a_base + a_koff(kt), a_off[t], lds0 + stage * W4_STAGE + wave * (RA * 128) + t * 1024);
    } else {
      const int j = t - NAI;
      const char* src = (EPI == EPI_SWIGLU && j >= 4) ? b3_base : b_base;
      dma16(src + koff, b_off[j], lds0 + (2 + stage) * W4_STAGE + wave * 8192 + j * 1024);
    }
  };

  // ---- fragment addresses: A row wm*128 + mi*32 + lane%32, chunk 2 kk + lane/32
  const int fr = lane & 31, fh = lane >> 5;
  const int swz = (fr >> 1) & 7;  // (row / 2) % 8 for every mi (rows step by 32)
  int fa[4], fb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int cs = ((kk * 2 + fh) ^ swz) * 16;
    fa[kk] = (wm * 32 * MI + fr) * 128 + cs;
    fb[kk] = 2 * W4_STAGE + (wn * 128 + fr) * 128 + cs;
  }

  f32x16_t acc[MI][4];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int nk = K / BK;
#pragma unroll
  for (int t = 0; t < NI; ++t) issue_dma(0, 0, t);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // one K step; MORE: tile kt+1 exists and is fetched during slice 0 (the
  // last step is a separate instantiation, so neither body branches)
  auto k_step = [&](int kt, auto more_tag) {
    constexpr bool MORE = decltype(more_tag)::value;
    const int so = (kt & 1) * W4_STAGE;
    bf16x8_t af[2][MI], bfr[2][4];
    // fragment j of slice kk: A0, B0..B3, A1..A3 (the order the MFMAs use them)
    auto read_frag = [&](int kk, int j) {
      const int c = kk & 1;
      if (j == 0) af[c][0] = *reinterpret_cast<const bf16x8_t*>(smem + fa[kk] + so);
      else if (j <= 4) bfr[c][j - 1] = *reinterpret_cast<const bf16x8_t*>(smem + fb[kk] + so + (j - 1) * 4096);
      else af[c][j - 4] = *reinterpret_cast<const bf16x8_t*>(smem + fa[kk] + so + (j - 4) * 4096);
    };
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      read_frag(0, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    // slice kk: 4 MI MFMAs (mi-major).  The NF fragments of slice kk+1 are
    // requested after the first NF of them (so they land before slice kk+1
    // starts); every second MFMA of the step is followed by one load of tile
    // kt+1 until its NI loads are issued (slices 0-1 at MI = 4, 0-2 at MI = 2).
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk & 1;
#pragma unroll
      for (int t = 0; t < 4 * MI; ++t) {
        const int mi = t >> 2, ni = t & 3;
        const int slot = kk * 4 * MI + t;
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[c][mi], bfr[c][ni], acc[mi][ni], 0, 0, 0);
        if (MORE && (slot & 1) && (slot >> 1) < NI) issue_dma(kt + 1, (kt + 1) & 1, slot >> 1);
        if (kk + 1 < 4 && t < NF) read_frag(kk + 1, t);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // tile kt+1 has landed (own DMAs) and is visible (barrier); stage kt&1 is free
    if (MORE) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  };
  for (int kt = 0; kt + 1 < nk; ++kt) k_step(kt, std::true_type{});
  k_step(nk - 1, std::false_type{});

  // ---- epilogue through LDS (shared with the FP8 kernel)
  gemm_tile::epilogue<EPI, MI>(smem, acc, C, ldc, gate, ld_gate, M, N, m0, tn, wm, wn, fr, fh, map);
}

// Work-groups [0, n_big) take 256-row tiles of rows [0, tiles_m * 256) in the
// XCD-aware order; the rest take 128-row tiles of rows [m_split, M) (the rows
// of what would be a last partial round of 256-row tiles, now packed into
// half-height tiles: launch_gemm chooses the split).
template <int EPI>
__global__ __launch_bounds__(W4_THREADS, 1) void gemm_bf16_w4_kernel(
    const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ B,
    const bf16_t* __restrict__ B3, int64_t ldb, bf16_t* C, int64_t ldc,
    const bf16_t* __restrict__ gate, int64_t ld_gate, int M, int N, int K, int tiles_m,
    int tiles_n, int n_big, int m_split, GemmMap map) {
  // [A stage 0 | A stage 1 | B stage 0 | B stage 1]; the epilogue reuses it
  // (256 x 264 bf16 or 128 x 264 fp32 = 135168 bytes)
  __shared__ __attribute__((aligned(1024))) char smem[135168];
  int tm, tn;
  if ((int)blockIdx.x < n_big) {
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    w4_tile<EPI, 4>(smem, A, lda, B, B3, ldb, C, ldc, gate, ld_gate, M, N, K, tm * BM, tn, map);
  } else {
    const int small_m = (M - m_split + 127) / 128;
    tile_of(blockIdx.x - n_big, small_m, tiles_n, tm, tn);
    w4_tile<EPI, 2>(smem, A, lda, B, B3, ldb, C, ldc, gate, ld_gate, M, N, K, m_split + tm * 128, tn,
                    map);
  }
}

// ---------------------------------------------------------------- fp32 path

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, int64_t lda, const float* __restrict__ B,
    const float* __restrict__ B3, int64_t ldb, float* C, int64_t ldc,
    const float* __restrict__ gate, int64_t ld_gate, int M, int N, int K) {
  constexpr int T = 64, TK = 16;
  __shared__ float as[TK][T + 1];
  __shared__ float bs[TK][T + 1];
  __shared__ float b3s[TK][T + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
  float acc[4][4] = {}, acc3[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += TK) {
    for (int i = threadIdx.x; i < T * TK; i += 256) {
      const int r = i / TK, c = i % TK;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + c;
      as[c][r] = (gm < M && gk < K) ? A[(int64_t)gm * lda + gk] : 0.f;
      bs[c][r] = (gn < N && gk < K) ? B[(int64_t)gn * ldb + gk] : 0.f;
      if constexpr (EPI == EPI_SWIGLU) b3s[c][r] = (gn < N && gk < K) ? B3[(int64_t)gn * ldb + gk] : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < TK; ++c) {
      float av[4], bv[4], b3v[4];
      for (int i = 0; i < 4; ++i) {
        av[i] = as[c][ty * 4 + i];
        bv[i] = bs[c][tx * 4 + i];
        if constexpr (EPI == EPI_SWIGLU) b3v[i] = b3s[c][tx * 4 + i];
      }
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) {
          acc[i][j] += av[i] * bv[j];
          if constexpr (EPI == EPI_SWIGLU) acc3[i][j] += av[i] * b3v[j];
        }
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + ty * 4 + i, col = n0 + tx * 4 + j;
      if (row >= M || col >= N) continue;
      float* p = C + (int64_t)row * ldc + col;
      if constexpr (EPI == EPI_SWIGLU) {
        *p = silu_f(acc[i][j]) * acc3[i][j];
      } else if constexpr (EPI == EPI_RESIDUAL) {
        *p = *p + gate[(int64_t)row * ld_gate + col] * acc[i][j];
      } else {
        *p = acc[i][j];
      }
    }
}

hipError_t launch_gemm(bool bf16, int epi, const void* A, int64_t lda, const void* B,
                       const void* B3, int64_t ldb, void* C, int64_t ldc, const void* gate,
                       int64_t ld_gate, int64_t M, int N, int K, hipStream_t s,
                       const GemmMap& map) {
  if (M == 0 || N == 0) return hipSuccess;
  // operand maps exist only on the bf16 K % 64 kernel (and a scatter only for plain stores)
  if (!map.empty() && (!bf16 || K < BK || K % BK != 0 || (map.a_kgroup % BK) != 0 ||
                       (map.peer_hc && epi != EPI_STORE) ||
                       (map.mx_q && (epi != EPI_SWIGLU || N % 32 != 0)) || (map.mx_only && !map.mx_q) ||
                       (map.qk_pos && (epi != EPI_STORE || (map.qk_D != 64 && map.qk_D != 128) ||
                                       N != 3 * map.qk_H * map.qk_D))))
    return hipErrorInvalidValue;
  if (bf16) {
    const int tiles_m = (int)ceil_div(M, BM);
    const int tiles_n = (int)ceil_div(N, epi == EPI_SWIGLU ? 128 : BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    // the K % 64 kernel keeps a lane's load offsets (up to 255 rows of A or B)
    // in 32 bits: row strides up to 2^22 elements; beyond that the general
    // kernel (64-bit addressing) runs, which has no operand maps
    const bool narrow = lda <= W4_MAX_LD && ldb <= W4_MAX_LD;
    if (!map.empty() && !narrow) return hipErrorInvalidValue;
    // 256-row tiles, and 128-row tiles for the rows of a last partial round
    // (appended to the same grid, so they fill the units the last 256-row
    // tiles leave idle)
    const gemm_tile::RowSplit sp = gemm_tile::split_rows(M, tiles_m, tiles_n);
    const dim3 grid_w4((unsigned)((sp.big + sp.small_m) * tiles_n));
    const int n_big = sp.big * tiles_n, m_split = sp.big * BM;
#define H3_G(E)                                                                                 \
  if (K >= BK && K % BK == 0 && narrow)                                                         \
    hipLaunchKernelGGL((gemm_bf16_w4_kernel<E>), grid_w4, dim3(W4_THREADS), 0, s,               \
                       (const bf16_t*)A, lda, (const bf16_t*)B, (const bf16_t*)B3, ldb,         \
                       (bf16_t*)C, ldc, (const bf16_t*)gate, ld_gate, (int)M, N, K, sp.big,     \
                       tiles_n, n_big, m_split, map);                                            \
  else                                                                                           \
    hipLaunchKernelGGL((gemm_bf16_kernel<E>), grid, dim3(NTHREADS), 0, s, (const bf16_t*)A, lda, \
                       (const bf16_t*)B, (const bf16_t*)B3, ldb, (bf16_t*)C, ldc,                \
                       (const bf16_t*)gate, ld_gate, (int)M, N, K, tiles_m, tiles_n)
    if (epi == EPI_SWIGLU) H3_G(EPI_SWIGLU);
    else if (epi == EPI_RESIDUAL) H3_G(EPI_RESIDUAL);
    else H3_G(EPI_STORE);
#undef H3_G
  } else {
    const dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ceil_div(M, 64));
#define H3_G(E)                                                                         \
  hipLaunchKernelGGL((gemm_f32_kernel<E>), grid, dim3(256), 0, s, (const float*)A, lda, \
                     (const float*)B, (const float*)B3, ldb, (float*)C, ldc,            \
                     (const float*)gate, ld_gate, (int)M, N, K)
    if (epi == EPI_SWIGLU) H3_G(EPI_SWIGLU);
    else if (epi == EPI_RESIDUAL) H3_G(EPI_RESIDUAL);
    else H3_G(EPI_STORE);
#undef H3_G
  }
  return hipGetLastError();
}

}  // namespace h3
