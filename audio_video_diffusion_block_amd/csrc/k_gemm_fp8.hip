// FP8 (MX-scaled e4m3) GEMMs of the block: out = A @ B^T with A [M, K]
// activations and B [N, K] weights, both stored as MX operands, fp32
// accumulation, bf16 output, and the bf16 kernel's three epilogues (store,
// SwiGLU, gated residual).
//
// MiniMax H3 通过 vLLM-Omni 实现 FastH3 实时推理, "超出 FastH3 配置的扩展能力"
// (quantization path): online FP8 cuts the peak HBM footprint and the
// latency of the pipeline.  The pages give no format; here both operands use
// the MX block format of h3_fp8.hpp along K, the one gfx950's scaled MFMA
// reads natively, so no dequantization appears in the kernel.
//
// MX operand layout (plain, row-major): e4m3 data [rows][ld] bytes holding
// Kp = round_up(K, 128) columns, zeros past K; E8M0 scales [rows][ld_s] bytes,
// byte b of a row is the scale of columns [32 b, 32 b + 32).
//
// Kernel: the bf16 K % 64 kernel's structure (k_gemm.hip) with e4m3 bytes --
// 256 x 256 output tile, 4 waves as 2 x 2 of 128 x 128, AGPR accumulators,
// K step 128 bytes (= 128 elements) loaded global -> LDS directly into
// XOR-swizzled 128-byte rows, two LDS stages, one barrier per K step.
//  * Per K step a wave runs two 64-deep steps of 16
//    v_mfma_scale_f32_32x32x64_f8f6f4, each twice the flops of a bf16 K step
//    slice for the same issue time per flop at the fp8 rate.
//  * A fragment (32 bytes per lane) is two 16-byte LDS reads: for step s and
//    lane half h, chunks 4 s + h (bytes 0-15) and 4 s + 2 + h (bytes 16-31).
//  * Scales: the 4-byte word of a row at K step kt holds blocks 4 kt .. 4 kt
//    + 3; lane half h shifts it right by 8 h, so byte 0 is its block of step 0
//    and byte 2 its block of step 1 (the MFMA's byte selects).  The words of
//    step kt + 1 are loaded into registers during step kt.
#include "h3_common.hpp"
#include "h3_fp8.hpp"
#include "h3_gemm_tile.hpp"
#include "h3_kernels.hpp"

namespace h3 {

using namespace fp8;

// ------------------------------------------------------------ quantization

// bf16 rows [rows][cols] (cols % 32 == 0) -> MX operand with kp columns
// (zeros and scale byte 127 past cols).  One thread per 32-element block.
// kgroup > 0: the source is grouped along the columns -- columns
// [g*kgroup, (g+1)*kgroup) of row r sit at x + g*gstride + r*ld_x.
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(const bf16_t* __restrict__ x,
                                                            int64_t ld_x, int64_t rows, int cols,
                                                            int kp, int kgroup, int64_t gstride,
                                                            uint8_t* __restrict__ q,
                                                            int64_t ld_q,
                                                            uint8_t* __restrict__ sc,
                                                            int64_t ld_s) {
  const int nb = kp / 32;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * nb) return;
  const int64_t r = t / nb;
  const int b = (int)(t - r * nb);
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint32_t e = 127;
  if (b * 32 < cols) {
    int64_t c0 = b * 32;
    if (kgroup > 0) {
      const int g = b * 32 / kgroup;
      c0 = g * gstride + (b * 32 - g * kgroup);
    }
    const uint4* src = reinterpret_cast<const uint4*>(x + r * ld_x + c0);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = src[i];
      const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(uw[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(uw[j] & 0xFFFF0000u);
      }
    }
    e = quant32(v, w);
  }
  uint4* dst = reinterpret_cast<uint4*>(q + r * ld_q + b * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  sc[r * ld_s + b] = (uint8_t)e;
}

// ------------------------------------------------------------------ GEMM

namespace {
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int F8_BM = 256;
constexpr int F8_BN = 256;
constexpr int F8_BK = 128;       // bytes = elements per K step
constexpr int F8_THREADS = 256;
constexpr int F8_STAGE = 32768;  // bytes of one 256 x 128 e4m3 tile
}  // namespace

// One output tile of 64 MI rows (MI = 4: 256; MI = 2: 128, for the rows of a
// last partial round) starting at row m0, in tile column tn.
template <int EPI, int MI>
__device__ __forceinline__ void f8_tile(
    char* smem, const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ As,
    int64_t ld_as, const uint8_t* __restrict__ B, const uint8_t* __restrict__ B3, int64_t ldb,
    const uint8_t* __restrict__ Bs, const uint8_t* __restrict__ B3s, int64_t ld_bs, bf16_t* C,
    int64_t ldc, const bf16_t* __restrict__ gate, int64_t ld_gate, int M, int N, int K, int m0,
    int tn, const GemmMap& map) {
  static_assert(MI == 4 || MI == 2, "tile of 256 or 128 rows");
  constexpr int RA = 16 * MI;   // A rows each wave loads into LDS
  constexpr int NAI = 2 * MI;   // ... in NAI instructions of 8 rows
  constexpr int NI = NAI + 8;   // load instructions per K tile (B: 8 per wave)
  constexpr int NR = 2 * (4 + MI);  // 16-byte fragment reads per 64-deep step
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int row_a = (int)lda, row_b = (int)ldb;

  // ---- DMA assignment (as the bf16 kernel): wave w fills LDS rows 64 w ..
  // 64 w + 63 of each tile, 8 rows per instruction j
  const char* a_base = reinterpret_cast<const char*>(A + (int64_t)m0 * lda);
  const char* b3_base = nullptr;
  int b_row0;
  if constexpr (EPI == EPI_SWIGLU) {
    b_row0 = tn * 128;
    b3_base = reinterpret_cast<const char*>(B3 + (int64_t)b_row0 * ldb);
  } else {
    b_row0 = tn * F8_BN;
  }
  const char* b_base = reinterpret_cast<const char*>(B + (int64_t)b_row0 * ldb);
  int a_off[NAI], b_off[8];
#pragma unroll
  for (int j = 0; j < NAI; ++j) {
    const int r = wave * RA + j * 8 + (lane >> 3);  // LDS row of the A tile
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    a_off[j] = (min(m0 + r, M - 1) - m0) * row_a + c * 16;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wave * 64 + j * 8 + (lane >> 3);  // LDS row of the B tile
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    int br;
    if constexpr (EPI == EPI_SWIGLU) {
      br = b_row0 + wave * 32 + ((j * 8 + (lane >> 3)) & 31);
    } else {
      br = b_row0 + r;
    }
    b_off[j] = (min(br, N - 1) - b_row0) * row_b + c * 16;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)smem;
  // global -> LDS, 16 bytes per lane; tracked by vmcnt only (see k_gemm.hip)
  auto dma16 = [&](const char* base, int voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds_addr) : "memory", "m0");
  };
  auto issue_dma = [&](int kt, int stage, int t) {
    const int koff = kt * F8_BK;
    if (t < NAI) {
      dma16(a_base + koff, a_off[t], lds0 + stage * F8_STAGE + wave * (RA * 128) + t * 1024);
    } else {
      const int j = t - NAI;
      const char* src = (EPI == EPI_SWIGLU && j >= 4) ? b3_base : b_base;
      dma16(src + koff, b_off[j], lds0 + (2 + stage) * F8_STAGE + wave * 8192 + j * 1024);
    }
  };

  // ---- fragment addresses: row wm*128 + mi*32 + lane%32; step s, half p
  // (bytes 16 p .. 16 p + 15 of the lane's 32) reads chunk 4 s + 2 p + lane/32
  const int fr = lane & 31, fh = lane >> 5;
  const int swz = (fr >> 1) & 7;
  int fa[2][2], fb[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int cs = ((4 * s + 2 * p + fh) ^ swz) * 16;
      fa[s][p] = (wm * 32 * MI + fr) * 128 + cs;
      fb[s][p] = 2 * F8_STAGE + (wn * 128 + fr) * 128 + cs;
    }

  // ---- scale rows of this lane (clamped like the data rows)
  const uint8_t* sa_row[MI];
  const uint8_t* sb_row[4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
    sa_row[i] = As + (int64_t)min(m0 + wm * 32 * MI + i * 32 + fr, M - 1) * ld_as;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (EPI == EPI_SWIGLU) {
      // B tile rows 64 w' .. +31 are W1 features b_row0 + 32 w' + (0..31), the
      // next 32 the W3 rows of the same features; wave column wn reads tile
      // rows wn*128 + ni*32 + fr, i.e. w' = 2 wn + ni/2, W3 when ni is odd
      const int feat = min(b_row0 + 32 * (2 * wn + (i >> 1)) + fr, N - 1);
      sb_row[i] = ((i & 1) ? B3s : Bs) + (int64_t)feat * ld_bs;
    } else {
      sb_row[i] = Bs + (int64_t)min(b_row0 + wn * 128 + i * 32 + fr, N - 1) * ld_bs;
    }
  }
  uint32_t sa_cur[MI], sb_cur[4];
  auto load_scales = [&](int kt, uint32_t (&sa)[MI], uint32_t (&sb)[4]) {
#pragma unroll
    for (int i = 0; i < MI; ++i) sa[i] = *reinterpret_cast<const uint32_t*>(sa_row[i] + kt * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) sb[i] = *reinterpret_cast<const uint32_t*>(sb_row[i] + kt * 4);
  };

  f32x16_t acc[MI][4];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int nk = K / F8_BK;
  load_scales(0, sa_cur, sb_cur);
#pragma unroll
  for (int t = 0; t < NI; ++t) issue_dma(0, 0, t);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  auto k_step = [&](int kt, auto more_tag) {
    constexpr bool MORE = decltype(more_tag)::value;
    const int so = (kt & 1) * F8_STAGE;
    uint32_t sa[MI], sb[4], sa_nxt[MI], sb_nxt[4];
#pragma unroll
    for (int i = 0; i < MI; ++i) sa[i] = sa_cur[i] >> (8 * fh);
#pragma unroll
    for (int i = 0; i < 4; ++i) sb[i] = sb_cur[i] >> (8 * fh);
    if (MORE) load_scales(kt + 1, sa_nxt, sb_nxt);
    i32x8_t af[2][MI], bf[2][4];
    // read j of step s: 0-1 A0, 2-9 B0..B3, 10-15 A1..A3 (two halves each)
    auto read = [&](int s, int j) {
      const int f = j >> 1, p = j & 1;
      const uint4* src;
      if (f == 0) src = reinterpret_cast<const uint4*>(smem + fa[s][p] + so);
      else if (f <= 4) src = reinterpret_cast<const uint4*>(smem + fb[s][p] + so + (f - 1) * 4096);
      else src = reinterpret_cast<const uint4*>(smem + fa[s][p] + so + (f - 4) * 4096);
      const uint4 u = *src;
      i32x8_t& dst = f == 0 ? af[s][0] : (f <= 4 ? bf[s][f - 1] : af[s][f - 4]);
      dst[4 * p + 0] = (int)u.x;
      dst[4 * p + 1] = (int)u.y;
      dst[4 * p + 2] = (int)u.z;
      dst[4 * p + 3] = (int)u.w;
    };
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      read(0, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    // 4 MI MFMAs per 64-deep step; during step 0 the NR reads of step 1 follow
    // its MFMAs (one or two each), and the NI loads of tile kt+1 one per MFMA
    // slot of the K tile until all are issued
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int t = 0; t < 4 * MI; ++t) {
        const int mi = t >> 2, ni = t & 3;
        const int slot = s * 4 * MI + t;
        if (s == 0)
          acc[mi][ni] = mfma_e4m3<0>(af[0][mi], bf[0][ni], acc[mi][ni], sa[mi], sb[ni]);
        else
          acc[mi][ni] = mfma_e4m3<2>(af[1][mi], bf[1][ni], acc[mi][ni], sa[mi], sb[ni]);
        if (MORE && slot < NI) issue_dma(kt + 1, (kt + 1) & 1, slot);
        if (s == 0) {
          read(1, t);
          if (t + 4 * MI < NR) read(1, t + 4 * MI);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (MORE) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MI; ++i) sa_cur[i] = sa_nxt[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) sb_cur[i] = sb_nxt[i];
    }
  };
  for (int kt = 0; kt + 1 < nk; ++kt) k_step(kt, std::true_type{});
  k_step(nk - 1, std::false_type{});
  // the epilogue reads every accumulator: let the last scaled MFMAs finish
  scaled_mfma_drain();

  gemm_tile::epilogue<EPI, MI>(smem, acc, C, ldc, gate, ld_gate, M, N, m0, tn, wm, wn, fr, fh, map);
}

// Work-groups [0, n_big) take 256-row tiles of rows [0, tiles_m * 256) in the
// XCD-aware order, the rest 128-row tiles of rows [m_split, M) (the split is
// chosen by launch_gemm_mx8).
template <int EPI>
__global__ __launch_bounds__(F8_THREADS, 1) void gemm_mx8_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ As, int64_t ld_as,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ B3, int64_t ldb,
    const uint8_t* __restrict__ Bs, const uint8_t* __restrict__ B3s, int64_t ld_bs, bf16_t* C,
    int64_t ldc, const bf16_t* __restrict__ gate, int64_t ld_gate, int M, int N, int K,
    int tiles_m, int tiles_n, int n_big, int m_split, GemmMap map) {
  // [A stage 0 | A stage 1 | B stage 0 | B stage 1]; the epilogue reuses it
  __shared__ __attribute__((aligned(1024))) char smem[135168];
  int tm, tn;
  if ((int)blockIdx.x < n_big) {
    gemm_tile::tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    f8_tile<EPI, 4>(smem, A, lda, As, ld_as, B, B3, ldb, Bs, B3s, ld_bs, C, ldc, gate, ld_gate, M, N,
                    K, tm * F8_BM, tn, map);
  } else {
    gemm_tile::tile_of(blockIdx.x - n_big, (M - m_split + 127) / 128, tiles_n, tm, tn);
    f8_tile<EPI, 2>(smem, A, lda, As, ld_as, B, B3, ldb, Bs, B3s, ld_bs, C, ldc, gate, ld_gate, M, N,
                    K, m_split + tm * 128, tn, map);
  }
}

// ------------------------------------------------------------------ launch

hipError_t launch_mx_quantize(const void* x, int64_t ld_x, int64_t rows, int cols, void* q,
                              int64_t ld_q, void* scale, int64_t ld_s, hipStream_t s, int kgroup,
                              int64_t gstride) {
  if (rows == 0) return hipSuccess;
  if (kgroup < 0 || kgroup % 32 != 0) return hipErrorInvalidValue;
  const int kp = (int)round_up((int64_t)cols, 128);
  const int64_t threads = rows * (kp / 32);
  hipLaunchKernelGGL(mx_quant_rows_kernel, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0,
                     s, (const bf16_t*)x, ld_x, rows, cols, kp, kgroup, gstride, (uint8_t*)q,
                     ld_q, (uint8_t*)scale, ld_s);
  return hipGetLastError();
}

hipError_t launch_gemm_mx8(int epi, const MxOperand& a, const MxOperand& b, const MxOperand& b3,
                           void* C, int64_t ldc, const void* gate, int64_t ld_gate, int64_t M,
                           int N, int K, hipStream_t s, const GemmMap& map) {
  if (M == 0 || N == 0) return hipSuccess;
  // only the store epilogue's peer-major scatter applies here (A is an MX operand)
  if (map.a_kgroup != 0 || (map.peer_hc && epi != EPI_STORE) ||
      (map.mx_q && (epi != EPI_SWIGLU || N % 32 != 0)) || (map.mx_only && !map.mx_q) ||
      (map.qk_pos && (epi != EPI_STORE || (map.qk_D != 64 && map.qk_D != 128) ||
                      N != 3 * map.qk_H * map.qk_D)))
    return hipErrorInvalidValue;
  const int kp = (int)round_up((int64_t)K, 128);
  const int tiles_m = (int)ceil_div(M, F8_BM);
  const int tiles_n = (int)ceil_div(N, epi == EPI_SWIGLU ? 128 : F8_BN);
  // 256-row tiles, and 128-row tiles for the rows of a last partial round
  // (appended to the same grid; the split model of the bf16 kernel)
  const gemm_tile::RowSplit sp = gemm_tile::split_rows(M, tiles_m, tiles_n);
  const dim3 grid((unsigned)((sp.big + sp.small_m) * tiles_n));
  const int n_big = sp.big * tiles_n, m_split = sp.big * F8_BM;
#define H3_G(E)                                                                              \
  hipLaunchKernelGGL((gemm_mx8_kernel<E>), grid, dim3(F8_THREADS), 0, s,                       \
                     (const uint8_t*)a.data, a.ld, (const uint8_t*)a.scale, a.ld_scale,        \
                     (const uint8_t*)b.data, (const uint8_t*)b3.data, b.ld,                    \
                     (const uint8_t*)b.scale, (const uint8_t*)b3.scale, b.ld_scale, (bf16_t*)C, \
                     ldc, (const bf16_t*)gate, ld_gate, (int)M, N, kp, sp.big, tiles_n, n_big,  \
                     m_split, map)
  if (epi == EPI_SWIGLU) H3_G(EPI_SWIGLU);
  else if (epi == EPI_RESIDUAL) H3_G(EPI_RESIDUAL);
  else H3_G(EPI_STORE);
#undef H3_G
  return hipGetLastError();
}

}  // namespace h3
