// Shared pieces of the 256 x 256-tile GEMM kernels (bf16 and FP8): the
// XCD-aware tile order and the LDS-staged epilogue.
#pragma once

#include "h3_common.hpp"
#include "h3_fp8.hpp"
#include "h3_kernels.hpp"

namespace h3 {
namespace gemm_tile {

constexpr int GROUP_M = 4;

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

// Host side: split of a tiled GEMM's rows into `big` rows of 256-row tiles
// followed by 128-row tiles for the rest.  The makespan of in-order dispatch
// onto 256 units (one tile at a time each) is estimated in units of one
// 256-row tile, a 128-row tile costing 0.8 of one (it has the same B tile and
// most of the per-step work; measured: a split predicted from half the cost
// made the QKV projection 1% slower), for splits near the last full round; a
// split is taken when it saves at least 1.5%.
struct RowSplit { int big, small_m; };
inline RowSplit split_rows(int64_t M, int tiles_m, int tiles_n) {
  constexpr int CUS = 256;
  constexpr double CS = 0.8;
  auto cdiv = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
  auto makespan = [&](int b, int small_m) {
    const int64_t nb = (int64_t)b * tiles_n, ns = (int64_t)small_m * tiles_n;
    const int64_t full = nb / CUS, rem = nb % CUS;
    if (rem == 0) return (double)full + CS * (double)cdiv(ns, CUS);
    // the last 256-row tiles run beside 128-row ones on the other units
    const int64_t beside = (int64_t)((CUS - rem) / CS);
    const int64_t left = ns > beside ? ns - beside : 0;
    return (double)full + 1.0 + CS * (double)cdiv(left, CUS);
  };
  const double t0 = (double)cdiv((int64_t)tiles_m * tiles_n, CUS);
  RowSplit best{tiles_m, 0};
  double best_t = t0;
  for (int b = tiles_m - 1; b >= 0 && b >= tiles_m - 16; --b) {
    const int small_m = (int)cdiv(M - (int64_t)b * 256, 128);
    const double t = makespan(b, small_m);
    if (t < best_t - 1e-9) {
      best_t = t;
      best = {b, small_m};
    }
  }
  if (best_t > 0.985 * t0) return {tiles_m, 0};
  return best;
}

// XCD-aware mapping of a linear work-group id to (tile_m, tile_n).
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int total8 = total / 8 * 8;
  // consecutive ids go to different XCDs; give each XCD a contiguous run of tiles
  const int logical = bid < total8 ? (bid % 8) * (total8 / 8) + bid / 8 : bid;
  const int per_group = GROUP_M * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Epilogue of a 64 MI-row output tile (MI = 4: 256 rows; MI = 2: 128) held by
// 4 waves as 2 (M) x 2 (N), each 32 MI x 128 in MI x 4 32x32 accumulator
// blocks (acc[mi][ni], 256 threads).  smem must hold 135168 bytes and be free
// (the caller's K loop is done).
template <int EPI, int MI = 4>
__device__ __forceinline__ void epilogue(char* smem, f32x16_t (&acc)[MI][4], bf16_t* C,
                                         int64_t ldc, const bf16_t* gate, int64_t ld_gate, int M,
                                         int N, int m0, int tn, int wm, int wn, int fr, int fh,
                                         const GemmMap& map) {
  constexpr int W4_THREADS = 256;
  constexpr int BN = 256;
  constexpr int RW = 32 * MI;  // rows per wave row
  constexpr int TR = 2 * RW;   // rows of the tile
  // Through LDS.  A lane holds column lane%32 and rows
  // (r/4)*8 + (lane/32)*4 + r%4 of each 32x32 block; the tile is written to LDS
  // in that layout and read back as row-contiguous 16-byte chunks, so every
  // global access is a 16-byte vector.  Padded LDS rows keep the lane-per-
  // column writes of the two lane halves (rows 4 apart) on disjoint banks.
  __syncthreads();  // every wave is done with the last tile's fragments
  const int tid = threadIdx.x;
  if constexpr (EPI == EPI_RESIDUAL) {
    // out = out + gate * acc with acc in fp32: passes of 128 rows (two for a
    // 256-row tile, each written by one wave row; one for a 128-row tile)
    constexpr int FS = 264;  // floats per LDS row
    float* ef = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int half = 0; half < TR / 128; ++half) {
      if ((wm * RW) / 128 == half) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              ef[(wm * RW - half * 128 + mi * 32 + (r >> 2) * 8 + fh * 4 + (r & 3)) * FS + wn * 128 +
                 ni * 32 + fr] = acc[mi][ni][r];
      }
      __syncthreads();
      if (m0 + half * 128 + 128 <= M && tn * BN + BN <= N && ldc <= (int64_t)1 << 22 &&
          ld_gate <= (int64_t)1 << 22) {
        // every chunk of this pass is inside the output: straight-line code
        // whose loads of x and gate for G chunks are all in flight before the
        // first is used.  Buffer accesses: a 32-bit lane offset plus a scalar
        // offset per chunk (chunk i of a thread is 8 i rows below its first),
        // so the addresses take no registers.
        constexpr int G = 4;
        const int64_t row0 = m0 + half * 128;
        const auto rc = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<char*>(C + row0 * ldc + tn * BN), 0, 0x7FFFFFF0, 0x00020000);
        const auto rg = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(reinterpret_cast<const char*>(gate + row0 * ld_gate + tn * BN)), 0,
            0x7FFFFFF0, 0x00020000);
        const int voc = (tid >> 5) * (int)(ldc * 2) + (tid & 31) * 16;
        const int vog = (tid >> 5) * (int)(ld_gate * 2) + (tid & 31) * 16;
        const int stc = 8 * (int)(ldc * 2), stg = 8 * (int)(ld_gate * 2);
#pragma unroll
        for (int i0 = 0; i0 < 16; i0 += G) {
          uint4 xv[G], gv[G];
#pragma unroll
          for (int u = 0; u < G; ++u) {
            xv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, voc, (i0 + u) * stc, 0));
            gv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rg, vog, (i0 + u) * stg, 0));
          }
#pragma unroll
          for (int u = 0; u < G; ++u) {
            const int chunk = tid + (i0 + u) * W4_THREADS;
            const float* src = ef + (chunk >> 5) * FS + (chunk & 31) * 8;
            const float4 y0 = *reinterpret_cast<const float4*>(src);
            const float4 y1 = *reinterpret_cast<const float4*>(src + 4);
            const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
            bf16_t* xe = reinterpret_cast<bf16_t*>(&xv[u]);
            const bf16_t* ge = reinterpret_cast<const bf16_t*>(&gv[u]);
#pragma unroll
            for (int e = 0; e < 8; ++e) xe[e] = f2bf(bf2f(xe[e]) + bf2f(ge[e]) * yv[e]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, xv[u]),
                                                   rc, voc, (i0 + u) * stc, 0);
          }
        }
        __syncthreads();
        continue;
      }
#pragma unroll 4
      for (int i = 0; i < 16; ++i) {
        const int chunk = tid + i * W4_THREADS;  // 128 rows x 32 chunks of 8
        const int rl = chunk >> 5, c8 = (chunk & 31) * 8;
        const int row = m0 + half * 128 + rl, col = tn * BN + c8;
        if (row >= M || col >= N) continue;
        const float* src = ef + rl * FS + c8;
        bf16_t* po = C + (int64_t)row * ldc + col;
        const bf16_t* pg = gate + (int64_t)row * ld_gate + col;
        if (col + 8 <= N) {
          const float4 y0 = *reinterpret_cast<const float4*>(src);
          const float4 y1 = *reinterpret_cast<const float4*>(src + 4);
          const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
          uint4 xo = *reinterpret_cast<const uint4*>(po);
          const uint4 gv = *reinterpret_cast<const uint4*>(pg);
          bf16_t* xe = reinterpret_cast<bf16_t*>(&xo);
          const bf16_t* ge = reinterpret_cast<const bf16_t*>(&gv);
#pragma unroll
          for (int e = 0; e < 8; ++e) xe[e] = f2bf(bf2f(xe[e]) + bf2f(ge[e]) * yv[e]);
          *reinterpret_cast<uint4*>(po) = xo;
        } else {
          for (int e = 0; col + e < N; ++e) po[e] = f2bf(bf2f(po[e]) + bf2f(pg[e]) * src[e]);
        }
      }
      __syncthreads();
    }
  } else {
    // bf16 tile: 256 rows x OC columns (256, or 128 SwiGLU outputs)
    constexpr int OC = EPI == EPI_SWIGLU ? 128 : 256;
    constexpr int ES = OC + 8;  // bf16 per LDS row
    bf16_t* eb = reinterpret_cast<bf16_t*>(smem);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = wm * RW + mi * 32 + (r >> 2) * 8 + fh * 4 + (r & 3);
        if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            eb[rl * ES + (wn * 2 + j) * 32 + fr] = f2bf(silu_f(acc[mi][2 * j][r]) * acc[mi][2 * j + 1][r]);
        } else {
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) eb[rl * ES + wn * 128 + ni * 32 + fr] = f2bf(acc[mi][ni][r]);
        }
      }
    __syncthreads();
    constexpr int CPR = OC / 8;  // 16-byte chunks per row
    // Q/K RMSNorm + RoPE (EPI_STORE of a QKV projection): a thread always
    // handles the same 8 columns (chunk tid % CPR of its rows), so its gains
    // and rotation pairs are fixed; the D/8 chunks of a head row sit in
    // adjacent lanes of one row of 16 lanes, whose DPP sum gives the norm
    const int qk_hd = map.qk_H * map.qk_D;
    float qk_gq[8], qk_gk[8];
    RopeLane qk_rl;
    if (EPI == EPI_STORE && map.qk_pos) {
      const int cd = ((tid % CPR) * 8) % map.qk_D;  // first dim of the thread's 8 columns in its head
      Vec8<bf16_t>::load(map.qk_gq + cd, qk_gq);
      Vec8<bf16_t>::load(map.qk_gk + cd, qk_gk);
      qk_rl = rope_lane(map.qk_tab, cd / 8);
    }
    if (EPI == EPI_STORE && map.qk_pos && !map.peer_hc && m0 + TR <= M && tn * BN + BN <= N &&
        tn * BN + BN <= 2 * qk_hd && ldc <= ((int64_t)1 << 22)) {
      // A tile of q and k head columns wholly inside the output: straight-line
      // code that requests the positions of G chunks' rows (one 16-byte entry
      // per row) together instead of waiting on each; buffer accesses, a lane
      // offset plus a scalar offset per chunk (chunk i of a thread is 8 i rows
      // below its first).  Same arithmetic as the general path below.
      constexpr int G = 4;
      const auto rp = __builtin_amdgcn_make_buffer_rsrc(const_cast<int4*>(map.qk_pos + m0), 0,
                                                        0x7FFFFFF0, 0x00020000);
      const auto rc = __builtin_amdgcn_make_buffer_rsrc(C + (int64_t)m0 * ldc + tn * BN, 0,
                                                        0x7FFFFFF0, 0x00020000);
      const int r0 = tid / CPR, c8 = (tid % CPR) * 8;
      const int vop = r0 * 16, voc = r0 * (int)(ldc * 2) + c8 * 2;
      const int stc = (W4_THREADS / CPR) * (int)(ldc * 2);
      const float* gain = tn * BN + c8 < qk_hd ? qk_gq : qk_gk;
#pragma unroll
      for (int i0 = 0; i0 < TR * CPR / W4_THREADS; i0 += G) {
        int4 ps[G];
#pragma unroll
        for (int u = 0; u < G; ++u)
          ps[u] = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rp, vop, (i0 + u) * (W4_THREADS / CPR) * 16, 0));
#pragma unroll
        for (int u = 0; u < G; ++u) {
          const uint4 raw = *reinterpret_cast<const uint4*>(eb + (r0 + (i0 + u) * (W4_THREADS / CPR)) * ES + c8);
          uint4 out = raw;
          if (ps[u].x == 0 || ps[u].x == 1) {
            float v[8], cs[4], sn[4];
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[2 * e] = __uint_as_float(w[e] << 16);
              v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
            rope_cos_sin(qk_rl, ps[u], cs, sn);
            if (map.qk_D == 128) qk_norm_rope_lane<16>(v, gain, cs, sn, map.qk_eps);
            else qk_norm_rope_lane<8>(v, gain, cs, sn, map.qk_eps);
            out.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
            out.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
            out.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
            out.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
          }
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, out), rc, voc,
              (i0 + u) * stc, 0);
        }
      }
      return;
    }
#pragma unroll 4
    for (int i = 0; i < TR * CPR / W4_THREADS; ++i) {
      const int chunk = tid + i * W4_THREADS;
      const int rl = chunk / CPR, c8 = (chunk % CPR) * 8;
      const int row = m0 + rl, col = (EPI == EPI_SWIGLU ? tn * 128 : tn * BN) + c8;
      if (row >= M || col >= N) continue;
      const bf16_t* src = eb + rl * ES + c8;
      bf16_t* po = C + (int64_t)row * ldc + col;
      if (EPI == EPI_STORE && map.peer_hc) {
        // peer-major scatter of an 8-column chunk (it never straddles a head)
        const int hd = map.peer_H * map.peer_D, which = col / hd;
        const int h = (col - which * hd) / map.peer_D, d = col - which * hd - h * map.peer_D;
        const int p = h / map.peer_hc, j = h - p * map.peer_hc;
        po = C + (((int64_t)p * M + row) * 3 + which) * map.peer_hc * map.peer_D + j * map.peer_D + d;
      }
      if (EPI == EPI_STORE && map.qk_pos && col < 2 * qk_hd) {
        // a q or k head column: the row's position decides (uniform over the head's lanes)
        const int4 ps = map.qk_pos[row];
        if (ps.x == 0 || ps.x == 1) {
          float v[8], cs[4], sn[4];
          const uint4 raw = *reinterpret_cast<const uint4*>(src);
          const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(u[e] << 16);
            v[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
          }
          rope_cos_sin(qk_rl, ps, cs, sn);
          if (map.qk_D == 128) qk_norm_rope_lane<16>(v, col < qk_hd ? qk_gq : qk_gk, cs, sn, map.qk_eps);
          else qk_norm_rope_lane<8>(v, col < qk_hd ? qk_gq : qk_gk, cs, sn, map.qk_eps);
          uint4 out;
          out.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
          out.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
          out.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
          out.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
          *reinterpret_cast<uint4*>(po) = out;
          continue;
        }
      }
      if (!(EPI == EPI_SWIGLU && map.mx_only)) {
        if (col + 8 <= N) *reinterpret_cast<uint4*>(po) = *reinterpret_cast<const uint4*>(src);
        else for (int e = 0; col + e < N; ++e) po[e] = src[e];
      }
      if (EPI == EPI_SWIGLU && map.mx_q) {
        // MX e4m3 copy: a 32-column block is the chunks of 4 adjacent lanes (N % 32 == 0,
        // so a quad is active or skipped as a whole)
        const uint4 raw = *reinterpret_cast<const uint4*>(src);
        const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
        float v[8], am = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = __uint_as_float(u[e] << 16);
          v[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[e]));
        am = fmaxf(am, dpp<0xB1>(am));  // quad_perm [1,0,3,2]
        am = fmaxf(am, dpp<0x4E>(am));  // quad_perm [2,3,0,1]
        const int ex = fp8::e8m0_exp(am);
        const float sc = __builtin_ldexpf(1.0f, -ex);
        const uint32_t w0 = fp8::pack4_e4m3(v[0], v[1], v[2], v[3], sc);
        const uint32_t w1 = fp8::pack4_e4m3(v[4], v[5], v[6], v[7], sc);
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(u32x2_t{w0, w1},
                                    reinterpret_cast<u32x2_t*>(map.mx_q + (int64_t)row * map.mx_ld + col));
        if ((tid & 3) == 0) map.mx_s[(int64_t)row * map.mx_lds + col / 32] = (uint8_t)(ex + 127);
      }
    }
  }
}

}  // namespace gemm_tile
}  // namespace h3
