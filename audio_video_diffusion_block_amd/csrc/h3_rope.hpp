// Q/K RMSNorm + RoPE arithmetic shared by the standalone pass (k_qk_norm_rope)
// and the QKV projection's store epilogue (h3_gemm_tile.hpp), so that the two
// give the same bits.
//
// Why Real-Time MiniMax H3 Serving Requires More Than a Faster DiT, "Key
// takeaways": Q/K RMSNorm and RoPE are one fused operation, and a rank computes
// RoPE only for its own rows.
//
// Pairs (2p, 2p+1) of a head row of D values rotate by an angle proportional
// to the token's position: video tokens use the position on the pair's axis
// (sections [t | h | w] of widths sec_t, sec_h, D - sec_t - sec_h, each an
// independent 1-D RoPE), audio tokens their audio index over one section of
// width D.  The per-position rotation of every pair, in revolutions, is
// computed on the host in double and kept as a 32-bit fixed-point fraction.
// A lane multiplies it by the position in 32-bit integers, which wraps
// exactly to the fractional turn (positions of any size keep the full
// precision and the sine/cosine inputs stay in [0, 1) turns), converts that
// to fp32 and applies the sine and cosine instructions (v_sin_f32/v_cos_f32,
// which take revolutions).
#pragma once

#include <cmath>

#include "h3_common.hpp"

namespace h3 {

struct RopeTab {
  // turns per unit of position, times 2^32 ([0] video, within the pair's
  // section; [1] audio); D <= 128.  Every rate is below 1/(2 pi) turn.
  uint32_t rev[2][64];
  int sec_t = 0, sec_h = 0;
};

inline RopeTab make_rope_tab(int D, int sec_t, int sec_h, float theta) {
  RopeTab t{};
  t.sec_t = sec_t;
  t.sec_h = sec_h;
  const double l2t = std::log2((double)theta);
  const double inv2pi = 1.0 / (2.0 * 3.14159265358979323846);
  auto fixed = [](double turns) { return (uint32_t)std::llround(std::ldexp(turns, 32)); };
  for (int p = 0; p < D / 2 && p < 64; ++p) {
    int jj, width;
    if (p < sec_t / 2) {
      jj = p; width = sec_t;
    } else if (p < (sec_t + sec_h) / 2) {
      jj = p - sec_t / 2; width = sec_h;
    } else {
      jj = p - (sec_t + sec_h) / 2; width = D - sec_t - sec_h;
    }
    t.rev[0][p] = fixed(std::exp2(-2.0 * jj / width * l2t) * inv2pi);
    t.rev[1][p] = fixed(std::exp2(-2.0 * p / D * l2t) * inv2pi);
  }
  return t;
}

// the 4 pairs 4*lane8 .. 4*lane8+3 of a lane holding dims 8*lane8 .. 8*lane8+7
struct RopeLane {
  uint32_t rv[4], ra[4];
  int axis[4];
};

__device__ __forceinline__ RopeLane rope_lane(const RopeTab& t, int lane8) {
  RopeLane r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = 4 * lane8 + j;
    r.rv[j] = t.rev[0][p];
    r.ra[j] = t.rev[1][p];
    r.axis[j] = p < t.sec_t / 2 ? 0 : (p < (t.sec_t + t.sec_h) / 2 ? 1 : 2);
  }
  return r;
}

// cos/sin of the lane's 4 pairs for a token at ps = {kind, t, h, w}
__device__ __forceinline__ void rope_cos_sin(const RopeLane& r, int4 ps, float (&c)[4],
                                             float (&s)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int pv = r.axis[j] == 0 ? ps.y : (r.axis[j] == 1 ? ps.z : ps.w);
    // the fractional turn, exact modulo 2^32 (negative positions wrap too)
    const uint32_t ph = ps.x == 1 ? (uint32_t)ps.y * r.ra[j] : (uint32_t)pv * r.rv[j];
    const float turns = (float)ph * 0x1p-32f;
    s[j] = __builtin_amdgcn_sinf(turns);
    c[j] = __builtin_amdgcn_cosf(turns);
  }
}

// RMSNorm of a head row held by L = D/8 adjacent lanes (8 values each), times
// the gain, then the rotation of the lane's 4 pairs; v in place.  Every lane
// of the L-lane group must run this together.
template <int L>
__device__ __forceinline__ void qk_norm_rope_lane(float (&v)[8], const float* g,
                                                  const float (&c)[4], const float (&s)[4],
                                                  float eps) {
  constexpr int D = 8 * L;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
  ss = group_sum<L>(ss);
  const float rinv = rsqrtf(ss * (1.0f / D) + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = v[i] * rinv * g[i];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = v[2 * j], b = v[2 * j + 1];
    v[2 * j] = a * c[j] - b * s[j];
    v[2 * j + 1] = a * s[j] + b * c[j];
  }
}

}  // namespace h3
