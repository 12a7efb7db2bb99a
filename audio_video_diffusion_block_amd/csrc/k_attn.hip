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
//  * Keys stream in tiles of 64 through a 4-stage LDS ring: K as [64][D]
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
//  * Online softmax in the log2 domain: Q is scaled once by scale*log2(e) and
//    every score chain starts from minus the running max, so scores leave the
//    matrix pipe ready for v_exp_f32.  The running max is raised only when a
//    row max exceeds it by more than 8 (2^8 bound on unnormalised weights), so
//    the O rescale is skipped on most tiles; the final 1/l uses the same stale
//    max, so the result is exact.
//  * Keys beyond the valid length are zero-filled in LDS (K) / scratch (V^T)
//    and their scores masked to -inf, so NaN/Inf pad rows never reach a product.
//  * No atomics, no split over keys: the result is deterministic.
//
// fp32 path: one thread per (query row, head), plain online softmax.
#include "h3_common.hpp"
#include "h3_kernels.hpp"
#include "h3_fp8.hpp"

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

// Accumulator row i of a 32x32 MFMA tile (lane half h, register r) is
// i = (r/4)*8 + h*4 + r%4.  Reading K row sigma(i) into A-operand row i makes
// register r of lane half h hold key (r/8)*16 + h*8 + r%8, i.e. registers
// 0..7 are keys h*8..h*8+7 and registers 8..15 keys 16+h*8.., which is the
// B-operand order of the P.V MFMA over keys 0..15 and 16..31.
__device__ __forceinline__ int sigma_row(int i) {
  const int a = i >> 3;
  return (a >> 1) * 16 + ((i >> 2) & 1) * 8 + (a & 1) * 4 + (i & 3);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two floats -> packed bf16x2 (one v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// raw buffer resource over [base, base + bytes); loads past the end return 0
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
}  // namespace

// ---------------------------------------------- software-pipelined MFMA kernel
//
// LDS layout of one stage: the K tile [64 keys][D + 8] then the V^T tile
// [D][64 + 8] (bf16).  The 16-byte row padding puts the 16 rows that one
// 16-lane group of a ds_read_b128 touches on 16 distinct 4-bank groups, and
// keeps every fragment read a compile-time offset from one per-lane base
// address.  The kernel is software-pipelined so the MFMA and VALU pipes
// overlap: in tile step j a wave issues S(j+1) = K(j+1) Q^T (MFMA,
// independent) while it runs the softmax of S(j) (VALU), then P(j).V(j).  The
// two halves of the work-group run these two phases in opposite order, so the
// two waves sharing a SIMD are in different phases.  Keys go through a 4-stage
// LDS ring with one barrier per tile.  8 waves (256 query rows) share each K/V
// tile; the row sums use v_dot2_f32_bf16 on the packed bf16 P (the values the
// MFMA multiplies).
// SKIP (Skip-Softmax): a wave gives a key tile exactly zero weight and leaves
// out its P.V when, for each of its valid query rows, the tile's largest score
// is more than |skip_log2| (log2 units) below the row's exact running max over
// the tiles before it.  The decision for tile j+1 is taken once its scores are
// known (the row max of phase B) and is uniform over the wave.
template <int D, int NW, bool SKIP = false>
__global__ __launch_bounds__(NW * 64, 1) void attn_fwd_bf16_pipe_kernel(
    const bf16_t* __restrict__ q, int64_t ld_q, const bf16_t* __restrict__ k, int64_t ld_k,
    const bf16_t* __restrict__ vt, int64_t vt_cols, bf16_t* __restrict__ o, int64_t ld_o,
    const int* __restrict__ cu, const int* __restrict__ valid, float scale_log2,
    float skip_log2 = 0.f) {
  constexpr int BMQ = NW * 32;
  constexpr int NTH = NW * 64;
  constexpr int KCH = D / 8;
  constexpr int KS = D + 8;
  constexpr int VS = KT + 8;
  constexpr int K_ELEMS = KT * KS;
  constexpr int STAGE = K_ELEMS + D * VS;
  constexpr int NSTAGE = 4;
  // The softmax scale and log2(e) are folded into Q once (one fp32 product,
  // rounded to bf16), and every score chain starts from -m (negm, the running
  // max in all 16 registers) instead of 0: scores leave the matrix pipe in
  // log2 units relative to the running max, ready for v_exp_f32, with no VALU
  // work per score before the exp.
  __shared__ __attribute__((aligned(16))) bf16_t smem[NSTAGE * STAGE];

  const int s = blockIdx.y;
  const int head = blockIdx.z;
  const int seg_lo = cu[s];
  const int len = seg_valid(cu, valid, s);
  const int q0 = blockIdx.x * BMQ;
  if (q0 >= len) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qi = lane & 31;
  const int hf = lane >> 5;
  const int qrow = q0 + wave * 32 + qi;
  const bool q_ok = qrow < len;
  const int n_tiles = (len + KT - 1) / KT;

  bf16x8_t qf[D / 16];
  {
    const bf16_t* qp = q + (int64_t)(seg_lo + (q_ok ? qrow : 0)) * ld_q + head * D + hf * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 val = q_ok ? *reinterpret_cast<const uint4*>(qp + kk * 16) : make_uint4(0, 0, 0, 0);
      bf16x8_t x = __builtin_bit_cast(bf16x8_t, val);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (__bf16)((float)x[e] * scale_log2);
      qf[kk] = x;
    }
  }

  constexpr int KPT = KT * KCH / NTH;
  constexpr int VPT = D * 8 / NTH;
  static_assert((KT * KCH) % NTH == 0 && (D * 8) % NTH == 0, "tile split");
  const char* kbase = reinterpret_cast<const char*>(k + (int64_t)seg_lo * ld_k + head * D);
  const char* vbase = reinterpret_cast<const char*>(vt + (int64_t)head * D * vt_cols +
                                                    vt_segment_base(seg_lo, s));
  const int k_row_bytes = (int)(ld_k * 2);
  int k_voff[KPT], k_lds[KPT], v_voff[VPT], v_lds[VPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int c = tid + i * NTH, r = c / KCH, ch = c % KCH;
    k_voff[i] = r * k_row_bytes + ch * 16;
    k_lds[i] = r * KS + ch * 8;
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = tid + i * NTH, r = c / 8, ch = c % 8;
    v_voff[i] = r * (int)(vt_cols * 2) + ch * 16;
    v_lds[i] = K_ELEMS + r * VS + ch * 8;
  }
  const int v_bytes = (int)(D * vt_cols * 2);
  // staging registers: tile t is loaded one step before it is stored
  uint4 rk[KPT], rv[VPT];
  // The loads of tile jt+2 are issued one by one inside phase A of step jt
  // (load_begin, then load_part(i) after every fourth MFMA) instead of in one
  // burst after the barrier, where all 8 waves of the CU would issue theirs at
  // once and stall on the address unit.  A load past the last tile re-reads
  // the last tile (in bounds) and is never stored.
  __amdgpu_buffer_rsrc_t ld_rk, ld_rv;
  auto load_begin = [&](int jt) {
    const int j0 = min(jt, n_tiles - 1) * KT;
    ld_rk = make_rsrc(kbase + (int64_t)j0 * k_row_bytes, min(len - j0, KT) * k_row_bytes);
    ld_rv = make_rsrc(vbase + (int64_t)j0 * 2, v_bytes);
  };
  auto load_part = [&](int i) {  // i < KPT: K chunk i, else V^T chunk i - KPT
    if (i < KPT) rk[i] = buf_load16(ld_rk, k_voff[i]);
    else rv[i - KPT] = buf_load16(ld_rv, v_voff[i - KPT]);
  };
  auto load_tile = [&](int jt) {
    const int j0 = jt * KT;
    const __amdgpu_buffer_rsrc_t rs_k =
        make_rsrc(kbase + (int64_t)j0 * k_row_bytes, min(len - j0, KT) * k_row_bytes);
    const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(vbase + (int64_t)j0 * 2, v_bytes);
#pragma unroll
    for (int i = 0; i < KPT; ++i) rk[i] = buf_load16(rs_k, k_voff[i]);
#pragma unroll
    for (int i = 0; i < VPT; ++i) rv[i] = buf_load16(rs_v, v_voff[i]);
  };
  auto store_tile = [&](int stage) {
    bf16_t* st = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < KPT; ++i) *reinterpret_cast<uint4*>(st + k_lds[i]) = rk[i];
#pragma unroll
    for (int i = 0; i < VPT; ++i) *reinterpret_cast<uint4*>(st + v_lds[i]) = rv[i];
  };

  const int k_frag = sigma_row(qi) * KS + hf * 8;
  const int v_frag = K_ELEMS + qi * VS + hf * 8;
  auto compute_s = [&](int stage, f32x16_t (&sc)[2]) {
    const bf16_t* st = smem + stage * STAGE;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[0][r] = sc[1][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(st + k_frag + kk * 16);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(st + k_frag + 32 * KS + kk * 16);
      sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kk], sc[0], 0, 0, 0);
      sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kk], sc[1], 0, 0, 0);
    }
  };

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  f32x16_t negm;             // -(running max) in every register
  float mt_rel = 0.f;        // SKIP: exact running max, relative to the running max
  float l_a = 0.f, l_b = 0.f;
  typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
  const bf16x2v_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  auto kfrag = [&](const bf16_t* sk, int kk, int ch) {
    return *reinterpret_cast<const bf16x8_t*>(sk + k_frag + ch * 32 * KS + kk * 16);
  };
  // V^T fragment of P.V group g (keys g*16 .. g*16+15 of the tile) and d block db
  auto vfrag = [&](const bf16_t* sv, int g, int db) {
    return *reinterpret_cast<const bf16x8_t*>(sv + v_frag + db * 32 * VS + g * 16);
  };
  auto mask_tile = [&](f32x16_t (&sc)[2], int jt) {
    const int base = jt * KT;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = base + kb * 32 + (r >> 3) * 16 + hf * 8 + (r & 7);
        if (key >= len) sc[kb][r] = -INFINITY;
      }
  };
  // mx: the lane's largest score of the tile (sc) relative to the running
  // max.  SKIP: the tile is skipped when every valid row's max is more than
  // |skip_log2| below its exact running max (mt_rel); a skipped tile's scores
  // become -inf, so its weights are exactly 0.  Then the running max is raised
  // to the tile max when that exceeds it by more than 8 (2^8 bound on the
  // unnormalised weights), rescaling O and l and shifting sc, negm and mt_rel;
  // skipped on most tiles.  Returns whether the tile is skipped.
  auto update_max = [&](float mx, f32x16_t (&sc)[2]) -> bool {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
    bool skip = false;
    if constexpr (SKIP) {
      skip = __all(!q_ok || mx < mt_rel + skip_log2);
      mt_rel = fmaxf(mt_rel, mx);
    }
    const bool raise = mx > 8.0f;
    if (__any(raise)) {
      const float delta = raise ? mx : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      l_a *= alpha;
      l_b *= alpha;
      if constexpr (SKIP) mt_rel -= delta;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        negm[r] -= delta;
        sc[0][r] -= delta;
        sc[1][r] -= delta;
      }
    }
    if constexpr (SKIP) {
      if (skip)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[0][r] = sc[1][r] = -INFINITY;
    }
    return skip;
  };

  // A tile step is two phases, hand-ordered so that each keeps both pipes fed:
  //  phase A: S(next) = K(next) Q^T (16 MFMAs), each followed by 1/16 of the
  //           softmax of S(cur): 2 exp + 1 pack + 1 dot2 (VALU-heavy), and
  //           every fourth by one load of tile jt+2;
  //  phase B: O^T += V(cur)^T P^T (16 MFMAs), each followed by one step of the
  //           row max of S(next) (MFMA-heavy).
  // LDS fragments are read 4 MFMAs ahead.  sched_barrier(0) keeps the order.
  // P (packed bf16) and the first V^T fragments pass from phase A to phase B.
  uint32_t w[4][4];
  bf16x8_t vf[4];
  constexpr int NA = 2 * (D / 16);  // phase A MFMAs: 2 key blocks x D/16 k-steps
  constexpr int NB = 4 * (D / 32);  // phase B MFMAs: 4 key groups x D/32 d blocks
  // SKIP: the softmax of a skipped tile runs on -inf scores, so its weights
  // are exactly 0 and its row sums unchanged (branch-free: a branch per slot
  // costs more than the VALU work it saves)
  auto phase_a = [&](int stage_k, f32x16_t (&nxt)[2], int stage_v, f32x16_t (&cur)[2], int jt,
                     bool skip) {
    const bf16_t* sk = smem + stage_k * STAGE;
    // the wave in this (VALU-heavy) phase wins issue arbitration against the
    // other wave of its SIMD, whose P.V MFMAs then fill the matrix pipe
    __builtin_amdgcn_s_setprio(2);
    const bf16_t* sv = smem + stage_v * STAGE;
    constexpr int SL = 16 / NA;       // softmax slices (2 exps each) per phase-A MFMA
    bf16x8_t kf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kf[i] = kfrag(sk, i >> 1, i & 1);
    load_begin(jt + 2);
    // Slot i: one MFMA of S(next), the fma/exp of softmax slice i and the
    // pack/row-sum of slice i-1 (so a pack never waits on the exp it consumes:
    // in-order issue would stall the wave there).
    float pe[2][SL][2];  // exp results in flight, by slot parity
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      nxt[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i & 3], qf[i >> 1],
                                                          i < 2 ? negm : nxt[i & 1], 0, 0, 0);
      if (i % 4 == 3 && i / 4 < KPT + VPT) load_part(i / 4);
      if (i + 4 < NA) kf[i & 3] = kfrag(sk, (i + 4) >> 1, (i + 4) & 1);
      else {
        const int pidx = i + 4 - NA;  // first P.V fragments of phase B
        vf[pidx & 3] = vfrag(sv, pidx / (D / 32), pidx % (D / 32));
      }
#pragma unroll
      for (int sl = 0; sl < SL; ++sl) {
        const int slice = i * SL + sl;
        const int g = slice >> 2, t = slice & 3, kb = g >> 1, half = g & 1;
        pe[i & 1][sl][0] = __builtin_amdgcn_exp2f(cur[kb][half * 8 + 2 * t]);
        pe[i & 1][sl][1] = __builtin_amdgcn_exp2f(cur[kb][half * 8 + 2 * t + 1]);
      }
      if (i > 0) {
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) {
          const int slice = (i - 1) * SL + sl;
          const int g = slice >> 2, t = slice & 3;
          w[g][t] = cvt_pk_bf16(pe[(i - 1) & 1][sl][0], pe[(i - 1) & 1][sl][1]);
          // keep this slice here, next to its MFMA (no sinking past the mask branch)
          asm volatile("" ::"v"(w[g][t]));
          if (t & 1) l_b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, w[g][t]), ones, l_b, false);
          else l_a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, w[g][t]), ones, l_a, false);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int sl = 0; sl < SL; ++sl) {
      const int slice = (NA - 1) * SL + sl;
      const int g = slice >> 2, t = slice & 3;
      w[g][t] = cvt_pk_bf16(pe[(NA - 1) & 1][sl][0], pe[(NA - 1) & 1][sl][1]);
      if (t & 1) l_b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, w[g][t]), ones, l_b, false);
      else l_a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, w[g][t]), ones, l_a, false);
    }
    __builtin_amdgcn_s_setprio(0);
    if (jt + 1 < n_tiles && (jt + 2) * KT > len) mask_tile(nxt, jt + 1);
  };
  // nxt holds S(jt+1), written by phase A of tile jt.  SKIP: a skipped tile's
  // P.V MFMAs are left out; returns whether tile jt+1 is skipped.
  auto phase_b = [&](int stage_v, f32x16_t (&nxt)[2], int jt, bool skip) -> bool {
    const bf16_t* sv = smem + stage_v * STAGE;
    constexpr int MX = 32 / NB;       // scores folded into the max per phase-B MFMA
    // Slot i: one P.V MFMA and the row-max step of score pair group i-2 (the
    // first two slots let the last S(next) MFMAs finish).
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NB + 2; ++i) {
      if (i < NB) {
        const int g = i / (D / 32), db = i % (D / 32);
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, make_uint4(w[g][0], w[g][1], w[g][2], w[g][3]));
        if (!(SKIP && skip))
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i & 3], pb, oacc[db], 0, 0, 0);
        if (i + 4 < NB) vf[i & 3] = vfrag(sv, (i + 4) / (D / 32), (i + 4) % (D / 32));
      }
      if (i >= 2) {
#pragma unroll
        for (int e = 0; e < MX; ++e) {
          const int idx = (i - 2) * MX + e;
          mx = fmaxf(mx, nxt[idx >> 4][idx & 15]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (jt + 1 < n_tiles) return update_max(mx, nxt);
    return false;
  };

  load_tile(0);
  store_tile(0);
  if (n_tiles > 1) {
    load_tile(1);
    store_tile(1);
  }
  __syncthreads();
  f32x16_t sa[2], sb[2];
  compute_s(0, sa);
  if (n_tiles == 1) mask_tile(sa, 0);
  {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sa[kb][r]);
    // the first reference: the exact max of S(0) (finite: a tile has a valid
    // key); the first tile is never skipped
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    const float m0 = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sa[0][r] -= m0;
      sa[1][r] -= m0;
      negm[r] = -m0;
    }
  }

  // Phase rotation: the two wave halves of the work-group share each SIMD
  // (waves w and w + NW/2).  The first half runs A(jt) then B(jt) in step jt;
  // the second runs B(jt-1) then A(jt).  Both do the same work between two
  // barriers, but at any moment one wave of a SIMD is in its VALU-heavy phase
  // while the other feeds the matrix core.
  // During step jt the ring holds tiles jt-1 (V, second half), jt (V, first
  // half) and jt+1 (K, both halves); tile jt+2 is loaded into registers during
  // phase A and stored to the fourth stage before the barrier.
  // After the last tile, S(next) reads a stale stage and is discarded.
  const bool lag = __builtin_amdgcn_readfirstlane(wave) >= NW / 2;
  // SKIP flags: sk_cur for the tile whose softmax runs in this step, sk_prev
  // for the lagging half's P.V of the tile before it
  bool sk_cur = false, sk_prev = false;
  auto step = [&](int jt, f32x16_t (&cur)[2], f32x16_t (&nxt)[2]) {
    if (lag && jt > 0) {
      sk_prev = sk_cur;
      sk_cur = phase_b((jt - 1) % NSTAGE, cur, jt - 1, sk_prev);
    }
    phase_a((jt + 1) % NSTAGE, nxt, jt % NSTAGE, cur, jt, sk_cur);
    if (!lag) sk_cur = phase_b(jt % NSTAGE, nxt, jt, sk_cur);
    if (jt + 2 < n_tiles) store_tile((jt + 2) % NSTAGE);
    __syncthreads();
  };
  for (int jt = 0; jt < n_tiles; jt += 2) {
    step(jt, sa, sb);
    if (jt + 1 >= n_tiles) break;
    step(jt + 1, sb, sa);
  }
  if (lag) {
    // S(n_tiles) sits in sb when n_tiles is odd, else in sa (unused: no max update)
    if (n_tiles & 1) phase_b((n_tiles - 1) % NSTAGE, sb, n_tiles - 1, sk_cur);
    else phase_b((n_tiles - 1) % NSTAGE, sa, n_tiles - 1, sk_cur);
  }

  float l_run = l_a + l_b;
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
      val.x = cvt_pk_bf16(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
      val.y = cvt_pk_bf16(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
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

template <int D, bool SKIP = false>
static hipError_t launch_attn_d(bool bf16, const void* q, int64_t ld_q, const void* k,
                                int64_t ld_k, const void* v, int64_t ld_v, void* o,
                                int64_t ld_o, int64_t n_buf, int n_heads, const int* cu,
                                const int* valid, int n_seg, int max_len, float scale, void* ws,
                                hipStream_t s, float skip_log2 = 0.f) {
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
    constexpr int NW = 8;
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((attn_fwd_bf16_pipe_kernel<D, NW, SKIP>),
                       dim3((unsigned)ceil_div(max_len, NW * 32), n_seg, n_heads), dim3(NW * 64), 0,
                       s, (const bf16_t*)q, ld_q, (const bf16_t*)k, ld_k, (const bf16_t*)ws, cols,
                       (bf16_t*)o, ld_o, cu, valid, scale_log2, skip_log2);
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

hipError_t launch_varlen_attn_skip(int head_dim, const void* q, int64_t ld_q, const void* k,
                                   int64_t ld_k, const void* v, int64_t ld_v, void* o,
                                   int64_t ld_o, int64_t n_buf, int n_heads, const int* cu,
                                   const int* valid, int n_seg, int max_len, float scale,
                                   float skip_log2, void* ws, hipStream_t s) {
  if (head_dim == 128)
    return launch_attn_d<128, true>(true, q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, cu,
                                    valid, n_seg, max_len, scale, ws, s, skip_log2);
  return launch_attn_d<64, true>(true, q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, cu,
                                 valid, n_seg, max_len, scale, ws, s, skip_log2);
}


// ================================================================== FP8 path
//
// MiniMax H3 通过 vLLM-Omni 实现 FastH3 实时推理, "超出 FastH3 配置的扩展能力" (sparse and
// quantized attention): an FP8 attention path (SAGE FP8) speeds up the base
// pipeline at small quality cost.  The pages give no algorithm; this path
// stores Q (softmax scale and log2 e folded in), K and V as OCP e4m3 with one
// power-of-two (E8M0) scale per 32 elements along the contraction (head dim
// for Q and K, keys for V), and rounds the probabilities to e4m3 as 256 * p.
// Block format and MFMA operand layout: h3_fp8.hpp.
using namespace fp8;


// Rows of a head slice (bf16, row stride ld, head h at columns h*D), times
// `fold` (one fp32 rounding) -> e4m3 [heads][n_buf][D] and E8M0 bytes
// [heads][n_buf][D/32] stored even blocks first, then odd blocks (lane half h
// of the MFMA takes blocks 2t + h).  Rows outside every segment's valid range
// are written as zeros (scale byte 127).  One thread per 32-element block.
template <int D>
__global__ __launch_bounds__(256) void quant_rows_e4m3_kernel(const bf16_t* __restrict__ x,
                                                              int64_t ld, int64_t n_buf, int heads,
                                                              const int* cu, const int* valid,
                                                              int n_seg, float fold,
                                                              uint8_t* __restrict__ q8,
                                                              uint8_t* __restrict__ sc) {
  constexpr int NB = D / 32;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)heads * n_buf * NB) return;
  const int blk = (int)(t % NB);
  const int64_t hr = t / NB;
  const int64_t row = hr % n_buf;
  const int head = (int)(hr / n_buf);
  const int s = find_segment(cu, n_seg, row);
  const bool ok = s >= 0 && row - cu[s] < seg_valid(cu, valid, s);
  uint4* dst = reinterpret_cast<uint4*>(q8 + ((int64_t)head * n_buf + row) * D + blk * 32);
  uint8_t* sdst = sc + ((int64_t)head * n_buf + row) * NB + (blk & 1) * (NB / 2) + (blk >> 1);
  if (!ok) {
    dst[0] = make_uint4(0, 0, 0, 0);
    dst[1] = make_uint4(0, 0, 0, 0);
    *sdst = 127;
    return;
  }
  const uint4* src = reinterpret_cast<const uint4*>(x + row * ld + head * D + blk * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = src[i];
    const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * i + 2 * k] = __uint_as_float(ws[k] << 16) * fold;
      v[8 * i + 2 * k + 1] = __uint_as_float(ws[k] & 0xffff0000u) * fold;
    }
  }
  uint32_t w[8];
  *sdst = (uint8_t)quant32(v, w);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// V [rows, heads*D] (row stride ld_v) -> V^T e4m3 [heads][D][cols] with the
// columns of vt_segment_base, and E8M0 bytes [heads][cols/32][D] (one per
// 32 keys and dimension).  Keys past the valid length are zeros.  One
// work-group transposes 64 keys x D dims of one head.
template <int D>
__global__ __launch_bounds__(256) void transpose_quant_v_kernel(const bf16_t* __restrict__ v,
                                                                int64_t ld_v,
                                                                uint8_t* __restrict__ vt8,
                                                                uint8_t* __restrict__ vts,
                                                                int64_t cols, const int* cu,
                                                                const int* valid) {
  __shared__ float tile[64][D + 1];
  const int s = blockIdx.y;
  const int head = blockIdx.z;
  const int lo = cu[s];
  const int len = seg_valid(cu, valid, s);
  const int j0 = blockIdx.x * 64;
  if (j0 >= len) return;
  constexpr int CPR = D / 8;
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int r = i / CPR, c = i % CPR;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (j0 + r < len)
      val = *reinterpret_cast<const uint4*>(v + (int64_t)(lo + j0 + r) * ld_v + head * D + c * 8);
    const uint32_t ws[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      tile[r][c * 8 + 2 * k] = __uint_as_float(ws[k] << 16);
      tile[r][c * 8 + 2 * k + 1] = __uint_as_float(ws[k] & 0xffff0000u);
    }
  }
  __syncthreads();
  const int64_t base = vt_segment_base(lo, s) + j0;  // a multiple of 64
  for (int i = threadIdx.x; i < 2 * D; i += 256) {
    const int d = i % D, b = i / D;
    float vv[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) vv[k] = tile[b * 32 + k][d];
    uint32_t w[8];
    const uint32_t e = quant32(vv, w);
    uint4* dst = reinterpret_cast<uint4*>(vt8 + ((int64_t)head * D + d) * cols + base + b * 32);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    vts[((int64_t)head * (cols / 32) + (base / 32) + b) * D + d] = (uint8_t)e;
  }
}


// FP8 flash attention.  Same work split and phase rotation as the bf16
// kernel; per 64-key tile a wave runs 2*(D/64) MFMAs for S and D/32 for P.V,
// each 64 deep.
//  * Scores: S^T = K Q^T with K rows read in the order sigma8 below, so the
//    accumulator register r of lane half h in key block kb holds key
//    32 kb + 16 h + r -- exactly the byte (16 kb + r) the P.V MFMA expects in
//    its B operand.  P never leaves registers.
//  * The scores come out in log2 units (the softmax scale and log2 e are in
//    Q).  They are kept relative to m_ref = M - 8, where the reference M is an
//    integer: the ceiling of the first tile's max, raised to the ceiling of a
//    later tile's max whenever that exceeds M by more than 0.75, so every
//    stored weight 2^(s - m_ref) = 256 * 2^(s - M) is at most 2^8.75 < 448.
//    Because M is an integer, the e4m3 value of a weight is the same as for
//    the reference ceil(row max) wherever it is an e4m3 normal, so the stored
//    weights do not depend on the tiling, and each raise rescales O and the
//    row sums by an exact power of two.  The weights are stored as e4m3 with
//    scale byte 127.  The row sums come from the matrix pipe: one more P.V
//    MFMA whose A operand is all e4m3 ones sums the stored weights of every
//    query, so numerator and denominator see the same rounded 256 p.
//  * Tiles go from global memory straight into LDS (global_load_lds_dwordx4:
//    no staging registers, no LDS stores), into a 5-stage ring: tile t + 4 is
//    requested right after the barrier of step t and has two steps to land.
//    Rows past the valid keys are clamped to the last valid row (their scores
//    are masked).
//  * LDS rows are unpadded; 16-byte chunk c of a row r sits at slot
//    c ^ swz(r), chosen so that the 16 rows one 16-lane group of a fragment
//    read touches (for K, in the sigma8 order) fall on 16 distinct bank groups.
namespace {
// K row read into A-operand row rho of a 32-key block
__device__ __forceinline__ int sigma8(int rho) {
  return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
}
__device__ __forceinline__ i32x8_t frag32(const uint8_t* p0, const uint8_t* p1) {
  const uint4 a = *reinterpret_cast<const uint4*>(p0);
  const uint4 b = *reinterpret_cast<const uint4*>(p1);
  i32x8_t r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}
}  // namespace

// SKIP (Skip-Softmax): as in the bf16 kernel, a wave gives a key tile zero
// weight when every valid row's tile max is more than |skip_log2| below its
// exact running max.  Here the softmax is most of the VALU work, so a skipped
// tile branches around its softmax slots; its packed P is zeroed instead, and
// its P.V and row-sum MFMAs then add exact zeros (no branch in phase B).
template <int D, int NW, bool SKIP = false>
__global__ __launch_bounds__(NW * 64, 1) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ qs,
    const uint8_t* __restrict__ k8, const uint8_t* __restrict__ ks, int64_t n_buf,
    const uint8_t* __restrict__ vt8, const uint8_t* __restrict__ vts, int64_t vt_cols,
    bf16_t* __restrict__ o, int64_t ld_o, const int* __restrict__ cu,
    const int* __restrict__ valid, float skip_log2 = 0.f) {
  constexpr int BMQ = NW * 32;
  constexpr int NTH = NW * 64;
  constexpr int NT = D / 64;          // 64-deep steps of S (1 or 2)
  static_assert(NT == 1 || NT == 2, "head_dim 64 or 128");
  constexpr int NB = D / 32;          // 32-element scale blocks of a head row
  constexpr int K_OFF = 0;                  // K [KT][D] bytes, swizzled rows
  constexpr int V_OFF = KT * D;             // V^T [D][KT] bytes, swizzled rows
  constexpr int KS_OFF = V_OFF + D * KT;    // K scales [KT][NB]
  constexpr int VS_OFF = KS_OFF + KT * NB;  // V^T scales [2][D]
  constexpr int STAGE = VS_OFF + 2 * D;
  static_assert(STAGE % 16 == 0 && KT == 64, "stage layout");
  constexpr int NSTAGE = 5;
  __shared__ __attribute__((aligned(16))) uint8_t smem[NSTAGE * STAGE];

  const int s = blockIdx.y;
  const int head = blockIdx.z;
  const int seg_lo = cu[s];
  const int len = seg_valid(cu, valid, s);
  const int q0 = blockIdx.x * BMQ;
  if (q0 >= len) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qi = lane & 31;
  const int hf = lane >> 5;
  const int qrow = q0 + wave * 32 + qi;
  const bool q_ok = qrow < len;
  const int n_tiles = (len + KT - 1) / KT;

  // ---- Q fragments (B operand of S) and their scale bytes, once
  i32x8_t qf[NT];
  uint32_t qsc = 0x7f7f7f7fu;
  {
    const uint8_t* qp = q8 + ((int64_t)head * n_buf + seg_lo + (q_ok ? qrow : 0)) * D + 16 * hf;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (q_ok) qf[t] = frag32(qp + 64 * t, qp + 64 * t + 32);
      else
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[t][i] = 0;
    }
    if (q_ok) {
      const uint8_t* sp = qs + ((int64_t)head * n_buf + seg_lo + qrow) * NB + hf * (NB / 2);
      qsc = NB / 2 == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(sp) : (uint32_t)*sp;
    }
  }

  // ---- tile loads: global -> LDS directly.  Per tile, K takes D/16 1-KB
  // instructions (waves 0 ..), V^T D/16 (the last waves), the K scales (2 D
  // bytes) part of one more on wave 0 and the V^T scales on wave NW - 1.
  // The DMA instructions are inline assembly: the compiler would otherwise
  // count them as pending LDS operations and make fragment reads wait on them;
  // their completion is tracked with explicit vmcnt waits before barriers.
  constexpr int KI = D / 16;                         // K instructions per tile
  constexpr int VI = D / 16;                         // V^T instructions per tile
  static_assert(KI <= NW && VI <= NW, "one instruction per wave");
  const char* kbase = reinterpret_cast<const char*>(k8 + ((int64_t)head * n_buf + seg_lo) * D);
  const char* ksb = reinterpret_cast<const char*>(ks + ((int64_t)head * n_buf + seg_lo) * NB);
  const int64_t vbase_col = vt_segment_base(seg_lo, s);
  const char* vbase = reinterpret_cast<const char*>(vt8 + (int64_t)head * D * vt_cols + vbase_col);
  const char* vsb = reinterpret_cast<const char*>(vts + ((int64_t)head * (vt_cols / 32) + vbase_col / 32) * D);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // swizzles (slot of chunk c in row r is c ^ swz(r)); see the bank argument above
  auto kswz = [](int r) { return D == 128 ? (((r >> 1) + 4 * (r >> 4)) & 7) : (((r >> 2) ^ (r >> 3)) & 3); };
  auto vswz = [](int r) { return ((r >> 2) ^ (r >> 3)) & 3; };
  constexpr int KCPR = D / 16;                       // 16-byte chunks per K row
  constexpr int KRPI = 1024 / D;                     // K rows per instruction
  const int k_dma_row = wv * KRPI + lane / KCPR;     // used by waves wv < KI
  const int k_dma_chunk = (lane % KCPR) ^ kswz(k_dma_row);
  const int v_dma_row = (wv - (NW - VI)) * 16 + lane / 4;   // used by waves wv >= NW - VI
  const int v_dma_off = v_dma_row * (int)vt_cols + ((lane % 4) ^ vswz(v_dma_row)) * 16;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;
  auto dma16 = [&](const char* base, int voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds_addr) : "memory", "m0");
  };
  // DMA instructions this wave issues per tile (every wave runs every tile)
  const int n_dma = (wv < KI) + (wv >= NW - VI) + (wv == 0) + (wv == NW - 1);
  auto issue_tile = [&](int jt) {
    const int j0 = jt * KT;
    const int nk = min(len - j0, KT);
    const uint32_t st = lds0 + (jt % NSTAGE) * STAGE;
    if (wv < KI)
      dma16(kbase + (int64_t)j0 * D, min(k_dma_row, nk - 1) * D + k_dma_chunk * 16,
            st + K_OFF + wv * 1024);
    if (wv >= NW - VI)
      dma16(vbase + j0, v_dma_off, st + V_OFF + (wv - (NW - VI)) * 1024);
    // scales: 16-byte chunks wholly past the valid rows are skipped (the stale
    // LDS scales they would have replaced belong to masked keys)
    if (wv == 0 && lane < 2 * D / 16 && lane * 16 < nk * NB)
      dma16(ksb + (int64_t)j0 * NB, lane * 16, st + KS_OFF);
    if (wv == NW - 1 && lane < 2 * D / 16)
      dma16(vsb + (int64_t)(j0 / 32) * D, lane * 16, st + VS_OFF);
  };
  // wait until at most `tiles` tiles of this wave's DMA are still in flight
  auto wait_dma = [&](int tiles) {
    const int n = tiles * n_dma;
    if (n == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else if (n == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if (n == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if (n == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  };

  // ---- fragment addressing
  const int k_row = sigma8(qi);
  int k_slot[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int p = 0; p < 2; ++p) k_slot[t][p] = ((4 * t + 2 * p + hf) ^ kswz(k_row)) * 16;
  const int v_slot0 = (hf ^ vswz(qi)) * 16, v_slot1 = ((2 + hf) ^ vswz(qi)) * 16;
  auto kfrag = [&](const uint8_t* st, int kb, int t) {
    const uint8_t* p = st + K_OFF + (kb * 32 + k_row) * D;
    return frag32(p + k_slot[t][0], p + k_slot[t][1]);
  };
  auto kscale = [&](const uint8_t* st, int kb) {
    const uint8_t* p = st + KS_OFF + (kb * 32 + k_row) * NB + hf * (NB / 2);
    return NB / 2 == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(p) : (uint32_t)*p;
  };
  auto vfrag = [&](const uint8_t* st, int db) {
    const uint8_t* p = st + V_OFF + (db * 32 + qi) * KT;
    return frag32(p + v_slot0, p + v_slot1);
  };
  auto vscale = [&](const uint8_t* st, int db) {
    return (uint32_t)st[VS_OFF + hf * D + db * 32 + qi];
  };

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  // Scores are kept relative to m_ref = M - 8 (M an integer): each score chain
  // starts from negm (= -m_ref in all 16 registers), so exp2 of a score is
  // 256 * 2^(s - M).
  float m_ref = 0.f;
  float mt_rel = 8.f;        // SKIP: exact running max, relative to m_ref
  f32x16_t negm;
  f32x16_t lacc;             // row sums of the stored weights (register 0 is used)
#pragma unroll
  for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
  i32x8_t ones8;             // e4m3 1.0 in every byte
#pragma unroll
  for (int r = 0; r < 8; ++r) ones8[r] = 0x38383838;
  constexpr uint32_t PSC = 127u;  // P is stored as 256 p; the row sums carry the same 256

  auto mask_tile = [&](f32x16_t (&sc)[2], int jt) {
    const int base = jt * KT;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (base + kb * 32 + 16 * hf + r >= len) sc[kb][r] = -INFINITY;
  };
  auto update_max = [&](float mx, f32x16_t (&sc)[2]) -> bool {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
    bool skip = false;
    if constexpr (SKIP) {
      skip = __all(!q_ok || mx < mt_rel + skip_log2);
      mt_rel = fmaxf(mt_rel, mx);
    }
    const bool raise = mx > 8.75f;  // tile max above M + 0.75
    if (__any(raise)) {
      scaled_mfma_drain();
      // M moves up by a whole number (>= 1): to the ceiling of the tile max
      const float delta = raise ? ceilf(mx - 8.0f) : 0.f;
      const float alpha = __builtin_ldexpf(1.0f, -(int)delta);
      m_ref += delta;
      if constexpr (SKIP) mt_rel -= delta;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[0][r] -= delta;
        sc[1][r] -= delta;
        negm[r] = -m_ref;
      }
      lacc[0] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    return skip;
  };
  auto compute_s = [&](int stage, f32x16_t (&sc)[2]) {
    const uint8_t* st = smem + stage * STAGE;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
      const uint32_t ksc = kscale(st, kb);
      sc[kb] = mfma_e4m3<0>(kfrag(st, kb, 0), qf[0], sc[kb], ksc, qsc);
      if constexpr (NT > 1) sc[kb] = mfma_e4m3<1>(kfrag(st, kb, 1), qf[NT - 1], sc[kb], ksc, qsc);
    }
  };

  // P of the current tile, packed in the B-operand byte order of P.V
  i32x8_t pw = {0, 0, 0, 0, 0, 0, 0, 0};
  constexpr int NA = 2 * NT;       // phase A MFMAs
  constexpr int NBM = D / 32;      // phase B MFMAs
  constexpr int SPS = 32 / NA;     // scores per phase-A slot (multiple of 4)
  static_assert(SPS % 4 == 0, "slot holds whole packed words");
  // phase A: S(next) MFMAs, each followed by 1/NA of the softmax of S(cur)
  auto phase_a = [&](int stage_k, f32x16_t (&nxt)[2], f32x16_t (&cur)[2], int jt,
                     bool skip) {
    const uint8_t* sk = smem + stage_k * STAGE;
    __builtin_amdgcn_s_setprio(2);
    uint32_t ksc[2];
    ksc[0] = kscale(sk, 0);
    ksc[1] = kscale(sk, 1);
    i32x8_t kf = kfrag(sk, 0, 0);
    nxt[0] = negm;
    nxt[1] = negm;
    if constexpr (SKIP) {
      // a skipped tile's P.V and row sums then add exact zeros
      if (skip)
#pragma unroll
        for (int w = 0; w < 8; ++w) pw[w] = 0;
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int kb = i & 1, t = i >> 1;
      const i32x8_t a = kf;
      if (i + 1 < NA) kf = kfrag(sk, (i + 1) & 1, (i + 1) >> 1);
      if (t == 0) nxt[kb] = mfma_e4m3<0>(a, qf[0], nxt[kb], ksc[kb], qsc);
      else nxt[kb] = mfma_e4m3<1>(a, qf[NT - 1], nxt[kb], ksc[kb], qsc);
      if (!(SKIP && skip)) {
#pragma unroll
      for (int w4 = 0; w4 < SPS / 4; ++w4) {
        const int word = i * (SPS / 4) + w4;  // packed word 0..7: scores 4*word .. 4*word+3
        const int pkb = word >> 2, r0 = (word & 3) * 4;
        float pv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          pv[u] = __builtin_amdgcn_exp2f(cur[pkb][r0 + u]);  // 256 p
        }
        // the first conversion's upper half is overwritten by the second
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], pw[word], false);
        pw[word] = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], lo, true);
        // keep this slice next to its MFMA (no sinking past the mask branch)
        asm volatile("" ::"v"(pw[word]));
      }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    if (jt + 1 < n_tiles && (jt + 2) * KT > len) {
      scaled_mfma_drain();
      mask_tile(nxt, jt + 1);
    }
  };
  // phase B: P.V MFMAs, each followed by part of the row max of S(next)
  // returns whether tile jt+1 is skipped (SKIP)
  auto phase_b = [&](int stage_v, f32x16_t (&nxt)[2], int jt, bool skip,
                     bool last = false) -> bool {
    const uint8_t* sv = smem + stage_v * STAGE;
    float mx = -INFINITY;
    i32x8_t vf[NBM];
    uint32_t vsc[NBM];
#pragma unroll
    for (int db = 0; db < NBM; ++db) {
      vf[db] = vfrag(sv, db);
      vsc[db] = vscale(sv, db);
    }
    lacc = mfma_e4m3<0>(ones8, pw, lacc, 127u, PSC);
#pragma unroll
    for (int db = 0; db < NBM; ++db) {
      oacc[db] = mfma_e4m3<0>(vf[db], pw, oacc[db], vsc[db], PSC);
#pragma unroll
      for (int e = 0; e < 32 / NBM; ++e) {
        const int idx = db * (32 / NBM) + e;
        mx = fmaxf(mx, nxt[idx >> 4][idx & 15]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // after the last tile's P.V the epilogue reads O: let these MFMAs finish
    if (last || jt + 1 >= n_tiles) scaled_mfma_drain();
    if (jt + 1 < n_tiles) return update_max(mx, nxt);
    return false;
  };

  // tiles 0 .. 3 in flight; 0 and 1 must land before the first step
  for (int t = 0; t < 4 && t < n_tiles; ++t) issue_tile(t);
  wait_dma(n_tiles > 3 ? 2 : (n_tiles > 2 ? 1 : 0));
  __syncthreads();
  f32x16_t sa[2], sb[2];
  compute_s(0, sa);
  if (n_tiles == 1) mask_tile(sa, 0);
  {
    // first reference: M = ceil(max of S(0)) (finite: a tile has a valid key)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sa[kb][r]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
    m_ref = ceilf(mx) - 8.0f;
    if constexpr (SKIP) mt_rel = mx - m_ref;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sa[0][r] -= m_ref;
      sa[1][r] -= m_ref;
      negm[r] = -m_ref;
    }
  }

  // During step jt the ring holds tiles jt-1 (V, second half), jt (V, first
  // half) and jt+1 (K, both halves); jt+2 and jt+3 are in flight.  Tile jt+2
  // is waited for before the barrier that ends the step, and tile jt+4 goes
  // into the stage of tile jt-1 right after it.
  const bool lag = wv >= NW / 2;
  // SKIP flags: sk_cur for the tile whose softmax runs in this step, sk_prev
  // for the lagging half's P.V of the tile before it
  bool sk_cur = false, sk_prev = false;
  auto step = [&](int jt, f32x16_t (&cur)[2], f32x16_t (&nxt)[2]) {
    if (lag && jt > 0) {
      sk_prev = sk_cur;
      sk_cur = phase_b((jt - 1) % NSTAGE, cur, jt - 1, sk_prev);
    }
    phase_a((jt + 1) % NSTAGE, nxt, cur, jt, sk_cur);
    if (!lag) sk_cur = phase_b(jt % NSTAGE, nxt, jt, sk_cur);
    wait_dma(jt + 3 < n_tiles ? 1 : 0);
    __syncthreads();
    if (jt + 4 < n_tiles) issue_tile(jt + 4);
  };
  for (int jt = 0; jt < n_tiles; jt += 2) {
    step(jt, sa, sb);
    if (jt + 1 >= n_tiles) break;
    step(jt + 1, sb, sa);
  }
  // the lagging half's last P.V (its score argument is unused: no max follows)
  if (lag) phase_b((n_tiles - 1) % NSTAGE, sa, n_tiles - 1, sk_cur, true);

  const float l_tot = lacc[0];  // every accumulator row holds the query's sum
  if (!q_ok) return;
  const float inv = 1.0f / l_tot;
  bf16_t* op = o + (int64_t)(seg_lo + qrow) * ld_o + head * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + hf * 4;
      uint2 val;
      val.x = cvt_pk_bf16(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
      val.y = cvt_pk_bf16(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d) = val;
    }
  }
}

// workspace: Q and K e4m3 [heads][n_buf][D] + scales, V^T e4m3 [heads][D][cols] + scales
size_t attn_fp8_workspace_bytes(int64_t n_buf, int n_heads, int head_dim, int n_seg) {
  const int64_t cols = vt_columns(n_buf, n_seg);
  const int64_t qk = round_up((int64_t)n_heads * n_buf * head_dim, 256);
  const int64_t qks = round_up((int64_t)n_heads * n_buf * (head_dim / 32), 256);
  const int64_t vt = round_up((int64_t)n_heads * head_dim * cols, 256);
  const int64_t vts = round_up((int64_t)n_heads * (cols / 32) * head_dim, 256);
  return (size_t)(2 * qk + 2 * qks + vt + vts);
}

template <int D>
static hipError_t launch_attn_fp8_d(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                                    const void* v, int64_t ld_v, void* o, int64_t ld_o,
                                    int64_t n_buf, int n_heads, const int* cu, const int* valid,
                                    int n_seg, int max_len, float scale, float skip_log2,
                                    void* ws, hipStream_t s) {
  if (n_buf == 0) return hipSuccess;
  const unsigned zblocks = (unsigned)ceil_div(n_buf, 4);
  hipLaunchKernelGGL((zero_pad_rows_kernel<bf16_t>), dim3(zblocks), dim3(256), 0, s,
                     (bf16_t*)o, ld_o, n_buf, n_heads * D, cu, valid, n_seg);
  if (max_len == 0) return hipGetLastError();
  const int64_t cols = vt_columns(n_buf, n_seg);
  uint8_t* w = (uint8_t*)ws;
  const int64_t qk = round_up((int64_t)n_heads * n_buf * D, 256);
  const int64_t qks = round_up((int64_t)n_heads * n_buf * (D / 32), 256);
  const int64_t vt = round_up((int64_t)n_heads * D * cols, 256);
  uint8_t *q8 = w, *k8 = w + qk, *qs = w + 2 * qk, *ks = w + 2 * qk + qks;
  uint8_t *vt8 = w + 2 * qk + 2 * qks, *vts = vt8 + vt;
  const int64_t nq = (int64_t)n_heads * n_buf * (D / 32);
  const unsigned qblocks = (unsigned)ceil_div(nq, 256);
  hipLaunchKernelGGL((quant_rows_e4m3_kernel<D>), dim3(qblocks), dim3(256), 0, s, (const bf16_t*)q,
                     ld_q, n_buf, n_heads, cu, valid, n_seg, scale * 1.4426950408889634f, q8, qs);
  hipLaunchKernelGGL((quant_rows_e4m3_kernel<D>), dim3(qblocks), dim3(256), 0, s, (const bf16_t*)k,
                     ld_k, n_buf, n_heads, cu, valid, n_seg, 1.0f, k8, ks);
  hipLaunchKernelGGL((transpose_quant_v_kernel<D>), dim3((unsigned)ceil_div(max_len, 64), n_seg, n_heads),
                     dim3(256), 0, s, (const bf16_t*)v, ld_v, vt8, vts, cols, cu, valid);
  constexpr int NW = 8;
  const dim3 grid((unsigned)ceil_div(max_len, NW * 32), n_seg, n_heads);
  if (skip_log2 < 0.f)
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, NW, true>), grid, dim3(NW * 64), 0, s, q8, qs, k8,
                       ks, n_buf, vt8, vts, cols, (bf16_t*)o, ld_o, cu, valid, skip_log2);
  else
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, NW>), grid, dim3(NW * 64), 0, s, q8, qs, k8, ks,
                       n_buf, vt8, vts, cols, (bf16_t*)o, ld_o, cu, valid, 0.f);
  return hipGetLastError();
}

hipError_t launch_varlen_attn_fp8(int head_dim, const void* q, int64_t ld_q, const void* k,
                                  int64_t ld_k, const void* v, int64_t ld_v, void* o,
                                  int64_t ld_o, int64_t n_buf, int n_heads, const int* cu,
                                  const int* valid, int n_seg, int max_len, float scale,
                                  float skip_log2, void* ws, hipStream_t s) {
  if (head_dim == 128)
    return launch_attn_fp8_d<128>(q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, cu, valid,
                                  n_seg, max_len, scale, skip_log2, ws, s);
  return launch_attn_fp8_d<64>(q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, cu, valid,
                               n_seg, max_len, scale, skip_log2, ws, s);
}

}  // namespace h3
