/*
 * h3dit -- one DiT block forward on a packed audio-video token sequence, for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Page titles cited (abbreviated):
 *   [RT-H3]  "Why Real-Time MiniMax H3 Serving Requires More Than a Faster DiT"
 *   [FH3-zh] "MiniMax H3 通过 vLLM-Omni 实现 FastH3 实时推理"
 *
 * The block: modulated norm -> QKV projection -> Q/K RMSNorm + RoPE ->
 * attention over each segment's valid rows -> output projection -> gated
 * residual -> modulated norm -> SwiGLU MLP -> gated residual.  The pages name
 * the packed sequence with valid lengths and no structural suffix padding,
 * rank-local RoPE rows, and the fused Q/K RMSNorm+RoPE, modulation/norm,
 * residual and SwiGLU operations ([RT-H3] Key takeaways; [FH3-zh]
 * vLLM-Omni 中的系统级优化).  Widths, norm kinds and layouts below are the
 * plain readings of pages that give no model code.
 *
 * Conventions for every entry point
 *  - Memory: every tensor argument is a DEVICE pointer unless marked "host".
 *    The caller allocates and owns all buffers and the stream; the library
 *    never allocates, frees or synchronises, and keeps no pointer after the
 *    call returns.  Scratch memory comes from the caller as `ws`/`ws_bytes`,
 *    sized by the matching *_workspace_size() query.
 *  - Layout: row-major.  `ld_*` arguments are row strides in ELEMENTS.  Every
 *    tensor pointer must be 16-byte aligned and every row stride times the
 *    element size a multiple of 16 bytes.
 *  - Types: storage is H3_F32 or H3_BF16 (all tensors of one call share it);
 *    accumulation is always fp32; outputs are rounded to nearest even.
 *    Position and offset tables are int32.
 *  - Streams: `stream` is a hipStream_t (NULL = the default stream).  All work
 *    is enqueued asynchronously on it, in order.
 *  - Errors: arguments are checked on the host before anything is enqueued; on
 *    any error nothing is launched and a status != H3_OK is returned, with a
 *    description in h3_last_error() (thread-local).  Faults inside kernels
 *    surface, as HIP reports them, at the caller's next synchronisation.
 *  - Determinism: no atomics and a fixed reduction order; identical inputs give
 *    byte-identical outputs run after run (the pages observe byte-identical
 *    output for a fixed seed, [FH3-zh] 质量与兼容性说明).
 */
#ifndef H3DIT_H
#define H3DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3_ABI_VERSION 7

typedef enum {
  H3_OK = 0,
  H3_ERR_ARG = 1,          /* bad pointer, size, stride, alignment or layout */
  H3_ERR_UNSUPPORTED = 2,  /* dtype, head_dim or device not supported (gfx950 only) */
  H3_ERR_WORKSPACE = 3,    /* ws_bytes below the size the query returns */
  H3_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} h3_status;

typedef enum { H3_F32 = 0, H3_BF16 = 1 } h3_dtype;

/* Token kinds of the position table. */
enum { H3_POS_VIDEO = 0, H3_POS_AUDIO = 1, H3_POS_PAD = 2 };

/* One token's RoPE position: video tokens use (t, h, w); audio tokens use t as
 * their audio index; pad tokens are left untouched by h3_qk_norm_rope. */
typedef struct {
  int32_t kind;
  int32_t t;
  int32_t h;
  int32_t w;
} h3_pos;

/* Library ABI version (H3_ABI_VERSION of the build). */
int h3_abi_version(void);
/* Static text for a status code. */
const char* h3_status_string(h3_status st);
/* Detail of the last error on the calling thread ("" if none). */
const char* h3_last_error(void);

/*
 * h3_qk_norm_rope -- in place, per (token, head): q <- RoPE(RMSNorm(q) * g_q),
 * k <- RoPE(RMSNorm(k) * g_k).  ([RT-H3] Key takeaways: fused Q/K RMSNorm
 * with RoPE; rank-local RoPE rows.)
 *   q, k      [n_tok rows] x [n_heads * head_dim], row strides ld_q, ld_k; heads
 *             contiguous at stride head_dim inside a row (e.g. the q and k
 *             thirds of a [n_tok, 3, H, D] QKV buffer, ld = 3*H*D).
 *   g_q, g_k  [head_dim] gains shared by all heads.
 *   pos       [n_tok] positions of exactly these rows (rank-local rows only).
 *   RMSNorm:  x / sqrt(mean(x^2) + eps) over one head's head_dim values.
 *   RoPE:     adjacent pairs (2j, 2j+1) turn by angle phi:
 *             (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi).
 *             Video: the head row is cut into sections [sec_t | sec_h | sec_w];
 *             pair j of a section of width d at position p turns by
 *             p * theta^(-2j/d).  Audio: one section of width head_dim at
 *             position t.  Pad rows: untouched (no norm either).
 *   Requires head_dim in {64, 128}; sec_* even, >= 0, summing to head_dim.
 *   n_tok == 0 is a no-op.
 */
h3_status h3_qk_norm_rope(void* q, int64_t ld_q, void* k, int64_t ld_k, int64_t n_tok,
                          int32_t n_heads, int32_t head_dim, const void* g_q, const void* g_k,
                          const h3_pos* pos, int32_t sec_t, int32_t sec_h, int32_t sec_w,
                          float theta, float eps, h3_dtype dtype, void* stream);

/*
 * h3_varlen_attn -- softmax attention over a packed buffer of segments, valid
 * rows only ([RT-H3] Key takeaways: valid sequence lengths, structural suffix
 * padding removed).
 *   q, k, v, o  [n_buf rows] x [n_heads * head_dim], row strides ld_*.
 *   cu_slots    device int32 [n_seg + 1]: segment s owns rows
 *               [cu_slots[s], cu_slots[s+1]), non-decreasing, 0 <= .. <= n_buf.
 *   valid_len   device int32 [n_seg]: the first valid_len[s] rows of slot s are
 *               valid (0 <= valid_len[s] <= slot length); NULL = whole slots.
 *   max_valid_len  host: an upper bound of max(valid_len) (sizes the grid).
 *   For each valid row i of segment s and each head:
 *     o_i = sum_j softmax_j(q_i . k_j * softmax_scale) v_j over valid rows j of s.
 *   Every other row of o (suffix pad, rows outside all slots) is written as 0.
 *   Pad rows of q, k, v are never read into the result (they may hold NaN/Inf).
 *   softmax_scale <= 0 means 1/sqrt(head_dim).  Bidirectional, no cross-segment
 *   attention.  head_dim in {64, 128}.
 *   ws: scratch of h3_varlen_attn_workspace_size(n_buf, n_heads, head_dim,
 *   n_seg, dtype) bytes (a transposed copy of v).  One head of that copy
 *   (head_dim rows of n_buf rounded up to 64 plus 128 (n_seg + 1) keys, 2 bytes
 *   each) must stay below 2^31 bytes, since the kernels address it with 32-bit
 *   offsets: larger calls return H3_ERR_ARG before any launch.
 */
size_t h3_varlen_attn_workspace_size(int64_t n_buf, int32_t n_heads, int32_t head_dim,
                                     int32_t n_seg, h3_dtype dtype);
h3_status h3_varlen_attn(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                         const void* v, int64_t ld_v, void* o, int64_t ld_o, int64_t n_buf,
                         int32_t n_heads, int32_t head_dim, const int32_t* cu_slots,
                         const int32_t* valid_len, int32_t n_seg, int32_t max_valid_len,
                         float softmax_scale, void* ws, size_t ws_bytes, h3_dtype dtype,
                         void* stream);

/*
 * h3_varlen_attn_noalloc -- h3_varlen_attn with no workspace argument and no
 * allocation, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, result and error behaviour as h3_varlen_attn, except:
 *   - the transposed copy of v lives in a device array inside the library,
 *     H3_NOALLOC_SCRATCH_BYTES (64 MiB) per device, held until the process
 *     ends; a call needing more (n_heads * head_dim * (round_up(n_buf, 64) +
 *     128 (n_seg + 1)) * 2 bytes for bf16; fp32 needs none) returns
 *     H3_ERR_WORKSPACE and launches nothing;
 *   - every call on one device shares that array (one per device in each
 *     process): calls of one process that overlap in time on one device (on
 *     different streams, or from different threads) race and give undefined
 *     results; calls in stream order are safe, since each call writes every
 *     scratch byte it reads before reading it;
 *   - it never calls hipMalloc, hipFree or another allocating routine; the
 *     first call on a device looks up the array's device address
 *     (hipGetSymbolAddress) once;
 *   - it does not run the H3_DEBUG_VALIDATE check (that check copies to the
 *     host and synchronises).
 */
#define H3_NOALLOC_SCRATCH_BYTES (64ull << 20)
h3_status h3_varlen_attn_noalloc(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                                 const void* v, int64_t ld_v, void* o, int64_t ld_o,
                                 int64_t n_buf, int32_t n_heads, int32_t head_dim,
                                 const int32_t* cu_slots, const int32_t* valid_len,
                                 int32_t n_seg, int32_t max_valid_len, float softmax_scale,
                                 h3_dtype dtype, void* stream);

/*
 * h3_varlen_attn_skip -- h3_varlen_attn with Skip-Softmax (MiniMax H3 通过
 * vLLM-Omni 实现 FastH3 实时推理, "超出 FastH3 配置的扩展能力": Skip-Softmax is
 * named among the attention variants that speed up the base pipeline).
 * Keys are visited in blocks of 64 from each segment's start, queries in
 * groups of 32 consecutive valid rows; a block is skipped for a group (its
 * probabilities are exactly zero and its P.V products are not computed) when, for
 * every valid row of the group, the block's largest score q.k * scale *
 * log2(e) is below the row's running maximum over the blocks before it plus
 * skip_log2.  The first block is never skipped.  A skipped key's weight is at
 * most 2^skip_log2 times its row's largest weight.  skip_log2 < 0 (-inf: no
 * block is skipped and the result equals h3_varlen_attn's bit for bit).
 * Arguments, layouts, workspace and errors as h3_varlen_attn; bf16 only
 * (H3_ERR_UNSUPPORTED otherwise).
 */
h3_status h3_varlen_attn_skip(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                              const void* v, int64_t ld_v, void* o, int64_t ld_o, int64_t n_buf,
                              int32_t n_heads, int32_t head_dim, const int32_t* cu_slots,
                              const int32_t* valid_len, int32_t n_seg, int32_t max_valid_len,
                              float softmax_scale, float skip_log2, void* ws, size_t ws_bytes,
                              h3_dtype dtype, void* stream);

/*
 * h3_varlen_attn_fp8 -- the same attention with FP8 operands (MiniMax H3 通过
 * vLLM-Omni 实现 FastH3 实时推理, "超出 FastH3 配置的扩展能力": an FP8 attention path
 * (SAGE FP8) speeds up the base pipeline at small quality cost).  Same
 * arguments and output contract as h3_varlen_attn (bf16 q, k, v, o), except:
 *   q (times softmax_scale * log2 e), k and v are rounded to OCP e4m3 with
 *   one power-of-two scale per 32 elements along the contraction (head dim
 *   for q and k, keys of each segment slot for v), and the softmax weights
 *   are rounded to e4m3 (as 256 * p with scale 2^-8) before P.V.  Accumulation
 *   is fp32.  The result approximates exact attention; it is not
 *   bit-compatible with h3_varlen_attn.
 *   ws: h3_varlen_attn_fp8_workspace_size(...) bytes (quantized operands).
 *   Errors as h3_varlen_attn; H3_ERR_UNSUPPORTED unless dtype is H3_BF16.
 */
size_t h3_varlen_attn_fp8_workspace_size(int64_t n_buf, int32_t n_heads, int32_t head_dim,
                                         int32_t n_seg);
h3_status h3_varlen_attn_fp8(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                             const void* v, int64_t ld_v, void* o, int64_t ld_o, int64_t n_buf,
                             int32_t n_heads, int32_t head_dim, const int32_t* cu_slots,
                             const int32_t* valid_len, int32_t n_seg, int32_t max_valid_len,
                             float softmax_scale, void* ws, size_t ws_bytes, h3_dtype dtype,
                             void* stream);

/*
 * h3_varlen_attn_fp8_skip -- h3_varlen_attn_fp8 with the Skip-Softmax rule of
 * h3_varlen_attn_skip (same page and section: SAGE FP8 and Skip-Softmax are
 * named together).  The rule is applied to the scores of the quantized
 * operands (log2 units: q already carries softmax_scale * log2 e).
 * skip_log2 < 0 (H3_ERR_ARG otherwise, NaN included); -inf skips nothing and
 * gives h3_varlen_attn_fp8's result.  Arguments, workspace and errors as
 * h3_varlen_attn_fp8.
 */
h3_status h3_varlen_attn_fp8_skip(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                                  const void* v, int64_t ld_v, void* o, int64_t ld_o,
                                  int64_t n_buf, int32_t n_heads, int32_t head_dim,
                                  const int32_t* cu_slots, const int32_t* valid_len,
                                  int32_t n_seg, int32_t max_valid_len, float softmax_scale,
                                  float skip_log2, void* ws, size_t ws_bytes, h3_dtype dtype,
                                  void* stream);

/*
 * h3_modulate_residual -- one pass over rows of width dim:
 *   if y != NULL:     x <- x + gate * y                       (gated residual)
 *   if h_out != NULL: h_out <- norm(x) * (1 + scale) + shift  (modulated norm)
 * ([RT-H3] Key takeaways: modulation, normalisation and residual updates fused.)
 *   x       [n_tok, dim] in/out, stride ld_x.   y [n_tok, dim], stride ld_y.
 *   gate, shift, scale  rows of stride ld_mod; ld_mod == 0 broadcasts row 0 to
 *           every token.  gate is required iff y != NULL; shift and scale iff
 *           h_out != NULL.
 *   norm_kind 0: LayerNorm without affine, biased variance, eps inside the
 *           square root; 1: RMSNorm.
 *   The norm sees the updated x in fp32 (before its rounding to storage).
 *   dim must be a multiple of 8 and at most 16384.
 */
h3_status h3_modulate_residual(void* x, int64_t ld_x, const void* y, int64_t ld_y,
                               const void* gate, const void* shift, const void* scale,
                               int64_t ld_mod, void* h_out, int64_t ld_h, int64_t n_tok,
                               int32_t dim, int32_t norm_kind, float eps, h3_dtype dtype,
                               void* stream);

/*
 * h3_linear -- out = a @ w^T (w stored [n_out, k_in], no bias); if gate != NULL
 * the result is instead added as a gated residual: out <- out + gate * (a @ w^T).
 * The QKV and output projections of the block.
 *   a [m, k_in] stride lda; w [n_out, k_in] stride ldw; out [m, n_out] stride
 *   ld_out; gate rows of stride ld_gate (0 = broadcast).  k_in % 8 == 0.
 */
h3_status h3_linear(const void* a, int64_t lda, const void* w, int64_t ldw, void* out,
                    int64_t ld_out, int64_t m, int32_t n_out, int32_t k_in, const void* gate,
                    int64_t ld_gate, h3_dtype dtype, void* stream);

/*
 * h3_swiglu -- SwiGLU MLP ([RT-H3] Key takeaways: SwiGLU fused):
 *   g = silu(h @ w1^T) * (h @ w3^T)    (silu(a) = a / (1 + e^-a); one GEMM
 *                                        pass with the gate in its epilogue)
 *   y = g @ w2^T
 *   gate == NULL: out <- y;  else out <- out + gate * y (gated residual, in place).
 *   h [n_tok, dim] stride ld_h; w1, w3 [ffn_dim, dim]; w2 [dim, ffn_dim];
 *   out [n_tok, dim] stride ld_out; gate rows of stride ld_gate (0 = broadcast).
 *   ws: h3_swiglu_workspace_size(n_tok, ffn_dim, dtype) bytes (holds g).
 *   dim % 8 == 0, ffn_dim % 8 == 0.
 */
size_t h3_swiglu_workspace_size(int64_t n_tok, int32_t ffn_dim, h3_dtype dtype);
h3_status h3_swiglu(const void* h, int64_t ld_h, const void* w1, const void* w3,
                    const void* w2, void* out, int64_t ld_out, const void* gate,
                    int64_t ld_gate, int64_t n_tok, int32_t dim, int32_t ffn_dim, void* ws,
                    size_t ws_bytes, h3_dtype dtype, void* stream);

/* ------------------------------------------- FP8 (MX e4m3) projections */

/*
 * Online FP8 projections (MiniMax H3 通过 vLLM-Omni 实现 FastH3 实时推理,
 * "超出 FastH3 配置的扩展能力": an online FP8 quantization path lowers the
 * peak HBM footprint and the latency).  Both operands of a projection are MX
 * operands: OCP e4m3 values with one power-of-two (E8M0) scale per 32
 * consecutive elements along the contraction, the smallest scale 2^e with
 * block amax <= 448 * 2^e, elements rounded to nearest (ties to even).
 * Weights are quantized once; activations on the fly, from bf16.
 *
 * h3_mx_operand -- k logical columns stored as:
 *   data:  e4m3 bytes [rows][ld]; 16-byte aligned; ld a multiple of 16 with
 *          round_up(k, 128) <= ld <= 2^23; columns [k, round_up(k, 128)) are zero.
 *   scale: E8M0 bytes [rows][ld_scale]; 4-byte aligned; ld_scale a multiple of 4,
 *          >= round_up(k, 128) / 32; byte b scales columns [32 b, 32 b + 32)
 *          (value = e4m3 * 2^(byte - 127)).
 * The caller owns both buffers.
 */
typedef struct {
  const void* data;
  int64_t ld;
  const void* scale;
  int64_t ld_scale;
} h3_mx_operand;

/*
 * h3_mx_quantize -- bf16 x [rows][cols] (row stride ld_x elements, cols % 32 == 0)
 * -> MX operand (q, ld_q, scale, ld_scale) as above, including the zero
 * columns up to round_up(cols, 128) (their scale byte is 127).
 * Errors: H3_ERR_UNSUPPORTED unless dtype is H3_BF16; H3_ERR_ARG for shapes,
 * strides or alignment.
 */
h3_status h3_mx_quantize(const void* x, int64_t ld_x, int64_t rows, int32_t cols, void* q,
                         int64_t ld_q, void* scale, int64_t ld_scale, h3_dtype dtype,
                         void* stream);

/*
 * h3_modulate_mx -- the modulated norm of h3_modulate_residual (no residual),
 * written as an MX operand instead of bf16 h ([RT-H3] Key takeaways:
 * modulation and normalisation fused; [FH3-zh] 超出 FastH3 配置的扩展能力:
 * online FP8 GEMMs): q, q_scale receive exactly the bytes that
 * h3_modulate_residual(h_out = h) followed by h3_mx_quantize(h) would give.
 *   x [n_tok][dim] bf16 (read only), shift/scale rows of stride ld_mod (0:
 *   broadcast), norm_kind and eps as in h3_modulate_residual.
 *   (q, ld_q, q_scale, ld_scale): MX operand of dim columns, as above.
 *   dim % 128 == 0 (no zero padding columns), dim <= 16384; bf16 only.
 * Errors: H3_ERR_ARG for shapes, strides or alignment.
 */
h3_status h3_modulate_mx(const void* x, int64_t ld_x, const void* shift, const void* scale,
                         int64_t ld_mod, void* q, int64_t ld_q, void* q_scale, int64_t ld_scale,
                         int64_t n_tok, int32_t dim, int32_t norm_kind, float eps, void* stream);

/*
 * h3_linear_fp8 -- out = a w^T over MX operands a [m][k_in] and w [n_out][k_in]
 * (k_in % 32 == 0), fp32 accumulation, bf16 out [m][n_out] (row stride ld_out).
 * gate != NULL: out = out + gate * (a w^T) in place (gate bf16 [m][n_out]).
 */
h3_status h3_linear_fp8(const h3_mx_operand* a, const h3_mx_operand* w, void* out,
                        int64_t ld_out, int64_t m, int32_t n_out, int32_t k_in,
                        const void* gate, int64_t ld_gate, void* stream);

/*
 * h3_swiglu_fp8 -- the SwiGLU MLP of h3_swiglu over MX operands: h [n_tok][dim],
 * w1, w3 [ffn_dim][dim] (same ld and ld_scale), w2 [dim][ffn_dim]; the gate
 * product g = silu(h w1^T) * (h w3^T) is rounded to bf16 and quantized on the
 * fly into the workspace before the down-projection.  out / gate as in
 * h3_linear_fp8.  dim % 32 == 0, ffn_dim % 32 == 0.
 *   ws: h3_swiglu_fp8_workspace_size(n_tok, ffn_dim) bytes, 16-byte aligned; on
 *   return it starts with g (bf16 [n_tok][ffn_dim]), followed by g's MX operand.
 */
size_t h3_swiglu_fp8_workspace_size(int64_t n_tok, int32_t ffn_dim);
h3_status h3_swiglu_fp8(const h3_mx_operand* h, const h3_mx_operand* w1,
                        const h3_mx_operand* w3, const h3_mx_operand* w2, void* out,
                        int64_t ld_out, const void* gate, int64_t ld_gate, int64_t n_tok,
                        int32_t dim, int32_t ffn_dim, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ whole block */

typedef struct {
  int32_t dim;        /* C, a multiple of 8, at most 16384 */
  int32_t n_heads;    /* H; H * D at most 2^22 */
  int32_t head_dim;   /* D, 64 or 128 */
  int32_t ffn_dim;    /* F, a multiple of 8, at most 2^22 */
  int32_t sec_t, sec_h, sec_w;  /* RoPE sections of a head row (video) */
  float theta;        /* RoPE base */
  float eps_qk;       /* Q/K RMSNorm epsilon */
  float eps_mod;      /* modulated-norm epsilon */
  int32_t norm_kind;  /* 0 LayerNorm, 1 RMSNorm (modulated norms) */
  h3_dtype dtype;
  int32_t attn_fp8;   /* 1: attention through h3_varlen_attn_fp8 (bf16 only); 0: exact path */
  int32_t gemm_fp8;   /* 1: the four projections on MX operands (bf16 only, weights.mx); 0: bf16 */
  float attn_skip_log2; /* < 0: attention with the Skip-Softmax rule at this threshold t
                           (h3_varlen_attn_skip, or h3_varlen_attn_fp8_skip with attn_fp8;
                           bf16 only; -inf never skips); 0: without it */
} h3_block_config;

typedef struct {
  const void* w_qkv;  /* [3*H*D, C]: rows q heads 0..H-1, then k heads, then v heads */
  const void* w_o;    /* [C, H*D] */
  const void* w1;     /* [F, C] (silu branch) */
  const void* w3;     /* [F, C] (linear branch) */
  const void* w2;     /* [C, F] */
  const void* g_q;    /* [D] */
  const void* g_k;    /* [D] */
  const h3_mx_operand* mx;  /* gemm_fp8: [5] MX copies of w_qkv, w_o, w1, w3, w2
                               (w1 and w3 with the same ld and ld_scale); else NULL */
} h3_block_weights;

typedef struct {
  void* x;              /* [n_tok_local, C] residual stream, updated in place */
  int64_t ld_x;
  const void* mod;      /* [rows, 6, C]: shift1, scale1, gate1, shift2, scale2, gate2 */
  int64_t ld_mod;       /* elements between token rows (6*C), or 0 = one row for all */
  const h3_pos* pos;    /* [n_tok_local] positions of the local rows */
  const int32_t* cu_slots;   /* device [n_seg+1] over the attention buffer rows */
  const int32_t* valid_len;  /* device [n_seg] (NULL = whole slots) */
  int32_t n_seg;
  int32_t max_valid_len;     /* host bound of max(valid_len) */
  int64_t n_tok_local;  /* this GPU's token rows */
  int64_t n_buf;        /* attention buffer rows (world 1: n_tok_local) */
  int64_t tok_begin;    /* attention-buffer row of local token 0 (world 1: 0) */
  int32_t head_begin;   /* first head of this GPU's attention slice (world 1: 0) */
  int32_t head_count;   /* heads in the slice (world 1: H) */
  /* Rank-share mode only (all NULL in world 1).  The sequence-parallel
   * exchange around attention ([RT-H3] Key takeaways: all-to-all around
   * attention) is outside this library: the caller provides its buffers with
   * the other ranks' rows and heads already in place. */
  void* qkv_attn;       /* [n_buf, 3, head_count, D]; rows [tok_begin, +n_tok_local) are written */
  void* o_attn;         /* [n_buf, head_count, D]; written by attention */
  void* o_local;        /* [n_tok_local, H, D]; heads [head_begin, +head_count) are written */
  /* Peer-major exchange layout (rank-share mode, bf16; optional: both NULL
   * selects the qkv_attn/o_local form above).  Each all-to-all around
   * attention then moves one contiguous, equal block per peer and nothing is
   * rearranged before or after it ([RT-H3] Key takeaways: Fast Ulysses
   * avoids layout rearrangement around the all-to-all).  With P = n_heads /
   * head_count peers, this rank r = head_begin / head_count, and tok_begin ==
   * r * n_tok_local:
   *   qkv_send [P, n_tok_local, 3, head_count, D]: written by the QKV
   *     projection's epilogue; block p holds heads [p*hc, (p+1)*hc), the part
   *     peer p receives.  Block r is copied to qkv_attn rows [tok_begin, ...).
   *   o_recv [P, n_tok_local, head_count, D]: block p is peer p's attention
   *     output for the local rows (the reverse all-to-all delivers blocks
   *     p != r; the caller provides them).  Block r is copied from o_attn,
   *     and the output projection reads o_recv in place.  o_local is unused.
   * Needs dim % 64 == 0 and head_count*D % 64 == 0. */
  void* qkv_send;
  void* o_recv;
} h3_block_io;

/*
 * h3_dit_block_forward -- one block on one GPU, all steps enqueued on `stream`:
 *   h1 = norm(x)(1+scale1)+shift1;  qkv = h1 w_qkv^T;  Q/K RMSNorm+RoPE (local rows);
 *   attention over cu_slots/valid_len (world 1: reads qkv in place; rank share:
 *   the local head slice is copied into qkv_attn rows first, attention runs on
 *   qkv_attn and its local rows are copied into o_local);
 *   x <- x + gate1 * (o w_o^T);  h2 = norm(x)(1+scale2)+shift2;
 *   x <- x + gate2 * (silu(h2 w1^T) * (h2 w3^T)) w2^T.
 * World 1: qkv_attn == NULL, tok_begin == 0, n_buf == n_tok_local, head_count == H.
 * cfg->attn_fp8 == 1 runs the attention step as h3_varlen_attn_fp8 does (MX-scaled
 * e4m3 operands); it needs dtype H3_BF16 (else H3_ERR_ARG), and the workspace size
 * depends on it, so query it with the same cfg.
 * cfg->gemm_fp8 == 1 runs the four projections as h3_linear_fp8 / h3_swiglu_fp8 do:
 * each bf16 activation (h1, o, h2, g) is quantized to an MX operand in the workspace
 * just before its projection, the weights come from w->mx (the bf16 weight pointers
 * may then be NULL).  Needs dtype H3_BF16 and dim, ffn_dim, H*D multiples of 32.
 *
 * h3_dit_block_workspace_size: bytes of the workspace h3_dit_block_forward needs
 * for this cfg.  head_count > 0: a rank share with that head slice over an
 * n_buf-row attention buffer; 0: enough for world 1 and for a share of any head
 * count.  The workspace holds, by lifetime, h1 and the MX activation copy for
 * the whole block, then qkv, the attention workspace and o (world 1), whose
 * bytes the SwiGLU's g and its MX copy reuse.  Returns 0 for a NULL cfg or a
 * negative size.
 */
size_t h3_dit_block_workspace_size(const h3_block_config* cfg, int64_t n_tok_local,
                                   int64_t n_buf, int32_t n_seg, int32_t head_count);
h3_status h3_dit_block_forward(const h3_block_config* cfg, const h3_block_weights* w,
                               const h3_block_io* io, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------ student loop glue */

/*
 * h3_timestep_modulation -- per-block modulation at noise level sigma for the
 * four-forward student ([FH3-zh] FastH3：四步学生模型: four forwards over five
 * sigma positions).  The pages give no embedding; this is the common
 * sinusoidal one:
 *   e = [cos(1000 sigma w_j) || sin(1000 sigma w_j)], w_j = 10000^(-j/(E/2)), j < E/2
 *   t = w_t2 @ silu(w_t1 @ e)                  (w_t1 [C, E], w_t2 [6C, C])
 *   mod_out[b] = t (as [6, C]) + table[b]      (table, mod_out [n_blocks, 6, C])
 * emb_dim E even, <= 1024.  ws: h3_timestep_workspace_size(dim) bytes.
 */
size_t h3_timestep_workspace_size(int32_t dim);
h3_status h3_timestep_modulation(float sigma, const void* w_t1, const void* w_t2,
                                 const void* table, void* mod_out, int32_t n_blocks,
                                 int32_t dim, int32_t emb_dim, void* ws, size_t ws_bytes,
                                 h3_dtype dtype, void* stream);

/*
 * h3_euler_update -- z <- z + (sigma_to - sigma_from) * u over n elements, then,
 * if x_next != NULL, x_next <- z (the next forward's input).  u may alias x_next.
 */
h3_status h3_euler_update(void* z, const void* u, void* x_next, int64_t n, float sigma_from,
                          float sigma_to, h3_dtype dtype, void* stream);

/* ------------------------------------------------- output frames (post-DiT) */

/*
 * h3_frames_to_u8 -- decoded video frames to compact uint8 (Why Real-Time
 * MiniMax H3 Serving Requires More Than a Faster DiT, "Key takeaways":
 * decoded frames are converted on the GPU, once, into contiguous uint8 BTHWC
 * data; the H.264 encoder is fed through planar paths).
 *   frames: device fp32 [B][3][T][H][W] (the decoder's channel-first output,
 *           nominally in [-1, 1]); read only.
 *   out:    device uint8; layout 0 writes [B][T][H][W][3] (interleaved RGB),
 *           layout 1 writes [B][T][3][H][W] (one plane per channel and frame).
 *   Each value: v = x * 0.5 + 0.5 in fp32, clamped to [0, 1] (NaN -> 0), then
 *   u = v * 255 rounded half to even.
 *   Both pointers 16-byte aligned and not overlapping; B, T, H, W >= 0.  A
 *   width that is a multiple of 16 takes the vectorised path.
 *   Errors: H3_ERR_ARG on a bad pointer, size or layout (nothing launched).
 */
h3_status h3_frames_to_u8(const void* frames, int64_t B, int64_t T, int64_t H, int64_t W,
                          void* out, int32_t layout, void* stream);

/* --------------------------------------------- segment metadata check */

/*
 * h3_check_segments -- checks segment metadata held in HOST memory against the
 * rules the attention entry points assume ([RT-H3] Key takeaways: attention
 * runs over each segment's valid length, suffix padding removed):
 *   0 <= cu_slots[0] <= cu_slots[1] <= ... <= cu_slots[n_seg] <= n_buf, and
 *   for each segment s: 0 <= valid_len[s] <= cu_slots[s+1] - cu_slots[s] (the
 *   slot length itself when valid_len is NULL) and valid_len[s] <= max_valid_len.
 *   cu_slots [n_seg + 1], valid_len [n_seg] or NULL: host arrays, read only.
 * The attention entry points and h3_dit_block_forward run the same check on
 * their device copies when the environment variable H3_DEBUG_VALIDATE is "1"
 * (a device-to-host copy that synchronises the stream, before any launch);
 * otherwise they trust the device metadata.
 * Errors: H3_ERR_ARG with the first violated rule in h3_last_error().
 */
h3_status h3_check_segments(const int32_t* cu_slots, const int32_t* valid_len, int32_t n_seg,
                            int64_t n_buf, int32_t max_valid_len);

#ifdef __cplusplus
}
#endif

#endif /* H3DIT_H */
