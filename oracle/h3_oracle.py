"""Float64 CPU oracle of one DiT block forward on a packed audio-video sequence.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the product path.

Page titles cited below (abbreviated):
  [RT-H3]  "Why Real-Time MiniMax H3 Serving Requires More Than a Faster DiT"
  [OMNI]   "vLLM-Omni pushes MiniMax H3 video generation below playback time"
  [FH3-zh] "MiniMax H3 通过 vLLM-Omni 实现 FastH3 实时推理"

What the pages fix: attention over the packed audio-video sequence runs on each
segment's valid length with structural suffix padding removed, and each rank
touches only its own embedding/RoPE rows ([RT-H3] Key takeaways; [FH3-zh]
vLLM-Omni 中的系统级优化); the block's Q/K RMSNorm with RoPE, modulation with
normalisation, residual updates and SwiGLU are the operations that get fused
(same sections); the DiT is a joint audio-video transformer ([OMNI] Who it
affects); the student runs four forwards over five sigma positions ([FH3-zh]
FastH3：四步学生模型).  Everything else -- norm kinds, epsilons, RoPE pair
convention and section split, modulation slot order, absence of biases, the
timestep embedding -- is a reading of silent pages (one plain choice each,
named at each function).  Every step is computed in float64 on the values it is
given; there is no blocking, fusion or intermediate rounding.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

POS_VIDEO, POS_AUDIO, POS_PAD = 0, 1, 2

# modulation slots along axis 1 of the [rows, 6, C] modulation tensor
SHIFT1, SCALE1, GATE1, SHIFT2, SCALE2, GATE2 = range(6)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ------------------------------------------------------------------ O1 modnorm

def modulated_norm(x, shift, scale, eps: float = 1e-6, kind: str = "layer") -> np.ndarray:
    """adaLN-style modulated normalisation of each row of x.

    kind="layer": n = (x - mean) / sqrt(var + eps), var the biased variance,
    no affine of its own; kind="rms": n = x / sqrt(mean(x^2) + eps).
    Returns n * (1 + scale) + shift.  The pages name modulation and
    normalisation as one fused piece of work ([RT-H3] Key takeaways); the norm
    kind and the (1 + scale) form are the plain adaLN reading.
    """
    x = _f64(x)
    if kind == "layer":
        mu = x.mean(axis=-1, keepdims=True)
        var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
        n = (x - mu) / np.sqrt(var + eps)
    elif kind == "rms":
        n = x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    else:
        raise ValueError(kind)
    return n * (1.0 + _f64(scale)) + _f64(shift)


def gated_residual(x, gate, y) -> np.ndarray:
    """x + gate * y: the gated residual update named among the fused operations
    ([RT-H3] Key takeaways)."""
    return _f64(x) + _f64(gate) * _f64(y)


# --------------------------------------------------------------- O2 projections

def linear(x, w) -> np.ndarray:
    """x @ w^T with w stored [out, in] and no bias."""
    return _f64(x) @ _f64(w).T


# ---------------------------------------------------------- O3 Q/K RMSNorm

def rms_norm_heads(t, gain, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis (one head's D values), times a gain [D] shared
    by all heads ([RT-H3] Key takeaways: Q/K RMSNorm)."""
    t = _f64(t)
    return t / np.sqrt((t * t).mean(axis=-1, keepdims=True) + eps) * _f64(gain)


# ------------------------------------------------------------------ O4 RoPE

def rope_angles(pos, head_dim: int, sections: Sequence[int], theta: float) -> np.ndarray:
    """Rotation angle of every adjacent pair (2j, 2j+1) of a head row, per token.

    Video tokens (kind 0): the head row is cut into contiguous sections of
    widths (d_t, d_h, d_w); in a section of width d at position p, pair j
    (j < d/2) turns by p * theta**(-2j/d).  Audio tokens (kind 1): one section
    of width D at the audio index.  Pad tokens (kind 2): angle 0.
    Returns float64 [n, D/2].  ([RT-H3] Key takeaways: RoPE rows.)
    """
    pos = np.asarray(pos)
    n = pos.shape[0]
    half = head_dim // 2
    ang = np.zeros((n, half), dtype=np.float64)
    kind = pos[:, 0]
    vid = kind == POS_VIDEO
    aud = kind == POS_AUDIO
    pair = 0
    for axis, d in enumerate(sections):
        j = np.arange(d // 2, dtype=np.float64)
        freq = theta ** (-2.0 * j / d)
        p = pos[:, 1 + axis].astype(np.float64)
        ang[vid, pair:pair + d // 2] = p[vid, None] * freq[None, :]
        pair += d // 2
    j = np.arange(half, dtype=np.float64)
    freq = theta ** (-2.0 * j / head_dim)
    ang[aud, :] = pos[aud, 1].astype(np.float64)[:, None] * freq[None, :]
    return ang


def apply_rope(t, ang) -> np.ndarray:
    """Rotate each adjacent pair (a, b) of t[n, H, D] by ang[n, D/2]:
    (a, b) -> (a cos - b sin, a sin + b cos)."""
    t = _f64(t)
    a = t[..., 0::2]
    b = t[..., 1::2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    out = np.empty_like(t)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def qk_norm_rope(q, k, pos, g_q, g_k, sections, theta: float = 10000.0, eps: float = 1e-6):
    """Q/K RMSNorm per head followed by RoPE, on q, k [n, H, D].

    Pad rows (kind 2) are returned unchanged.  ([RT-H3] Key takeaways: Q/K
    RMSNorm with RoPE fused; rank-local RoPE rows.)
    """
    q = _f64(q)
    k = _f64(k)
    pos = np.asarray(pos)
    d = q.shape[-1]
    ang = rope_angles(pos, d, sections, theta)
    live = pos[:, 0] != POS_PAD
    qo = q.copy()
    ko = k.copy()
    qo[live] = apply_rope(rms_norm_heads(q[live], g_q, eps), ang[live])
    ko[live] = apply_rope(rms_norm_heads(k[live], g_k, eps), ang[live])
    return qo, ko


# ------------------------------------------------------------- O5 attention

def attention_dense(q, k, v, scale: float) -> np.ndarray:
    """softmax(q k^T * scale) v for one segment and head; q [m, D], k, v [n, D].

    Written with the row maximum subtracted before exponentiation.
    """
    s = _f64(q) @ _f64(k).T * scale
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ _f64(v)


def varlen_attention(q, k, v, cu_slots, valid_len, scale: Optional[float] = None,
                     q_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Attention over a packed buffer of segments, valid rows only.

    Segment s owns slot rows [cu_slots[s], cu_slots[s+1]); its first
    valid_len[s] rows are valid.  A valid row attends, bidirectionally, to the
    valid rows of its own segment only; every other row's output is 0.
    ([RT-H3] Key takeaways: valid sequence lengths, structural suffix padding
    removed.)  q, k, v are [n_buf, H, D]; scale defaults to 1/sqrt(D).

    q_rows: if given, q holds only those buffer rows (in that order) and the
    result has q's shape; keys and values are always the whole buffer.
    """
    k = np.asarray(k)
    v = np.asarray(v)
    n_buf, h, d = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(n_buf) if q_rows is None else np.asarray(q_rows)
    q = np.asarray(q)
    out = np.zeros((len(rows), h, d), dtype=np.float64)
    cu = np.asarray(cu_slots)
    vl = np.asarray(valid_len) if valid_len is not None else np.diff(cu)
    for s in range(len(cu) - 1):
        lo = int(cu[s])
        hi = lo + int(vl[s])
        if hi <= lo:
            continue
        sel = np.nonzero((rows >= lo) & (rows < hi))[0]
        if sel.size == 0:
            continue
        for head in range(h):
            out[sel, head] = attention_dense(q[sel, head], k[lo:hi, head], v[lo:hi, head], scale)
    return out


# ---------------------------------------------------------------- O8 SwiGLU

def silu(a) -> np.ndarray:
    a = _f64(a)
    return a / (1.0 + np.exp(-a))


def swiglu_gate(a, b) -> np.ndarray:
    """silu(a) * b, a from the W1 branch, b from the W3 branch."""
    return silu(a) * _f64(b)


def swiglu_mlp(h, w1, w3, w2) -> np.ndarray:
    """(silu(h W1^T) * (h W3^T)) W2^T ([RT-H3] Key takeaways: SwiGLU)."""
    return linear(swiglu_gate(linear(h, w1), linear(h, w3)), w2)


# ----------------------------------------------------------- whole block

@dataclasses.dataclass
class BlockShape:
    dim: int
    n_heads: int
    head_dim: int
    ffn_dim: int
    sections: tuple
    theta: float = 10000.0
    eps_qk: float = 1e-6
    eps_mod: float = 1e-6
    norm_kind: str = "layer"
    # rank-share description (world 1: tok_begin 0, head_begin 0, head_count = n_heads)
    tok_begin: int = 0
    head_begin: int = 0
    head_count: Optional[int] = None

    @staticmethod
    def of(wl) -> "BlockShape":
        return BlockShape(dim=wl.dim, n_heads=wl.n_heads, head_dim=wl.head_dim, ffn_dim=wl.ffn_dim,
                          sections=tuple(wl.sections), theta=wl.theta, eps_qk=wl.eps_qk,
                          eps_mod=wl.eps_mod, tok_begin=wl.tok_begin if wl.share_mode else 0,
                          head_begin=wl.head_begin if wl.share_mode else 0,
                          head_count=wl.head_count if wl.share_mode else wl.n_heads)


def _mod_rows(mod, rows):
    mod = np.asarray(mod)
    if mod.shape[0] == 1:
        return _f64(mod[0])[None]            # broadcast [1, 6, C]
    return _f64(mod[rows])


def dit_block(x, mod, w, pos, cu_slots, valid_len, shape: BlockShape,
              qkv_attn_fill=None, o_local_fill=None, rows: Optional[np.ndarray] = None,
              intermediates: bool = False, attention=None, projection=None):
    """One DiT block forward on this GPU's token rows x [n, C].

    Steps: h1 = modnorm(x; shift1, scale1) -> qkv = h1 Wqkv^T -> Q/K RMSNorm +
    RoPE -> varlen attention -> y1 = o Wo^T -> x1 = x + gate1 * y1 ->
    h2 = modnorm(x1; shift2, scale2) -> x2 = x1 + gate2 * SwiGLU(h2).

    World 1 (qkv_attn_fill is None): attention runs over the n local rows with
    all heads, segments given by cu_slots/valid_len over those rows.
    Rank share: the attention buffer is qkv_attn_fill [N, 3, hc, D] (rows of
    other ranks, as the sequence-parallel exchange would deliver them) with
    rows [tok_begin, tok_begin + n) replaced by this rank's own q, k, v of heads
    [head_begin, head_begin + hc); the attention output for those rows fills
    heads [head_begin, head_begin + hc) of o_local_fill [n, H, D], whose other
    heads stand for what the reverse exchange would deliver.
    ([RT-H3] Key takeaways: rank-local rows, all-to-all around attention;
    [FH3-zh] FastH3 推理配置: sequence-parallel degree 8.)

    rows: return only these local rows (keys/values still use every row).
    attention: the attention step, called as varlen_attention is (default);
    varlen_attention_fp8_operands gives the block with MX-e4m3 attention.
    projection: the four projections, called as linear is (default);
    linear_fp8_operands gives the block with MX-e4m3 projections.
    Returns x2 [len(rows), C], or a dict of every intermediate if asked.
    """
    sh = shape
    proj = linear if projection is None else projection
    x = np.asarray(x)
    n = x.shape[0]
    H, D, C = sh.n_heads, sh.head_dim, sh.dim
    hc = sh.head_count or H
    hb, tb = sh.head_begin, sh.tok_begin
    out_rows = np.arange(n) if rows is None else np.asarray(rows)

    # keys and values need every local row; queries and everything after need only out_rows
    all_rows = np.arange(n)
    mod_all = _mod_rows(mod, all_rows)
    h1 = modulated_norm(x, mod_all[:, SHIFT1], mod_all[:, SCALE1], sh.eps_mod, sh.norm_kind)
    wq = _f64(w.w_qkv).reshape(3, H, D, C)
    share = qkv_attn_fill is not None
    heads = slice(hb, hb + hc) if share else slice(0, H)
    wk = wq[1, heads].reshape(-1, C)
    wv = wq[2, heads].reshape(-1, C)
    k_loc = proj(h1, wk).reshape(n, -1, D)
    v_loc = proj(h1, wv).reshape(n, -1, D)
    h1r = h1[out_rows]
    q_loc = proj(h1r, wq[0, heads].reshape(-1, C)).reshape(len(out_rows), -1, D)
    pos = np.asarray(pos)
    # norm + RoPE on the local rows (q only on out_rows)
    kq_dummy = np.zeros_like(k_loc)
    _, k_loc = qk_norm_rope(kq_dummy, k_loc, pos, w.g_q, w.g_k, sh.sections, sh.theta, sh.eps_qk)
    q_loc, _ = qk_norm_rope(q_loc, np.zeros_like(q_loc), pos[out_rows], w.g_q, w.g_k,
                            sh.sections, sh.theta, sh.eps_qk)
    if share:
        buf = _f64(qkv_attn_fill).copy()
        buf[tb:tb + n, 1] = k_loc
        buf[tb:tb + n, 2] = v_loc
        kbuf, vbuf = buf[:, 1], buf[:, 2]
        qrows = out_rows + tb
    else:
        kbuf, vbuf = k_loc, v_loc
        qrows = out_rows
    attend = varlen_attention if attention is None else attention
    o_h = attend(q_loc, kbuf, vbuf, cu_slots, valid_len, q_rows=qrows)
    if share:
        o = _f64(o_local_fill)[out_rows].copy()
        o[:, hb:hb + hc] = o_h
    else:
        o = o_h
    y1 = proj(o.reshape(len(out_rows), H * D), w.w_o)
    mod_r = _mod_rows(mod, out_rows)
    xr = _f64(x[out_rows])
    x1 = gated_residual(xr, mod_r[:, GATE1], y1)
    h2 = modulated_norm(x1, mod_r[:, SHIFT2], mod_r[:, SCALE2], sh.eps_mod, sh.norm_kind)
    a = proj(h2, w.w1)
    b = proj(h2, w.w3)
    g = swiglu_gate(a, b)
    y2 = proj(g, w.w2)
    x2 = gated_residual(x1, mod_r[:, GATE2], y2)
    if not intermediates:
        return x2
    return dict(h1=h1r, q=q_loc, k=k_loc[out_rows], v=v_loc[out_rows], o=o.reshape(len(out_rows), H, D),
                o_heads=o_h, y1=y1, x1=x1, h2=h2, g=g, y2=y2, x2=x2)


# -------------------------------------------------- O9 four-forward student loop

def timestep_embedding(sigma: float, dim: int = 256, max_period: float = 10000.0,
                       sigma_scale: float = 1000.0) -> np.ndarray:
    """Sinusoidal embedding [cos(s w_j) || sin(s w_j)], s = 1000 sigma,
    w_j = max_period**(-j/(dim/2)), j < dim/2.  The pages give none; this is
    the common diffusion-transformer form."""
    half = dim // 2
    j = np.arange(half, dtype=np.float64)
    om = max_period ** (-j / half)
    a = sigma_scale * float(sigma) * om
    return np.concatenate([np.cos(a), np.sin(a)])


def timestep_modulation(sigma: float, tw) -> np.ndarray:
    """Per-block modulation [n_blocks, 6, C] at noise level sigma:
    W_t2 silu(W_t1 e(sigma)) reshaped [6, C], plus each block's table."""
    e = timestep_embedding(sigma, _f64(tw.w_t1).shape[1])
    hid = silu(_f64(tw.w_t1) @ e)
    tvec = (_f64(tw.w_t2) @ hid).reshape(6, -1)
    return tvec[None] + _f64(tw.table)


def euler_update(z, u, sigma_from: float, sigma_to: float) -> np.ndarray:
    """z + (sigma_to - sigma_from) * u."""
    return _f64(z) + (float(sigma_to) - float(sigma_from)) * _f64(u)


def student_loop(z, blocks_w, tw, pos, cu_slots, valid_len, shape: BlockShape, sigmas,
                 qkv_attn_fill=None, o_local_fill=None):
    """Four forwards over five sigma positions ([FH3-zh] FastH3：四步学生模型).

    For k = 0..len(sigmas)-2: every block b takes its modulation from
    timestep_modulation(sigma_k)[b] (broadcast over rows); u is the stack's
    output on z; then z <- z + (sigma_{k+1} - sigma_k) u.  In rank-share mode
    every block sees the same fill buffers for the other ranks' rows.
    """
    z = _f64(z)
    for k in range(len(sigmas) - 1):
        mods = timestep_modulation(sigmas[k], tw)
        u = z
        for b, w in enumerate(blocks_w):
            u = dit_block(u, mods[b][None], w, pos, cu_slots, valid_len, shape,
                          qkv_attn_fill, o_local_fill)
        z = euler_update(z, u, sigmas[k], sigmas[k + 1])
    return z


# ------------------------------------------------------------ output frames

def frames_to_u8(frames, layout: int = 0) -> np.ndarray:
    """Decoded video [B, 3, T, H, W] -> compact uint8 frames.

    [RT-H3] Key takeaways (decoding and media output) and [FH3-zh]
    vLLM-Omni 中的系统级优化 (GPU output preparation): decoded FP32 frames are
    converted once, on the GPU, into contiguous uint8 BTHWC data, and the
    H.264 encoder takes planar data without another interleaved buffer.

    The pages give no value rule.  Reading: the usual decoder post-processing,
    v = clamp(x / 2 + 1 / 2, 0, 1), u = v * 255 rounded half to even, with NaN
    mapped to 0.  Because rounding decides an integer here, the oracle takes
    each step in float32, the precision the kernel decides in (x * 0.5 is exact,
    so x * 0.5 + 0.5 rounds once).

    layout 0 returns [B, T, H, W, 3] (interleaved RGB), layout 1 returns
    [B, T, 3, H, W] (one plane per channel and frame).
    """
    x = np.asarray(frames, dtype=np.float32)
    v = x * np.float32(0.5) + np.float32(0.5)
    v = np.where(np.isnan(v), np.float32(0.0), v)
    v = np.minimum(np.maximum(v, np.float32(0.0)), np.float32(1.0))
    u = np.rint(v * np.float32(255.0)).astype(np.uint8)
    if layout == 0:
        return np.ascontiguousarray(u.transpose(0, 2, 3, 4, 1))
    if layout == 1:
        return np.ascontiguousarray(u.transpose(0, 2, 1, 3, 4))
    raise ValueError("layout must be 0 or 1")


# ------------------------------------------- FP8 (MX-scaled e4m3) attention

# [FH3-zh] 超出 FastH3 配置的扩展能力 (sparse and quantized attention): an FP8 attention
# path (SAGE FP8) gives up to 1.24x on the base pipeline with small quality
# loss.  The pages give no algorithm.  Reading: Q (with the softmax scale and
# log2 e folded in), K and V are stored as OCP e4m3 with one power-of-two
# (E8M0) scale per 32 consecutive elements along the contraction (head dim
# for Q and K, keys for V).  The softmax weights enter P.V as e4m3 values
# too: with scores s in log2 units and M the smallest integer >= the row's
# largest score, key j carries w_j = e4m3(2^(8 + s_j - M)) (nearest, ties to
# even), and the output row is sum_j w_j v_j / sum_j w_j.  Because M is an
# integer, w_j is 2^(8 - M) times the e4m3 rounding of 2^(s_j) wherever that
# value is an e4m3 normal (w_j >= 2^-6), so any integer reference gives the
# same weights there.  Everything else is exact.

E4M3_MAX = 448.0


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest OCP e4m3 value (ties to even), for |x| <= 464.

    e4m3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; normals 2^-6 .. 448,
    subnormals k * 2^-9.  Values are returned as float64.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # quantum of the binade containing a (subnormal binade below 2^-6)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    q = np.ldexp(1.0, (e - 3).astype(np.int64))
    r = np.round(a / q) * q          # numpy rounds ties to even, a / q is exact
    return np.where(x < 0, -r, r)


def e8m0_exponent(amax) -> np.ndarray:
    """Block scale exponent: the smallest e in [-127, 127] with amax <= 448 * 2^e
    (0 for an all-zero block)."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.ceil(np.log2(np.where(a > 0, a, 1.0) / E4M3_MAX))
    # log2 can be off by one ulp at exact powers: settle on the exact inequality
    e = np.where(a > E4M3_MAX * np.ldexp(1.0, e.astype(np.int64)), e + 1, e)
    e = np.where(a <= E4M3_MAX * np.ldexp(1.0, (e - 1).astype(np.int64)), e - 1, e)
    e = np.where(a > 0, e, 0.0)
    return np.clip(e, -127, 127).astype(np.int64)


def mx_quantize(x, fold: float = 1.0, block: int = 32):
    """Rows of x (float32 values, last axis a multiple of `block`) times `fold`
    (rounded to float32 once, as a float32 product) -> (e4m3 values as float64,
    E8M0 exponents per block).  Dequantized value = q * 2^e."""
    v = np.asarray(x, dtype=np.float32) * np.float32(fold)
    shp = v.shape
    vb = v.astype(np.float64).reshape(*shp[:-1], shp[-1] // block, block)
    e = e8m0_exponent(np.max(np.abs(vb), axis=-1))
    q = e4m3_round(vb / np.ldexp(1.0, e)[..., None])
    return q.reshape(shp), e


def mx_dequantize(q, e, block: int = 32) -> np.ndarray:
    q = np.asarray(q, dtype=np.float64)
    shp = q.shape
    qb = q.reshape(*shp[:-1], shp[-1] // block, block)
    return (qb * np.ldexp(1.0, np.asarray(e))[..., None]).reshape(shp)


def fp8_fold(head_dim: int) -> np.float32:
    """The factor folded into Q: fp32 1/sqrt(D) (correctly rounded fp32 square
    root and quotient) times fp32 log2(e), one fp32 product."""
    inv = np.float32(1.0) / np.sqrt(np.float32(head_dim))
    return np.float32(inv * np.float32(1.4426950408889634))


def fp8_weights(sc) -> np.ndarray:
    """The softmax weights of the FP8 path for score rows sc [r, n] (log2
    units): w = e4m3(2^(8 + s - M)), M = ceil(row max) (see above).  The
    largest weight of a row lies in [128, 256]; the output row is
    (w @ v) / w.sum()."""
    sc = _f64(sc)
    m = np.ceil(sc.max(axis=-1, keepdims=True))
    return e4m3_round(np.exp2(sc - m + 8.0))


def _valid_row_mask(n_buf: int, cu, vl) -> np.ndarray:
    mask = np.zeros(n_buf, dtype=bool)
    for s in range(len(cu) - 1):
        lo = int(cu[s])
        mask[lo:lo + int(vl[s])] = True
    return mask


def varlen_attention_fp8_operands(q, k, v, cu_slots, valid_len, q_rows=None, skip_log2=None,
                                  round_p: bool = True):
    """Attention over the MX-e4m3-quantized operands of the FP8 path.  k, v
    [N, h, D] float32 values; q is [N, h, D], or [len(q_rows), h, D] already
    restricted to the query rows q_rows (buffer rows).  Q is quantized after
    folding scale * log2(e); the scores are then in log2 units, and softmax
    uses base 2.  round_p: the weights are fp8_weights of the scores (the
    reading above); False keeps them exact (2^(s - max)), the attention of the
    quantized operands alone.  Only rows inside a segment's valid range are
    quantized (pad rows may hold anything, NaN included).
    skip_log2: apply the Skip-Softmax rule to the scores of the quantized
    operands; q_rows must then be whole query groups of each segment."""
    q = np.asarray(q, dtype=np.float32)
    D = q.shape[-1]
    c = float(fp8_fold(D))
    N, h, _ = np.asarray(k).shape
    rows = np.arange(q.shape[0]) if q_rows is None else np.asarray(q_rows)
    cu = np.asarray(cu_slots)
    vl = np.asarray(valid_len) if valid_len is not None else cu[1:] - cu[:-1]
    valid = _valid_row_mask(N, cu, vl)
    # Q is quantized row by row: only the rows asked for are needed, and only valid ones
    qsel = q if q_rows is None or q.shape[0] == len(rows) else q[rows]
    qsel = np.where(valid[rows][:, None, None], qsel, np.float32(0))
    kv = np.where(valid[:, None, None], np.asarray(k, dtype=np.float32), np.float32(0))
    kq, ke = mx_quantize(kv)
    # V is quantized along the keys of each segment slot: blocks of 32 keys from the slot start
    vt = np.asarray(v, dtype=np.float32)
    vdq = np.zeros((N, h, D))
    for s in range(len(cu) - 1):
        lo, n = int(cu[s]), int(vl[s])
        if n == 0:
            continue
        npad = -(-n // 32) * 32
        seg = np.zeros((npad, h, D), np.float32)
        seg[:n] = vt[lo:lo + n]
        segT = seg.transpose(1, 2, 0)                     # [h, D, keys]
        vq, ve = mx_quantize(segT)
        vdq[lo:lo + n] = mx_dequantize(vq, ve).transpose(2, 0, 1)[:n]
    qd = mx_dequantize(*mx_quantize(qsel, fold=c))
    kd = mx_dequantize(kq, ke)
    weights = fp8_weights if round_p else None
    if skip_log2 is not None:
        # the scores qd.kd are already in log2 units: scale 1/log2(e) cancels
        # the log2(e) the Skip-Softmax oracle applies
        return varlen_attention_skip(qd, kd, vdq, cu, vl, skip_log2, scale=1.0 / np.log2(np.e),
                                     q_rows=None if q_rows is None else rows, weights=weights)
    out = np.zeros((len(rows), h, D))
    for s in range(len(cu) - 1):
        lo, n = int(cu[s]), int(vl[s])
        sel = np.nonzero((rows >= lo) & (rows < lo + n))[0]
        if sel.size == 0:
            continue
        for hh in range(h):
            sc = qd[sel, hh] @ kd[lo:lo + n, hh].T                  # log2 units
            p = fp8_weights(sc) if round_p else np.exp2(sc - sc.max(axis=1, keepdims=True))
            out[sel, hh] = (p @ vdq[lo:lo + n, hh]) / p.sum(axis=1, keepdims=True)
    return out


# ------------------------------------------------- FP8 (MX-scaled e4m3) GEMMs

# [FH3-zh] 超出 FastH3 配置的扩展能力 (quantization path): online FP8 lowers the
# peak HBM footprint by about 39% and the latency by about 5%.  The pages give
# no format.  Reading: both operands of a projection, the weight [out, in] and
# the activation [rows, in], are stored as OCP e4m3 with one power-of-two
# (E8M0) scale per 32 consecutive elements along the contraction (in), the
# same MX block rule as the FP8 attention operands; the weight is quantized
# once, the activation on the fly from its bf16 value.  The product of the
# dequantized operands is exact; only its final rounding to the output type
# remains.

def linear_fp8_operands(x, w) -> np.ndarray:
    """x @ w^T over MX-e4m3-quantized operands: x [rows, K] and w [out, K]
    (float32 values, K a multiple of 32), each quantized along K.  Returns the
    exact float64 product of the dequantized operands."""
    xd = mx_dequantize(*mx_quantize(x))
    wd = mx_dequantize(*mx_quantize(w))
    return xd @ wd.T


# ------------------------------------------------------------ Skip-Softmax

# [FH3-zh] 超出 FastH3 配置的扩展能力 (sparse and quantized attention):
# Skip-Softmax is named among the attention variants that speed up the base
# pipeline at small quality cost; the pages give no rule.  Reading: keys are
# visited in blocks of 64 from the segment start and queries in groups of 32
# consecutive valid rows from the segment start; a key block is skipped for a
# query group -- its probabilities are taken as zero -- when, for every row of
# the group, the block's largest score is more than |t| below the row's
# running maximum over the blocks visited before it (scores in log2 units,
# i.e. q.k * scale * log2 e; t < 0).  The first block is never skipped.  A
# skipped key's weight is at most 2^t times the row's largest weight.  The
# pages give no granularity either: the 64-key block and the 32-row group are
# taken from the GPU kernels' own key tile and wave, so that a decision never
# splits a tile or a wave (a reading fixed by the implementation, not by the
# pages).

def skip_softmax_rows(sc, v, skip_log2: float, q_group: int = 32, k_block: int = 64,
                      weights=None) -> np.ndarray:
    """Query rows of one segment and head under the rule above: sc [r, n]
    scores in log2 units of r consecutive query rows against the segment's n
    keys, v [n, D].  The rows start at a multiple of q_group from the segment
    start and hold whole groups (the segment's last group may be shorter).
    Returns the r output rows, each a base-2 softmax over the keys its group
    keeps (weights: a function of the kept score rows giving their weights,
    default 2^(s - row max))."""
    r, n = sc.shape
    out = np.zeros((r, v.shape[1]))
    for g0 in range(0, r, q_group):
        rows = slice(g0, min(g0 + q_group, r))
        keep = np.zeros(n, dtype=bool)
        m_run = None
        for b0 in range(0, n, k_block):
            blk = slice(b0, min(b0 + k_block, n))
            bmax = sc[rows, blk].max(axis=1)
            if m_run is not None and np.all(bmax < m_run + skip_log2):
                continue
            keep[blk] = True
            m_run = bmax if m_run is None else np.maximum(m_run, bmax)
        ss = sc[rows][:, keep]
        p = np.exp2(ss - ss.max(axis=1, keepdims=True)) if weights is None else weights(ss)
        out[rows] = (p @ v[keep]) / p.sum(axis=1, keepdims=True)
    return out


def varlen_attention_skip(q, k, v, cu_slots, valid_len, skip_log2: float,
                          scale: Optional[float] = None, q_group: int = 32,
                          k_block: int = 64, q_rows: Optional[np.ndarray] = None,
                          weights=None) -> np.ndarray:
    """Attention with the Skip-Softmax rule above; k, v [n_buf, H, D].
    Returns [n_buf, H, D] (rows outside every segment are 0) and applies the
    rule exactly in float64: a block is skipped or kept whole.
    q_rows: if given, q holds only those buffer rows, in increasing order, and
    the result has q's shape; within each segment they must be whole query
    groups (the rule is decided per group)."""
    k, v = _f64(k), _f64(v)
    n_buf, h, d = k.shape
    rows = np.arange(n_buf) if q_rows is None else np.asarray(q_rows)
    q = _f64(q)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    c = scale * np.log2(np.e)
    out = np.zeros((len(rows), h, d))
    cu = np.asarray(cu_slots)
    vl = np.asarray(valid_len) if valid_len is not None else np.diff(cu)
    for s in range(len(cu) - 1):
        lo, n = int(cu[s]), int(vl[s])
        if n == 0:
            continue
        sel = np.nonzero((rows >= lo) & (rows < lo + n))[0]
        if sel.size == 0:
            continue
        rel = rows[sel] - lo
        # whole groups, in order: each run starts at a group boundary and is
        # contiguous up to its group's end (or the segment's end)
        starts = np.nonzero(np.diff(np.concatenate([[-2], rel])) != 1)[0]
        ends = np.concatenate([starts[1:], [len(rel)]])
        for a, b in zip(starts, ends):
            end = int(rel[b - 1]) + 1
            assert int(rel[a]) % q_group == 0 and (end % q_group == 0 or end == n), \
                "q_rows must be whole query groups"
            for head in range(h):
                sc = (q[sel[a:b], head] @ k[lo:lo + n, head].T) * c   # log2 units
                out[sel[a:b], head] = skip_softmax_rows(sc, v[lo:lo + n, head], skip_log2, q_group, k_block,
                                                        weights)
    return out
