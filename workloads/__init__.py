"""Seeded synthetic workloads for the packed audio-video DiT block.

This module only *describes and draws* inputs: shapes, positions, segment
offsets and seeded random tensors.  It holds none of the block's arithmetic, so
both the CPU oracle (``oracle/``) and the GPU path (the package, ``bench.py``)
may import it without sharing any computation.

Sources for the shapes (page titles abbreviated):
  [RT-H3]  "Why Real-Time MiniMax H3 Serving Requires More Than a Faster DiT"
  [FH3-zh] "MiniMax H3 通过 vLLM-Omni 实现 FastH3 实时推理"
The request is 1344x768 at 24 FPS ([RT-H3] Key takeaways; [FH3-zh] FastH3
推理配置) with 124/243/362 frames for 5/10/15 s ([FH3-zh] 时长扫描).  The pages
give no model dimensions; hidden size, heads, latent compression, patch size,
audio token rate and the RoPE split used here are assumed values, not the
pages'.  Token order in the packed sequence is [video | audio | structural
suffix pad]; the pad brings N up to a multiple of the sequence-parallel degree
8 ([RT-H3] Key takeaways: valid lengths, suffix padding removed; [FH3-zh]
FastH3 推理配置: ``--usp 8``).

Random draws: numpy PCG64.  Every tensor has its own stream, keyed by
(seed, tensor name, chunk index), so a tensor's values do not depend on which
other tensors were drawn, nor on how many threads drew it.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
import zlib
from typing import Dict, Optional

import numpy as np

# position kinds, one int32 per token, in the first column of the position table
POS_VIDEO = 0
POS_AUDIO = 1
POS_PAD = 2

_CHUNK = 1 << 22  # elements per independently seeded chunk


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dim: int            # C, hidden width
    n_heads: int        # H
    head_dim: int       # D
    ffn_dim: int        # F, SwiGLU inner width
    sections: tuple     # RoPE (t, h, w) widths, summing to head_dim
    latent_t: int       # latent frames T
    grid_h: int         # patch rows
    grid_w: int         # patch columns
    n_audio: int        # audio tokens
    sp_degree: int = 1  # sequence-parallel degree P (1 = one GPU holds everything)
    rank: int = 0       # which share this GPU runs (rank-share mode when sp_degree > 1)
    theta: float = 10000.0
    eps_qk: float = 1e-6
    eps_mod: float = 1e-6
    mod_per_token: bool = True
    pad_to: int = 0     # if set, the packed buffer is at least this long (extra suffix pad rows)
    n_blocks: int = 1
    n_forwards: int = 1

    @property
    def n_video(self) -> int:
        return self.latent_t * self.grid_h * self.grid_w

    @property
    def n_valid(self) -> int:
        return self.n_video + self.n_audio

    @property
    def n_pad_total(self) -> int:
        p = self.sp_degree
        return max((self.n_valid + p - 1) // p * p, self.pad_to)

    @property
    def n_loc(self) -> int:
        return self.n_pad_total // self.sp_degree

    @property
    def tok_begin(self) -> int:
        return self.rank * self.n_loc

    @property
    def head_count(self) -> int:
        return self.n_heads // self.sp_degree

    @property
    def head_begin(self) -> int:
        return self.rank * self.head_count

    @property
    def share_mode(self) -> bool:
        return self.sp_degree > 1

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _ffn(c: int, multiple_of: int) -> int:
    # inner width: smallest multiple of `multiple_of` >= 8C/3
    return multiple_of * (-(-(8 * c // 3) // multiple_of))


def _latent_frames(frames: int) -> int:
    return frames // 4 + 1


TINY = Workload(name="tiny", dim=256, n_heads=4, head_dim=64, ffn_dim=_ffn(256, 64),
                sections=(16, 24, 24), latent_t=4, grid_h=8, grid_w=12, n_audio=96)

_BIG = dict(dim=5120, n_heads=40, head_dim=128, ffn_dim=_ffn(5120, 256),
            sections=(32, 48, 48), grid_h=48, grid_w=84, sp_degree=8, rank=7)

SHARE_5S = Workload(name="share5s", latent_t=_latent_frames(124), n_audio=126, **_BIG)
SHARE_10S = Workload(name="share10s", latent_t=_latent_frames(243), n_audio=254, **_BIG)
LOOP_15S = Workload(name="loop15s", latent_t=_latent_frames(362), n_audio=379,
                    mod_per_token=False, n_blocks=8, n_forwards=4, **_BIG)

PRESETS: Dict[str, Workload] = {w.name: w for w in (TINY, SHARE_5S, SHARE_10S, LOOP_15S)}

# Five noise levels for the four-forward student ([FH3-zh] FastH3：四步学生模型: four
# forwards over five sigma positions).  The values are not on the pages.
STUDENT_SIGMAS = (1.0, 0.75, 0.5, 0.25, 0.0)


# --------------------------------------------------------------------------- rng

def _key(name: str) -> int:
    return zlib.crc32(name.encode("utf-8"))


def _fill_chunk(out: np.ndarray, seed: int, key: int, idx: int, lo: int, hi: int):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, key, idx])))
    out[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)


def normal(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0,
           threads: Optional[int] = None) -> np.ndarray:
    """float32 N(mean, std^2) draws of `shape`, independent per (seed, name)."""
    n = int(np.prod(shape)) if len(shape) else 1
    flat = np.empty(n, dtype=np.float32)
    key = _key(name)
    chunks = [(i, i * _CHUNK, min(n, (i + 1) * _CHUNK)) for i in range((n + _CHUNK - 1) // _CHUNK)]
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if len(chunks) <= 1 or threads <= 1:
        for i, lo, hi in chunks:
            _fill_chunk(flat, seed, key, i, lo, hi)
    else:
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda c: _fill_chunk(flat, seed, key, *c), chunks))
    if std != 1.0:
        flat *= np.float32(std)
    if mean != 0.0:
        flat += np.float32(mean)
    return flat.reshape(shape)


def _fill_uniform(out: np.ndarray, seed: int, key: int, idx: int, lo: int, hi: int):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, key, idx])))
    out[lo:hi] = g.random(hi - lo, dtype=np.float32)


def uniform(seed: int, name: str, shape, low: float, high: float,
            threads: Optional[int] = None) -> np.ndarray:
    """float32 U[low, high) draws of `shape`, independent per (seed, name)."""
    n = int(np.prod(shape)) if len(shape) else 1
    flat = np.empty(n, dtype=np.float32)
    key = _key(name)
    chunks = [(i, i * _CHUNK, min(n, (i + 1) * _CHUNK)) for i in range((n + _CHUNK - 1) // _CHUNK)]
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if len(chunks) <= 1 or threads <= 1:
        for i, lo, hi in chunks:
            _fill_uniform(flat, seed, key, i, lo, hi)
    else:
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda c: _fill_uniform(flat, seed, key, *c), chunks))
    flat *= np.float32(high - low)
    flat += np.float32(low)
    return flat.reshape(shape)


def uniform_ints(seed: int, name: str, low: int, high: int, size: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _key(name), 0])))
    return g.integers(low, high, size=size, endpoint=True)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value (ties to even), kept as float32.

    This is a storage step of input preparation: the GPU path receives these
    exact values as bf16, and the oracle receives the same values upcast.
    NaN stays NaN.
    """
    src = np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
    out = np.empty_like(src)
    step = 1 << 22

    def one(lo):
        u = src[lo:lo + step].view(np.uint32)
        r = (u >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += u                       # wraps only for NaN bit patterns, fixed below
        r &= np.uint32(0xFFFF0000)
        o = r.view(np.float32)
        nan = np.isnan(src[lo:lo + step])
        if nan.any():
            o[nan] = np.float32(np.nan)
        out[lo:lo + step] = o

    starts = range(0, src.size, step)
    if src.size > step:
        with _cf.ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
            list(ex.map(one, starts))
    else:
        for lo in starts:
            one(lo)
    return out.reshape(np.shape(a))


def as_dtype_values(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(a)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(dtype)


# --------------------------------------------------------------------- positions

def positions(wl: Workload) -> np.ndarray:
    """int32 [N_pad_total, 4] = (kind, t, h, w) for every token of the packed sequence.

    Video tokens enumerate (t, h, w) with t slowest; audio tokens carry their audio
    index in column 1; structural pad rows have kind POS_PAD and zeros.
    """
    npad = wl.n_pad_total
    pos = np.zeros((npad, 4), dtype=np.int32)
    t, h, w = np.meshgrid(np.arange(wl.latent_t), np.arange(wl.grid_h), np.arange(wl.grid_w),
                          indexing="ij")
    nv = wl.n_video
    pos[:nv, 0] = POS_VIDEO
    pos[:nv, 1] = t.reshape(-1)
    pos[:nv, 2] = h.reshape(-1)
    pos[:nv, 3] = w.reshape(-1)
    pos[nv:wl.n_valid, 0] = POS_AUDIO
    pos[nv:wl.n_valid, 1] = np.arange(wl.n_audio)
    pos[wl.n_valid:, 0] = POS_PAD
    return pos


def block_segments(wl: Workload):
    """One joint audio-video segment per request: slot [0, N_pad_total), first N valid."""
    cu = np.array([0, wl.n_pad_total], dtype=np.int32)
    valid = np.array([wl.n_valid], dtype=np.int32)
    return cu, valid


# ------------------------------------------------------------- varlen attention

@dataclasses.dataclass
class VarlenCase:
    n_buf: int
    n_heads: int
    head_dim: int
    cu_slots: np.ndarray   # int32 [S+1]
    valid_len: np.ndarray  # int32 [S]
    q: np.ndarray          # [n_buf, H, D] float32 (dtype-representable)
    k: np.ndarray
    v: np.ndarray


def varlen_case(seed: int = 0, lengths=(4032, 1500, 17), n_buf: int = 8192, n_heads: int = 8,
                head_dim: int = 128, dtype: str = "bf16", pad_fill: str = "normal") -> VarlenCase:
    """Packed segments, each followed by suffix padding, filling an n_buf buffer.

    The total padding n_buf - sum(lengths) is split over the segments by sorted
    seeded uniform cut points.  pad_fill: "normal" (N(0,1) like valid rows),
    "nan" (NaN in q/k/v pad rows, +Inf in alternate rows) or "zero".
    """
    lengths = [int(x) for x in lengths]
    s = len(lengths)
    total_pad = n_buf - sum(lengths)
    if total_pad < 0:
        raise ValueError("segments do not fit the buffer")
    cuts = np.sort(uniform_ints(seed, "pad_cuts", 0, total_pad, s - 1)) if s > 1 else np.zeros(0, int)
    bounds = np.concatenate([[0], cuts, [total_pad]])
    pads = np.diff(bounds)
    cu = np.zeros(s + 1, dtype=np.int32)
    for i in range(s):
        cu[i + 1] = cu[i] + lengths[i] + pads[i]
    assert cu[-1] == n_buf
    shape = (n_buf, n_heads, head_dim)
    q = as_dtype_values(normal(seed, "q", shape), dtype)
    k = as_dtype_values(normal(seed, "k", shape), dtype)
    v = as_dtype_values(normal(seed, "v", shape), dtype)
    if pad_fill != "normal":
        for i in range(s):
            lo, hi = cu[i] + lengths[i], cu[i + 1]
            for j, t in enumerate((q, k, v)):
                if pad_fill == "zero":
                    t[lo:hi] = 0.0
                else:
                    t[lo:hi] = np.nan
                    t[lo:hi:2] = np.inf if j != 1 else -np.inf
    return VarlenCase(n_buf, n_heads, head_dim, cu, np.array(lengths, dtype=np.int32), q, k, v)


# ----------------------------------------------------------------- block inputs

WEIGHT_STD = 0.02
MOD_STD = 0.1
GAIN_STD = 0.02


@dataclasses.dataclass
class BlockWeights:
    w_qkv: np.ndarray  # [3C, C]  rows: q heads 0..H-1, then k heads, then v heads (D rows each)
    w_o: np.ndarray    # [C, H*D]
    w1: np.ndarray     # [F, C]
    w3: np.ndarray     # [F, C]
    w2: np.ndarray     # [C, F]
    g_q: np.ndarray    # [D]
    g_k: np.ndarray    # [D]


def block_weights(wl: Workload, seed: int, dtype: str, block: int = 0) -> BlockWeights:
    c, f, hd, d = wl.dim, wl.ffn_dim, wl.n_heads * wl.head_dim, wl.head_dim
    p = f"blk{block}."

    def w(name, shape, std=WEIGHT_STD, mean=0.0):
        return as_dtype_values(normal(seed, p + name, shape, std=std, mean=mean), dtype)

    return BlockWeights(
        w_qkv=w("w_qkv", (3 * hd, c)), w_o=w("w_o", (c, hd)), w1=w("w1", (f, c)),
        w3=w("w3", (f, c)), w2=w("w2", (c, f)),
        g_q=w("g_q", (d,), std=GAIN_STD, mean=1.0), g_k=w("g_k", (d,), std=GAIN_STD, mean=1.0))


@dataclasses.dataclass
class BlockInputs:
    x: np.ndarray                 # [n_loc, C]   this GPU's token rows
    mod: np.ndarray               # [n_loc, 6, C] per token, or [1, 6, C] broadcast
    pos: np.ndarray               # [n_loc, 4] int32 (this GPU's rows only)
    cu_slots: np.ndarray          # int32 [S+1] over the attention buffer
    valid_len: np.ndarray         # int32 [S]
    # rank-share mode only: what the two sequence-parallel exchanges would deliver
    qkv_attn: Optional[np.ndarray] = None  # [N_pad_total, 3, head_count, D]; local rows unused
    o_local: Optional[np.ndarray] = None   # [n_loc, H, D]; local head slice unused


def block_inputs(wl: Workload, seed: int, dtype: str) -> BlockInputs:
    n, c = wl.n_loc, wl.dim
    x = as_dtype_values(normal(seed, "x", (n, c)), dtype)
    if wl.mod_per_token:
        mod = as_dtype_values(normal(seed, "mod", (n, 6, c), std=MOD_STD), dtype)
    else:
        mod = as_dtype_values(normal(seed, "mod", (1, 6, c), std=MOD_STD), dtype)
    pos_all = positions(wl)
    pos = np.ascontiguousarray(pos_all[wl.tok_begin:wl.tok_begin + n])
    cu, valid = block_segments(wl)
    bi = BlockInputs(x=x, mod=mod, pos=pos, cu_slots=cu, valid_len=valid)
    if wl.share_mode:
        bi.qkv_attn = as_dtype_values(
            normal(seed, "qkv_attn", (wl.n_pad_total, 3, wl.head_count, wl.head_dim)), dtype)
        bi.o_local = as_dtype_values(
            normal(seed, "o_local", (n, wl.n_heads, wl.head_dim), std=0.05), dtype)
    return bi


# --------------------------------------------------------- student loop inputs

TIME_EMB_DIM = 256


@dataclasses.dataclass
class TimestepWeights:
    w_t1: np.ndarray     # [C, 256]
    w_t2: np.ndarray     # [6C, C]
    table: np.ndarray    # [n_blocks, 6, C]


def timestep_weights(wl: Workload, seed: int, dtype: str) -> TimestepWeights:
    c = wl.dim
    return TimestepWeights(
        w_t1=as_dtype_values(normal(seed, "w_t1", (c, TIME_EMB_DIM), std=WEIGHT_STD), dtype),
        w_t2=as_dtype_values(normal(seed, "w_t2", (6 * c, c), std=WEIGHT_STD), dtype),
        table=as_dtype_values(normal(seed, "mod_table", (wl.n_blocks, 6, c), std=MOD_STD), dtype))


# ------------------------------------------------------------- output frames

# 10 s request at 1344x768, 24 FPS: 243 decoded frames, one video
FRAMES_10S = dict(B=1, T=243, H=768, W=1344)


def frames(seed: int, B: int, T: int, H: int, W: int, specials: bool = True) -> np.ndarray:
    """Decoded-video stand-in, float32 [B, 3, T, H, W].

    Values are U[-1.05, 1.05) (about 5% outside the nominal [-1, 1] range).
    With `specials`, a seeded 1/64 of the entries are replaced by boundary
    cases: the exact grid points 2k/255 - 1 (as float32), the float32 values
    nearest to the half-way points (2k + 1)/255 - 1, +-1, 0, +-inf and NaN.
    """
    shape = (B, 3, T, H, W)
    x = uniform(seed, "frames", shape, -1.05, 1.05)
    if specials and x.size:
        k = np.arange(256, dtype=np.float64)
        grid = (2.0 * k / 255.0 - 1.0).astype(np.float32)
        half = (2.0 * (k + 0.5) / 255.0 - 1.0).astype(np.float32)
        table = np.concatenate([grid, half, np.array([-1.0, 1.0, 0.0, np.inf, -np.inf, np.nan],
                                                     dtype=np.float32)])
        n = x.size
        m = max(1, n // 64)
        where = uniform_ints(seed, "frames.where", 0, n - 1, m)
        which = uniform_ints(seed, "frames.which", 0, table.size - 1, m)
        flat = x.reshape(-1)
        flat[where] = table[which]
    return x

