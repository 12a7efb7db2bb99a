"""Per-kernel parity of the HIP path against the float64 oracle (GPU).

Inputs come from the seeded generators in ``workloads``; expected values come
from ``oracle`` only.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _util import assert_close, dev, dev_i32, host

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------- qk_norm_rope

def _qk_case(wl, dtype, seed, n_rows=None):
    pos = W.positions(wl)
    if n_rows is not None:  # a contiguous window that holds video, audio and pad rows
        lo = max(0, len(pos) - n_rows)
        pos = pos[lo:]
    n = len(pos)
    hd = wl.n_heads * wl.head_dim
    qkv = W.as_dtype_values(W.normal(seed, "qkv_rows", (n, 3 * hd)) * 1.7, dtype)
    gq = W.as_dtype_values(W.normal(seed, "gq", (wl.head_dim,), std=0.02, mean=1.0), dtype)
    gk = W.as_dtype_values(W.normal(seed, "gk", (wl.head_dim,), std=0.02, mean=1.0), dtype)
    return pos, qkv, gq, gk


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", ["tiny", "tiny_pad", "h40d128", "h16d64", "h3d128", "h24d128",
                                   "h20d128"])
def test_qk_norm_rope_parity(lib, dtype, shape):
    """Row walk (tokens of fewer than 256 16-byte chunks) and one work-group per
    token (256 and more: 1, 3 and 5 chunks per thread, and 640 chunks, where
    the last of a thread's 3 chunks is masked for half the threads)."""
    if shape == "tiny":
        wl, rows = W.TINY, None
    elif shape == "tiny_pad":
        wl, rows = W.TINY.replace(pad_to=520), None
    elif shape == "h16d64":
        wl, rows = W.TINY.replace(n_heads=16, dim=1024, pad_to=500), None
    elif shape == "h3d128":
        wl, rows = W.SHARE_10S.replace(n_heads=3), 700
    elif shape == "h24d128":
        wl, rows = W.SHARE_10S.replace(n_heads=24, dim=3072), 1000
    elif shape == "h20d128":
        wl, rows = W.SHARE_10S.replace(n_heads=20, dim=2560), 1000
    else:  # the 10 s share's head layout on the tail of the sequence (video, audio, pad rows)
        wl, rows = W.SHARE_10S, 3000
    pos, qkv, gq, gk = _qk_case(wl, dtype, seed=11, n_rows=rows)
    H, D = wl.n_heads, wl.head_dim
    hd = H * D
    t = dev(qkv, dtype)
    lib.h3_qk_norm_rope(t[:, :hd], t[:, hd:2 * hd], H, D, dev(gq, dtype), dev(gk, dtype),
                        dev_i32(pos), wl.sections, wl.theta, wl.eps_qk)
    torch.cuda.synchronize()
    got = host(t)
    n = len(pos)
    q = qkv[:, :hd].reshape(n, H, D)
    k = qkv[:, hd:2 * hd].reshape(n, H, D)
    rq, rk = O.qk_norm_rope(q, k, pos, gq, gk, wl.sections, wl.theta, wl.eps_qk)
    assert_close(got[:, :hd], rq.reshape(n, hd), dtype, "q")
    assert_close(got[:, hd:2 * hd], rk.reshape(n, hd), dtype, "k")
    # v untouched bit for bit; pad rows untouched bit for bit
    assert np.array_equal(got[:, 2 * hd:], qkv[:, 2 * hd:].astype(np.float64))
    pad = pos[:, 0] == W.POS_PAD
    assert np.array_equal(got[pad], qkv[pad].astype(np.float64))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_qk_norm_rope_large_positions(lib, dtype):
    """Positions far beyond the test workloads' (video t < 3000, h < 500, w < 800;
    audio index < 20000, i.e. a rotation of up to ~3200 turns of the first pair).
    The QKV projection's store epilogue runs the same rotation code; its bit
    equality with this pass is checked in the block tests."""
    H, D, n = 3, 128, 640
    sections, theta, eps = W.SHARE_10S.sections, W.SHARE_10S.theta, W.SHARE_10S.eps_qk
    r = np.random.default_rng(17)
    pos = np.zeros((n, 4), np.int32)
    pos[:320, 0] = W.POS_VIDEO
    pos[:320, 1] = r.integers(0, 3000, 320)
    pos[:320, 2] = r.integers(0, 500, 320)
    pos[:320, 3] = r.integers(0, 800, 320)
    pos[320:, 0] = W.POS_AUDIO
    pos[320:, 1] = r.integers(0, 20000, 320)
    pos[-8:, 1] = [0, 1, 1608, 1609, 1610, 9999, 19998, 19999]
    hd = H * D
    qkv = W.as_dtype_values(W.normal(12, "qkv_rows_far", (n, 3 * hd)) * 1.7, dtype)
    gq = W.as_dtype_values(W.normal(12, "gq", (D,), std=0.02, mean=1.0), dtype)
    gk = W.as_dtype_values(W.normal(12, "gk", (D,), std=0.02, mean=1.0), dtype)
    t = dev(qkv, dtype)
    lib.h3_qk_norm_rope(t[:, :hd], t[:, hd:2 * hd], H, D, dev(gq, dtype), dev(gk, dtype), dev_i32(pos),
                        sections, theta, eps)
    torch.cuda.synchronize()
    got = host(t)
    q = qkv[:, :hd].reshape(n, H, D)
    k = qkv[:, hd:2 * hd].reshape(n, H, D)
    rq, rk = O.qk_norm_rope(q, k, pos, gq, gk, sections, theta, eps)
    assert_close(got[:, :hd], rq.reshape(n, hd), dtype, "q far positions")
    assert_close(got[:, hd:2 * hd], rk.reshape(n, hd), dtype, "k far positions")


# ----------------------------------------------------------- modulate/residual

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dim,n,mode", [(256, 480, "per_token"), (5120, 777, "per_token"),
                                        (5120, 300, "broadcast"), (1024, 65, "rms"),
                                        # every launch tier (threads x chunks per thread), whole and
                                        # partial, and the limits: 1, 129, 257, 512, 641, 1025, 2048 chunks
                                        (8, 33, "per_token"), (1032, 17, "per_token"), (2056, 17, "rms"),
                                        (4096, 9, "broadcast"), (5128, 9, "per_token"),
                                        (8200, 5, "per_token"), (16384, 5, "rms")])
def test_modulate_residual_parity(lib, dtype, dim, n, mode):
    seed = 3
    x = W.as_dtype_values(W.normal(seed, "x", (n, dim)) * 1.3 + 0.2, dtype)
    y = W.as_dtype_values(W.normal(seed, "y", (n, dim)), dtype)
    rows = 1 if mode == "broadcast" else n
    mod = W.as_dtype_values(W.normal(seed, "mod", (rows, 6, dim), std=0.1), dtype)
    kind = 1 if mode == "rms" else 0
    xt, yt, mt = dev(x, dtype), dev(y, dtype), dev(mod, dtype)
    ht = torch.empty_like(xt)
    # residual + norm in one pass (slots: gate 2, shift 3, scale 4)
    lib.h3_modulate_residual(xt, y=yt, gate=mt[:, 2], shift=mt[:, 3], scale=mt[:, 4], h_out=ht,
                             norm_kind=kind)
    torch.cuda.synchronize()
    x1 = O.gated_residual(x, mod[:, 2], y)
    h = O.modulated_norm(x1, mod[:, 3], mod[:, 4], 1e-6, "rms" if kind else "layer")
    assert_close(host(xt), x1, dtype, "x+gate*y")
    assert_close(host(ht), h, dtype, "modnorm")
    # norm only (residual off): x must stay bit-identical
    x0 = host(xt).copy()
    lib.h3_modulate_residual(xt, shift=mt[:, 0], scale=mt[:, 1], h_out=ht, norm_kind=kind)
    torch.cuda.synchronize()
    assert np.array_equal(host(xt), x0)
    h = O.modulated_norm(x0, mod[:, 0], mod[:, 1], 1e-6, "rms" if kind else "layer")
    assert_close(host(ht), h, dtype, "modnorm-only")


# -------------------------------------------------------------------- GEMMs

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("m,n,k", [(480, 768, 256), (1000, 1408, 704), (257, 304, 136),
                                   (513, 5120, 1024), (4000, 5120, 128)])
def test_linear_parity(lib, dtype, m, n, k):
    """Unit-scale operands (weights std 1/sqrt(k)) so outputs are O(1), like the block's;
    ragged M, N and K tiles.  At 4000 x 5120 the 320 tiles of 256 rows would leave a
    last round of 256 CUs mostly idle: its rows run as 128-row tiles."""
    seed = 5
    a = W.as_dtype_values(W.normal(seed, "a", (m, k)), dtype)
    w = W.as_dtype_values(W.normal(seed, "w", (n, k), std=k ** -0.5), dtype)
    out = torch.empty((m, n), dtype=dev(a[:1], dtype).dtype, device="cuda")
    lib.h3_linear(dev(a, dtype), dev(w, dtype), out)
    torch.cuda.synchronize()
    ref = O.linear(a, w)
    assert_close(host(out), ref, dtype, f"linear {m}x{n}x{k}")
    # gated residual epilogue, per-row gate and broadcast gate
    x = W.as_dtype_values(W.normal(seed, "x", (m, n)), dtype)
    g = W.as_dtype_values(W.normal(seed, "g", (m, n), std=0.1), dtype)
    xt = dev(x, dtype)
    lib.h3_linear(dev(a, dtype), dev(w, dtype), xt, gate=dev(g, dtype))
    torch.cuda.synchronize()
    assert_close(host(xt), O.gated_residual(x, g, ref), dtype, "linear+residual")
    xt = dev(x, dtype)
    lib.h3_linear(dev(a, dtype), dev(w, dtype), xt, gate=dev(g[:1], dtype))
    torch.cuda.synchronize()
    assert_close(host(xt), O.gated_residual(x, g[:1], ref), dtype, "linear+residual(bcast)")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("m,n,k", [(300, 100, 64), (300, 100, 136), (77, 36, 40), (1, 1, 8),
                                   (5, 260, 1024), (257, 9, 64)])
def test_linear_ragged_widths(lib, dtype, m, n, k):
    """Output widths that are not a multiple of 8 (the epilogues' element-wise tail),
    K a multiple of 64 (the tiled kernel) or only of 8, single rows; a, w, out and
    the gate are column windows of wider buffers, and the output's columns past n
    stay untouched."""
    seed = 6
    a = W.as_dtype_values(W.normal(seed, "a", (m, k)), dtype)
    w = W.as_dtype_values(W.normal(seed, "w", (n, k), std=k ** -0.5), dtype)
    x = W.as_dtype_values(W.normal(seed, "x", (m, n)), dtype)
    g = W.as_dtype_values(W.normal(seed, "g", (m, n), std=0.1), dtype)
    wide = lambda arr, extra: torch.cat([dev(arr, dtype), dev(np.zeros((arr.shape[0], extra), np.float32), dtype)],
                                        dim=1)
    n8 = -(-n // 8) * 8 + 8
    at, wt = wide(a, 8)[:, :k], wide(w, 16)[:, :k]
    ref = O.linear(a, w)
    for gated in (False, True):
        buf = torch.full((m, n8), float("nan"), dtype=at.dtype, device="cuda")
        out = buf[:, :n]
        if gated:
            out.copy_(dev(x, dtype))
            lib.h3_linear(at, wt, out, gate=wide(g, n8 + 8 - n)[:, :n])
        else:
            lib.h3_linear(at, wt, out)
        torch.cuda.synchronize()
        want = O.gated_residual(x, g, ref) if gated else ref
        # (a mean over a handful of elements is one rounding, not an average: the max bar then)
        few = {"mean_abs": 2e-2} if dtype == "bf16" and m * n < 64 else {}
        assert_close(host(out), want, dtype, f"linear {m}x{n}x{k} gated={gated}", **few)
        assert torch.isnan(buf[:, n:].float()).all(), "columns past n were written"


@pytest.mark.parametrize("which", ["a", "w"])
def test_linear_wide_row_strides(lib, which):
    """Row strides above 2^22 elements: K a multiple of 64, yet the call must not
    take the tiled kernel, whose per-lane load offsets are 32-bit (it runs on the
    general kernel); plain and gated residual epilogues."""
    seed, k, ld = 7, 128, (1 << 22) + 64
    m, n = (70, 296) if which == "a" else (300, 40)
    a = W.as_dtype_values(W.normal(seed, "a", (m, k)), "bf16")
    w = W.as_dtype_values(W.normal(seed, "w", (n, k), std=k ** -0.5), "bf16")
    x = W.as_dtype_values(W.normal(seed, "x", (m, n)), "bf16")
    g = W.as_dtype_values(W.normal(seed, "g", (m, n), std=0.1), "bf16")

    def strided(arr):
        buf = torch.empty((arr.shape[0], ld), dtype=torch.bfloat16, device="cuda")
        buf[:, :k] = dev(arr, "bf16")
        return buf[:, :k]

    at = strided(a) if which == "a" else dev(a, "bf16")
    wt = strided(w) if which == "w" else dev(w, "bf16")
    assert (at.stride(0) if which == "a" else wt.stride(0)) == ld
    ref = O.linear(a, w)
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    lib.h3_linear(at, wt, out)
    torch.cuda.synchronize()
    assert_close(host(out), ref, "bf16", f"linear wide {which} stride")
    xt = dev(x, "bf16")
    lib.h3_linear(at, wt, xt, gate=dev(g, "bf16"))
    torch.cuda.synchronize()
    assert_close(host(xt), O.gated_residual(x, g, ref), "bf16", f"linear+residual wide {which} stride")
    del at, wt
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n,c,f", [(480, 256, 704), (300, 512, 1408), (129, 1024, 2816), (4000, 256, 2816),
                                   # ffn_dim off the 32-row W1/W3 interleave and the 128-wide
                                   # output tile; dim off the 64-deep K step
                                   (65, 136, 712), (33, 64, 200)])
def test_swiglu_parity(lib, dtype, n, c, f):
    seed = 9
    h = W.as_dtype_values(W.normal(seed, "h", (n, c)), dtype)
    # unit-scale weights (std 1/sqrt(fan_in)): pre-activations and outputs are O(1)
    w1 = W.as_dtype_values(W.normal(seed, "w1", (f, c), std=c ** -0.5), dtype)
    w3 = W.as_dtype_values(W.normal(seed, "w3", (f, c), std=c ** -0.5), dtype)
    w2 = W.as_dtype_values(W.normal(seed, "w2", (c, f), std=f ** -0.5), dtype)
    out = dev(np.zeros((n, c), np.float32), dtype)
    lib.h3_swiglu(dev(h, dtype), dev(w1, dtype), dev(w3, dtype), dev(w2, dtype), out)
    torch.cuda.synchronize()
    ref = O.swiglu_mlp(h, w1, w3, w2)
    assert_close(host(out), ref, dtype, "swiglu")
    x = W.as_dtype_values(W.normal(seed, "x", (n, c)), dtype)
    g = W.as_dtype_values(W.normal(seed, "g", (n, c), std=0.1), dtype)
    xt = dev(x, dtype)
    lib.h3_swiglu(dev(h, dtype), dev(w1, dtype), dev(w3, dtype), dev(w2, dtype), xt, gate=dev(g, dtype))
    torch.cuda.synchronize()
    assert_close(host(xt), O.gated_residual(x, g, ref), dtype, "swiglu+residual")


# ------------------------------------------------------------- attention

def _attn_gpu(lib, c, dtype, max_len=None):
    q, k, v = (dev(t.reshape(c.n_buf, -1), dtype) for t in (c.q, c.k, c.v))
    o = torch.full_like(q, float("nan"))
    lib.h3_varlen_attn(q, k, v, o, c.n_heads, c.head_dim, dev_i32(c.cu_slots), dev_i32(c.valid_len),
                       int(max_len if max_len is not None else c.valid_len.max()))
    torch.cuda.synchronize()
    return host(o).reshape(c.n_buf, c.n_heads, c.head_dim)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lengths,n_buf,H,D", [((480,), 480, 4, 64), ((300, 77, 1, 64), 512, 3, 64),
                                              ((1000, 129, 17), 1300, 2, 128)])
def test_varlen_attention_parity_small(lib, dtype, lengths, n_buf, H, D):
    c = W.varlen_case(seed=21, lengths=lengths, n_buf=n_buf, n_heads=H, head_dim=D, dtype=dtype)
    got = _attn_gpu(lib, c, dtype)
    ref = O.varlen_attention(c.q, c.k, c.v, c.cu_slots, c.valid_len)
    assert_close(got, ref, dtype, f"attn {lengths}")


def test_varlen_attention_8k_three_segments(lib):
    """Packed 4032/1500/17 in an 8192 buffer, 8 heads x 128, bf16: parity, pad rows
    exactly 0, NaN/Inf pads change nothing bit for bit, each segment alone equals
    the packed run bit for bit, reruns are byte-identical."""
    c = W.varlen_case(seed=0, dtype="bf16")
    got = _attn_gpu(lib, c, "bf16")
    ref = O.varlen_attention(c.q, c.k, c.v, c.cu_slots, c.valid_len)
    assert_close(got, ref, "bf16", "attn 8k")
    valid = np.zeros(c.n_buf, bool)
    for s in range(3):
        valid[c.cu_slots[s]:c.cu_slots[s] + c.valid_len[s]] = True
    assert np.all(got[~valid] == 0)
    poisoned = W.varlen_case(seed=0, dtype="bf16", pad_fill="nan")
    got_p = _attn_gpu(lib, poisoned, "bf16")
    assert np.array_equal(got_p, got)
    again = _attn_gpu(lib, c, "bf16")
    assert np.array_equal(again, got)
    for s in range(3):
        lo, n = int(c.cu_slots[s]), int(c.valid_len[s])
        one = W.VarlenCase(n, 8, 128, np.array([0, n], np.int32), np.array([n], np.int32),
                           c.q[lo:lo + n], c.k[lo:lo + n], c.v[lo:lo + n])
        alone = _attn_gpu(lib, one, "bf16")
        assert np.array_equal(alone, got[lo:lo + n])


def _attn_noalloc(lib, c):
    q, k, v = (dev(t.reshape(c.n_buf, -1), "bf16") for t in (c.q, c.k, c.v))
    o = torch.full_like(q, float("nan"))
    lib.h3_varlen_attn_noalloc(q, k, v, o, c.n_heads, c.head_dim, dev_i32(c.cu_slots),
                               dev_i32(c.valid_len), int(c.valid_len.max()))
    torch.cuda.synchronize()
    return host(o).reshape(c.n_buf, c.n_heads, c.head_dim)


@pytest.mark.parametrize("kind", ["packed", "rising", "falling"])
def test_varlen_attention_long_segments(lib, kind):
    """Segments of 1025 (one key past 16 tiles), 4096 and 6400 keys beside 17-
    and 1024-key ones, with NaN/Inf pads; and one 6400-key segment whose running
    max rises on every tile or sits in the first tile (later weights underflow).
    Parity with the oracle, pad rows 0, reruns byte-identical, the no-allocation
    entry point byte-identical, a segment alone equal to its packed run."""
    if kind == "packed":
        c = W.varlen_case(seed=11, lengths=(1025, 17, 4096, 1024, 6400), n_buf=13000, n_heads=2,
                          head_dim=128, dtype="bf16", pad_fill="nan")
    else:
        c = _ramp_case(6400, 1, 64, "bf16", 0.1 if kind == "rising" else -0.1, 0.05, seed=43)
    print(f"long segments case {kind}: n_buf={c.n_buf} H={c.n_heads} D={c.head_dim}", flush=True)
    got = _attn_gpu(lib, c, "bf16")
    ref = O.varlen_attention(c.q, c.k, c.v, c.cu_slots, c.valid_len)
    assert_close(got, ref, "bf16", f"attn long segments {kind}")
    assert np.array_equal(_attn_noalloc(lib, c), got)
    valid = np.zeros(c.n_buf, bool)
    for s in range(len(c.valid_len)):
        valid[c.cu_slots[s]:c.cu_slots[s] + c.valid_len[s]] = True
    assert np.all(got[~valid] == 0)
    assert np.array_equal(_attn_gpu(lib, c, "bf16"), got)
    if kind == "packed":
        s = 2
        lo, n = int(c.cu_slots[s]), int(c.valid_len[s])
        one = W.VarlenCase(n, 2, 128, np.array([0, n], np.int32), np.array([n], np.int32),
                           c.q[lo:lo + n], c.k[lo:lo + n], c.v[lo:lo + n])
        assert np.array_equal(_attn_gpu(lib, one, "bf16"), got[lo:lo + n])


def test_varlen_attention_edge_segments(lib):
    """Zero-length and one-row segments, a segment ending exactly at the buffer end,
    a grid bound above the true maximum."""
    H, D = 2, 128
    n_buf = 200
    r = np.random.default_rng(0)
    q, k, v = (W.round_to_bf16(r.standard_normal((n_buf, H, D)).astype(np.float32)) for _ in range(3))
    cu = np.array([0, 10, 10, 11, 75, 200], np.int32)
    vl = np.array([0, 0, 1, 64, 125], np.int32)
    c = W.VarlenCase(n_buf, H, D, cu, vl, q, k, v)
    got = _attn_gpu(lib, c, "bf16", max_len=190)
    ref = O.varlen_attention(q, k, v, cu, vl)
    assert_close(got, ref, "bf16", "attn edges")
    assert np.all(got[0:10] == 0)
    assert np.allclose(got[10], v[10], atol=0)  # one-row segment: o = v exactly (p = 1)


def _ramp_case(n, H, D, dtype, slope, noise, seed):
    """One segment whose scores follow a ramp along the keys: every query is
    sqrt(D) u (u a unit vector per head) and key j is slope * j * u plus
    N(0, noise^2), so score(i, j) ~ slope * j.  With slope >= 0.1 the largest
    score of each 64-key tile exceeds the one before by more than 8 in log2
    units (a raise of the running max on every tile); a negative slope puts
    the max in the first tile and lets later tiles underflow."""
    r = np.random.default_rng(seed)
    u = r.standard_normal((H, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    q = np.broadcast_to(u[None] * np.sqrt(D), (n, H, D)) + noise * r.standard_normal((n, H, D))
    k = u[None] * (slope * np.arange(n, dtype=np.float64)[:, None, None]) + noise * r.standard_normal((n, H, D))
    v = r.standard_normal((n, H, D))
    q, k, v = (W.as_dtype_values(a.astype(np.float32), dtype) for a in (q, k, v))
    return W.VarlenCase(n, H, D, np.array([0, n], np.int32), np.array([n], np.int32), q, k, v)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["rising", "falling", "wide"])
def test_varlen_attention_running_max_paths(lib, dtype, D, kind):
    """The running max raised on every tile (O and the row sums rescaled each
    time), never raised while later tiles underflow, and raised at random
    positions (q and k of standard deviation 1.6: scores of standard deviation
    ~3.7 log2 units, a raise in ~1% of the rows; much wider scores exceed the
    bf16 bar through the bf16 rounding of the prescaled Q)."""
    n, H = 700, 2
    if kind == "wide":
        c = W.varlen_case(seed=41, lengths=(n,), n_buf=n, n_heads=H, head_dim=D, dtype=dtype)
        c = W.VarlenCase(n, H, D, c.cu_slots, c.valid_len, W.as_dtype_values(c.q * 1.6, dtype),
                         W.as_dtype_values(c.k * 1.6, dtype), c.v)
    else:
        c = _ramp_case(n, H, D, dtype, 0.1 if kind == "rising" else -0.1, 0.05, seed=42)
    got = _attn_gpu(lib, c, dtype)
    ref = O.varlen_attention(c.q, c.k, c.v, c.cu_slots, c.valid_len)
    assert_close(got, ref, dtype, f"attn running max {kind} D{D}")


def test_varlen_attention_many_segments_strided(lib):
    """Fifteen segments with lengths around the 64-key and 256-query tile edges
    (0 and 1 included) and NaN/Inf suffix pads; q, k, v read as column windows
    of one [n_buf, 3 H D] buffer, o written into a window of a wider buffer whose
    other columns must stay untouched."""
    lengths = (64, 63, 65, 1, 0, 255, 256, 257, 128, 2, 511, 17, 700, 129, 33)
    H, D = 3, 128
    hd = H * D
    n_buf = sum(lengths) + 300
    c = W.varlen_case(seed=7, lengths=lengths, n_buf=n_buf, n_heads=H, head_dim=D, dtype="bf16",
                      pad_fill="nan")
    qkv = torch.cat([dev(a.reshape(n_buf, hd), "bf16") for a in (c.q, c.k, c.v)], dim=1)
    o_big = torch.full((n_buf, hd + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    o = o_big[:, 32:32 + hd]
    lib.h3_varlen_attn(qkv[:, :hd], qkv[:, hd:2 * hd], qkv[:, 2 * hd:], o, H, D, dev_i32(c.cu_slots),
                       dev_i32(c.valid_len), max(lengths))
    torch.cuda.synchronize()
    assert torch.isnan(o_big[:, :32].float()).all() and torch.isnan(o_big[:, 32 + hd:].float()).all()
    got = host(o).reshape(n_buf, H, D)
    ref = O.varlen_attention(c.q, c.k, c.v, c.cu_slots, c.valid_len)
    assert_close(got, ref, "bf16", "attn many segments strided")
