"""Whole-block parity of h3_dit_block_forward against the float64 oracle (GPU)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _util import assert_close, dev, dev_i32, host, share_buffers, TORCH_DT

pytestmark = pytest.mark.gpu


def weights_dev(w, dtype):
    return {k: dev(getattr(w, k), dtype) for k in ("w_qkv", "w_o", "w1", "w3", "w2", "g_q", "g_k")}


def cfg_of(lib, wl, dtype):
    return lib.block_config(wl.dim, wl.n_heads, wl.head_dim, wl.ffn_dim, wl.sections, wl.theta,
                            wl.eps_qk, wl.eps_mod, 0, TORCH_DT[dtype])


def run_block(lib, wl, w, bi, dtype, x_override=None, mod_override=None, peer=False):
    x = dev(bi.x if x_override is None else x_override, dtype)
    mod = dev(bi.mod if mod_override is None else mod_override, dtype)
    extra = share_buffers(wl, bi, dtype, peer) if wl.share_mode else {}
    lib.h3_dit_block_forward(cfg_of(lib, wl, dtype), weights_dev(w, dtype), x, mod, dev_i32(bi.pos),
                             dev_i32(bi.cu_slots), dev_i32(bi.valid_len), int(bi.valid_len.max()),
                             **extra)
    torch.cuda.synchronize()
    return host(x)


def oracle_block(wl, w, bi, rows=None, x=None, mod=None):
    return O.dit_block(bi.x if x is None else x, bi.mod if mod is None else mod, w, bi.pos,
                       bi.cu_slots, bi.valid_len, O.BlockShape.of(wl), bi.qkv_attn,
                       None if bi.o_local is None else bi.o_local, rows=rows)


def check_block(got, ref, x_in, dtype, what, update=None):
    """Whole output, and (fp32, or when the update dominates x) the update x2 - x.

    In bf16 the output x2 = x + update is rounded once more to bf16; with
    |update| << |x| that rounding (2^-9 |x|) is as large as the update itself,
    so the update is only compared where it is not hidden by it.
    """
    assert_close(got, ref, dtype, what)
    if update is None:
        update = dtype == "f32"
    if update:
        upd_tol = {"bf16": dict(max_abs=2e-2, mean_abs=2e-3, rel_l2=3e-2),
                   "f32": dict(max_abs=1e-4, mean_abs=1e-5, rel_l2=1e-4)}[dtype]
        assert_close(got - x_in, ref - x_in, dtype, what + " update", **upd_tol)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_tiny_world1(lib, dtype):
    wl = W.TINY
    w = W.block_weights(wl, 0, dtype)
    bi = W.block_inputs(wl, 0, dtype)
    got = run_block(lib, wl, w, bi, dtype)
    ref = oracle_block(wl, w, bi)
    check_block(got, ref, bi.x, dtype, "block tiny")


def test_block_tiny_bf16_update_dominant(lib):
    """bf16 block where the update dominates the residual (x scaled by 1/128, gates by 8):
    the attention and MLP branches are then checked through x2 itself."""
    wl = W.TINY
    w = W.block_weights(wl, 4, "bf16")
    bi = W.block_inputs(wl, 4, "bf16")
    x = W.round_to_bf16(bi.x / 128)
    mod = bi.mod.copy()
    mod[:, O.GATE1] *= 8
    mod[:, O.GATE2] *= 8
    mod = W.round_to_bf16(mod)
    got = run_block(lib, wl, w, bi, "bf16", x_override=x, mod_override=mod)
    ref = oracle_block(wl, w, bi, x=x, mod=mod)
    upd = ref - x
    assert np.linalg.norm(upd) > 2 * np.linalg.norm(x)  # the update dominates
    check_block(got, ref, x, "bf16", "block tiny update-dominant", update=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_tiny_padded_invariance(lib, dtype):
    """Padded to 512 rows with NaN/Inf pad rows: valid rows equal the unpadded run bit for bit."""
    wl = W.TINY
    w = W.block_weights(wl, 0, dtype)
    bi = W.block_inputs(wl, 0, dtype)
    base = run_block(lib, wl, w, bi, dtype)
    wlp = wl.replace(pad_to=512)
    bip = W.block_inputs(wlp, 0, dtype)
    x = np.full((512, wl.dim), np.nan, np.float32)
    x[:480] = bi.x
    x[480::2] = np.inf
    mod = np.full((512, 6, wl.dim), np.nan, np.float32)
    mod[:480] = bi.mod
    got = run_block(lib, wlp, w, bip, dtype, x_override=x, mod_override=mod)
    assert np.array_equal(got[:480], base)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_tiny_rank_share(lib, dtype):
    """Rank-share mode at tiny size (4 ranks, 1 head each) vs the oracle's share composition."""
    for rank in (0, 3):
        wl = W.TINY.replace(sp_degree=4, rank=rank)
        w = W.block_weights(wl, 1, dtype)
        bi = W.block_inputs(wl, 1, dtype)
        got = run_block(lib, wl, w, bi, dtype)
        ref = oracle_block(wl, w, bi)
        check_block(got, ref, bi.x, dtype, f"block share r{rank}")


def test_block_tiny_peer_major_layout(lib):
    """Peer-major exchange buffers (QKV epilogue scattering into the all-to-all send
    layout, output projection reading the receive layout in place) give exactly
    the stand-in result, and so match the oracle."""
    for rank in (0, 2, 3):
        wl = W.TINY.replace(sp_degree=4, rank=rank)
        w = W.block_weights(wl, 4, "bf16")
        bi = W.block_inputs(wl, 4, "bf16")
        ref_gpu = run_block(lib, wl, w, bi, "bf16")
        got = run_block(lib, wl, w, bi, "bf16", peer=True)
        assert np.array_equal(got, ref_gpu), f"rank {rank}"
        check_block(got, oracle_block(wl, w, bi), bi.x, "bf16", f"block peer-major r{rank}")


def test_block_deterministic(lib):
    wl = W.TINY
    w = W.block_weights(wl, 2, "bf16")
    bi = W.block_inputs(wl, 2, "bf16")
    a = run_block(lib, wl, w, bi, "bf16")
    b = run_block(lib, wl, w, bi, "bf16")
    assert np.array_equal(a, b)
