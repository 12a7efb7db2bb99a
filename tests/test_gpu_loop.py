"""Four-forward student loop glue (timestep modulation, Euler update) and a small
whole loop against the float64 oracle (GPU)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _util import TORCH_DT, assert_close, dev, dev_i32, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("sigma", [1.0, 0.75, 0.25, 0.0])
def test_timestep_modulation(lib, dtype, sigma):
    wl = W.TINY.replace(n_blocks=3)
    tw = W.timestep_weights(wl, 0, dtype)
    out = torch.empty((wl.n_blocks, 6, wl.dim), dtype=TORCH_DT[dtype], device="cuda")
    lib.h3_timestep_modulation(sigma, dev(tw.w_t1, dtype), dev(tw.w_t2, dtype), dev(tw.table, dtype), out)
    torch.cuda.synchronize()
    assert_close(host(out), O.timestep_modulation(sigma, tw), dtype, f"temb sigma={sigma}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_euler_update(lib, dtype):
    n = 480 * 256
    z = W.as_dtype_values(W.normal(0, "z", (n,)), dtype)
    u = W.as_dtype_values(W.normal(0, "u", (n,)), dtype)
    zt, ut = dev(z, dtype), dev(u, dtype)
    xn = torch.empty_like(zt)
    lib.h3_euler_update(zt, ut, xn, 0.75, 0.5)
    torch.cuda.synchronize()
    ref = O.euler_update(z, u, 0.75, 0.5)
    assert_close(host(zt), ref, dtype, "euler z")
    assert np.array_equal(host(xn), host(zt))
    # u aliasing x_next (the loop passes the stack output as both)
    zt, ut = dev(z, dtype), dev(u, dtype)
    lib.h3_euler_update(zt, ut, ut, 0.25, 0.0)
    torch.cuda.synchronize()
    assert_close(host(zt), O.euler_update(z, u, 0.25, 0.0), dtype, "euler aliased")
    assert np.array_equal(host(ut), host(zt))


def run_student_loop(lib, wl, blocks, tw, bi, dtype, sigmas):
    """Device loop: x is the stack's running input, z the latent; per forward the
    blocks update x in place, then z += dsigma * x and x <- z."""
    z = dev(bi.x, dtype)
    x = z.clone()
    cfg = lib.block_config(wl.dim, wl.n_heads, wl.head_dim, wl.ffn_dim, wl.sections, wl.theta,
                           wl.eps_qk, wl.eps_mod, 0, TORCH_DT[dtype])
    wd = [{k: dev(getattr(w, k), dtype) for k in ("w_qkv", "w_o", "w1", "w3", "w2", "g_q", "g_k")}
          for w in blocks]
    t1, t2, tab = dev(tw.w_t1, dtype), dev(tw.w_t2, dtype), dev(tw.table, dtype)
    mods = torch.empty((wl.n_blocks, 6, wl.dim), dtype=TORCH_DT[dtype], device="cuda")
    pos, cu, vl = dev_i32(bi.pos), dev_i32(bi.cu_slots), dev_i32(bi.valid_len)
    extra = {}
    if wl.share_mode:
        extra = dict(qkv_attn=dev(bi.qkv_attn.reshape(wl.n_pad_total, -1), dtype),
                     o_attn=torch.zeros((wl.n_pad_total, wl.head_count * wl.head_dim),
                                        dtype=TORCH_DT[dtype], device="cuda"),
                     o_local=dev(bi.o_local.reshape(wl.n_loc, -1), dtype), tok_begin=wl.tok_begin,
                     head_begin=wl.head_begin, head_count=wl.head_count)
    for k in range(len(sigmas) - 1):
        lib.h3_timestep_modulation(sigmas[k], t1, t2, tab, mods)
        for b in range(wl.n_blocks):
            lib.h3_dit_block_forward(cfg, wd[b], x, mods[b:b + 1], pos, cu, vl, int(bi.valid_len.max()),
                                     **extra)
        lib.h3_euler_update(z, x, x, sigmas[k], sigmas[k + 1])
    torch.cuda.synchronize()
    return host(z)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_student_loop_tiny(lib, dtype):
    """Two blocks, four forwards over the five sigma positions, broadcast modulation."""
    wl = W.TINY.replace(n_blocks=2, n_forwards=4, mod_per_token=False)
    blocks = [W.block_weights(wl, 0, dtype, block=b) for b in range(wl.n_blocks)]
    tw = W.timestep_weights(wl, 0, dtype)
    bi = W.block_inputs(wl, 0, dtype)
    got = run_student_loop(lib, wl, blocks, tw, bi, dtype, W.STUDENT_SIGMAS)
    ref = O.student_loop(bi.x, blocks, tw, bi.pos, bi.cu_slots, bi.valid_len, O.BlockShape.of(wl),
                         W.STUDENT_SIGMAS)
    assert_close(got, ref, dtype, "student loop tiny")
    # sigma 1 -> 0 in four steps moves the latent: the result is not the input
    assert not np.allclose(got, bi.x, atol=1e-3)


def test_student_loop_tiny_rank_share(lib):
    """The loop in rank-share mode (4 ranks, rank 2): every block reuses the other ranks' rows."""
    wl = W.TINY.replace(n_blocks=2, mod_per_token=False, sp_degree=4, rank=2)
    blocks = [W.block_weights(wl, 3, "f32", block=b) for b in range(wl.n_blocks)]
    tw = W.timestep_weights(wl, 3, "f32")
    bi = W.block_inputs(wl, 3, "f32")
    got = run_student_loop(lib, wl, blocks, tw, bi, "f32", W.STUDENT_SIGMAS)
    ref = O.student_loop(bi.x, blocks, tw, bi.pos, bi.cu_slots, bi.valid_len, O.BlockShape.of(wl),
                         W.STUDENT_SIGMAS, bi.qkv_attn, bi.o_local)
    assert_close(got, ref, "f32", "student loop share")
