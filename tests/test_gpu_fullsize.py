"""Parity at the full sizes of the 10 s request share, in the launch configuration
the benchmark times, on sampled outputs the oracle computes one by one (GPU)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _util import TORCH_DT, assert_close, dev, dev_i32, host

pytestmark = pytest.mark.gpu

WL = W.SHARE_10S


@pytest.fixture(scope="module")
def share10s():
    w = W.block_weights(WL, 0, "bf16")
    bi = W.block_inputs(WL, 0, "bf16")
    return w, bi


def _sample_rows(n, extra, k=24, seed=0):
    r = np.random.default_rng(seed).choice(n, size=k, replace=False)
    return np.unique(np.concatenate([r, np.asarray(extra)]))


def test_attention_10s_share_sampled(lib, share10s):
    """5 heads x 128 over the whole 246,208-row buffer (246,206 valid rows)."""
    _, bi = share10s
    hc, D = WL.head_count, WL.head_dim
    qa = dev(bi.qkv_attn.reshape(WL.n_pad_total, -1), "bf16")
    o = torch.full((WL.n_pad_total, hc * D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lib.h3_varlen_attn(qa[:, :hc * D], qa[:, hc * D:2 * hc * D], qa[:, 2 * hc * D:], o, hc, D,
                       dev_i32(bi.cu_slots), dev_i32(bi.valid_len), int(bi.valid_len.max()))
    torch.cuda.synchronize()
    n = WL.n_valid
    rows = _sample_rows(n, [0, 1, 255, 256, n - 1])
    got = host(o[torch.from_numpy(rows).cuda()]).reshape(len(rows), hc, D)
    q, k, v = bi.qkv_attn[:, 0], bi.qkv_attn[:, 1], bi.qkv_attn[:, 2]
    ref = O.varlen_attention(q[rows], k, v, bi.cu_slots, bi.valid_len, q_rows=rows)
    # outputs are means over ~2.5e5 keys (|o| ~ 1e-2): check the relative error too
    assert_close(got, ref, "bf16", "attn 10s sampled", rel_l2=1e-2)
    pad = host(o[WL.n_valid:])
    assert np.all(pad == 0)


def test_block_10s_share_sampled(lib, share10s):
    """The whole block on rank 7's 30,776 rows (video, audio and structural pad rows)."""
    w, bi = share10s
    wd = {k: dev(getattr(w, k), "bf16") for k in ("w_qkv", "w_o", "w1", "w3", "w2", "g_q", "g_k")}
    x = dev(bi.x, "bf16")
    hc, D = WL.head_count, WL.head_dim
    cfg = lib.block_config(WL.dim, WL.n_heads, D, WL.ffn_dim, WL.sections, WL.theta, WL.eps_qk,
                           WL.eps_mod, 0, torch.bfloat16)
    lib.h3_dit_block_forward(cfg, wd, x, dev(bi.mod, "bf16"), dev_i32(bi.pos), dev_i32(bi.cu_slots),
                             dev_i32(bi.valid_len), int(bi.valid_len.max()),
                             qkv_attn=dev(bi.qkv_attn.reshape(WL.n_pad_total, -1), "bf16"),
                             o_attn=torch.zeros((WL.n_pad_total, hc * D), dtype=torch.bfloat16, device="cuda"),
                             o_local=dev(bi.o_local.reshape(WL.n_loc, -1), "bf16"), tok_begin=WL.tok_begin,
                             head_begin=WL.head_begin, head_count=hc)
    torch.cuda.synchronize()
    n = WL.n_loc
    pos = bi.pos
    first_audio = int(np.nonzero(pos[:, 0] == W.POS_AUDIO)[0][0])
    rows = _sample_rows(n, [0, first_audio - 1, first_audio, n - 3, n - 2, n - 1], k=12)
    got = host(x[torch.from_numpy(rows).cuda()])
    ref = O.dit_block(bi.x, bi.mod, w, bi.pos, bi.cu_slots, bi.valid_len, O.BlockShape.of(WL),
                      bi.qkv_attn, bi.o_local, rows=rows)
    assert_close(got, ref, "bf16", "block 10s sampled")
