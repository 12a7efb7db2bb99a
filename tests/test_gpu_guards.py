"""Guards around the kernels' outputs (GPU): canary bytes before and after every
output region must survive each entry point, and H3_DEBUG_VALIDATE must turn
malformed segment metadata into H3_ERR_ARG before anything is launched.

The malformed cases used here are ones that would stay inside the buffers even
if they reached a kernel (an over-long valid length of a segment that is not
the last, a decreasing offset with an empty valid range, a too-small
max_valid_len), so the test never depends on the check for memory safety.
"""
import os

import numpy as np
import pytest
import torch

import workloads as W
from _util import dev, dev_i32

pytestmark = pytest.mark.gpu

PAD = 4096          # guard elements on each side of an output region
CANARY = -12345.0   # exactly representable in bf16 and fp32


def guarded(shape, dtype, fill=0.0):
    """A tensor of `shape` carved from the middle of a larger buffer whose
    PAD elements on either side hold CANARY; returns (view, check)."""
    n = int(np.prod(shape))
    buf = torch.full((PAD + n + PAD,), CANARY, dtype=dtype, device="cuda")
    view = buf[PAD:PAD + n].view(*shape)
    view.fill_(fill)

    def check(what):
        torch.cuda.synchronize()
        lo, hi = buf[:PAD], buf[PAD + n:]
        assert torch.all(lo == CANARY) and torch.all(hi == CANARY), f"{what}: write outside its output"
    return view, check


def rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (scale * torch.randn(shape, generator=g, device="cuda")).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_canaries_elementwise_and_projections(lib, dtype):
    n, C, F = 333, 256, 704          # ragged row count: partial tiles and tails
    x, cx = guarded((n, C), dtype)
    x.copy_(rand((n, C), dtype, 1))
    y = rand((n, C), dtype, 2)
    mod = rand((n, 6, C), dtype, 3, 0.1)
    h, ch = guarded((n, C), dtype)
    lib.h3_modulate_residual(x, y=y, gate=mod[:, 2], shift=mod[:, 0], scale=mod[:, 1], h_out=h)
    cx("modulate_residual x")
    ch("modulate_residual h")
    w = rand((3 * C, C), dtype, 4, C ** -0.5)
    qkv, cq = guarded((n, 3 * C), dtype)
    lib.h3_linear(h, w, qkv)
    cq("linear store")
    lib.h3_linear(h, rand((C, C), dtype, 5, C ** -0.5), x, gate=mod[:, 2])
    cx("linear gated residual")
    w1, w3 = rand((F, C), dtype, 6, C ** -0.5), rand((F, C), dtype, 7, C ** -0.5)
    w2 = rand((C, F), dtype, 8, F ** -0.5)
    lib.h3_swiglu(h, w1, w3, w2, x, gate=mod[:, 5])
    cx("swiglu gated residual")


def test_canaries_qk_norm_rope_and_attention(lib):
    bf = torch.bfloat16
    wl = W.TINY
    H, D = wl.n_heads, wl.head_dim
    pos = dev_i32(W.positions(wl))
    n = pos.shape[0]
    qkv, cq = guarded((n, 3 * H * D), bf)
    qkv.copy_(rand((n, 3 * H * D), bf, 9))
    v_before = qkv[:, 2 * H * D:].clone()
    g = (1 + rand((D,), bf, 10, 0.02))
    lib.h3_qk_norm_rope(qkv[:, :H * D], qkv[:, H * D:2 * H * D], H, D, g, g, pos, wl.sections)
    cq("qk_norm_rope")
    assert torch.equal(qkv[:, 2 * H * D:], v_before), "qk_norm_rope wrote into v"
    # one work-group per token (2 H D / 8 >= 256 chunks): H = 16 and 20 at D = 128,
    # a window of the 10 s positions with video, audio and pad rows
    for Hb in (16, 20):
        wb = W.SHARE_10S.replace(n_heads=Hb, dim=Hb * 128)
        pb = W.positions(wb)[-300:]
        nb, Db = len(pb), 128
        qb, cqb = guarded((nb, 3 * Hb * Db), bf)
        qb.copy_(rand((nb, 3 * Hb * Db), bf, 12))
        vb = qb[:, 2 * Hb * Db:].clone()
        gb = (1 + rand((Db,), bf, 13, 0.02))
        lib.h3_qk_norm_rope(qb[:, :Hb * Db], qb[:, Hb * Db:2 * Hb * Db], Hb, Db, gb, gb, dev_i32(pb),
                            wb.sections)
        cqb(f"qk_norm_rope per-token H={Hb}")
        assert torch.equal(qb[:, 2 * Hb * Db:], vb), "qk_norm_rope wrote into v"
    case = W.varlen_case(seed=0, lengths=(300, 45, 17), n_buf=512, n_heads=2, head_dim=128)
    q, k, v = (dev(a.reshape(case.n_buf, -1), "bf16") for a in (case.q, case.k, case.v))
    o, co = guarded((case.n_buf, 2 * 128), bf, fill=7.0)
    cu, vl = dev_i32(case.cu_slots), dev_i32(case.valid_len)
    lib.h3_varlen_attn(q, k, v, o, 2, 128, cu, vl, int(case.valid_len.max()))
    co("varlen_attn")
    o8, co8 = guarded((case.n_buf, 2 * 128), bf, fill=7.0)
    lib.h3_varlen_attn_fp8(q, k, v, o8, 2, 128, cu, vl, int(case.valid_len.max()))
    co8("varlen_attn_fp8")


def test_canaries_frames(lib):
    B, T, Hh, Ww = 1, 2, 5, 37       # width not a multiple of 16: the element-wise tail
    fr = rand((B, 3, T, Hh, Ww), torch.float32, 11)
    for layout, shape in ((0, (B, T, Hh, Ww, 3)), (1, (B, T, 3, Hh, Ww))):
        n = int(np.prod(shape))
        buf = torch.full((PAD + n + PAD,), 0xA5, dtype=torch.uint8, device="cuda")
        out = buf[PAD:PAD + n].view(*shape)
        lib.h3_frames_to_u8(fr, out, layout)
        torch.cuda.synchronize()
        assert torch.all(buf[:PAD] == 0xA5) and torch.all(buf[PAD + n:] == 0xA5), f"frames layout {layout}"


def _attn_call(lib, case, cu, vl, max_len, o):
    q, k, v = (dev(a.reshape(case.n_buf, -1), "bf16") for a in (case.q, case.k, case.v))
    lib.h3_varlen_attn(q, k, v, o, case.n_heads, case.head_dim, dev_i32(cu), dev_i32(vl), max_len)


@pytest.fixture
def debug_validate():
    old = os.environ.get("H3_DEBUG_VALIDATE")
    os.environ["H3_DEBUG_VALIDATE"] = "1"
    yield
    if old is None:
        del os.environ["H3_DEBUG_VALIDATE"]
    else:
        os.environ["H3_DEBUG_VALIDATE"] = old


def test_debug_validate_accepts_good_and_rejects_malformed_metadata(lib, debug_validate):
    case = W.varlen_case(seed=1, lengths=(100, 100), n_buf=256, n_heads=2, head_dim=64)
    o_ref = torch.zeros((256, 128), dtype=torch.bfloat16, device="cuda")
    del os.environ["H3_DEBUG_VALIDATE"]
    _attn_call(lib, case, case.cu_slots, case.valid_len, 100, o_ref)
    os.environ["H3_DEBUG_VALIDATE"] = "1"
    o = torch.zeros_like(o_ref)
    _attn_call(lib, case, case.cu_slots, case.valid_len, 100, o)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "the checked call must give the unchecked result"
    slot1 = int(case.cu_slots[1])
    malformed = [
        # segment 0's valid length runs past its slot, but stays inside the buffer
        (np.array([0, slot1, 256]), np.array([slot1 + 20, 100]), 120, "outside"),
        # decreasing offsets, with nothing valid in the inverted slot
        (np.array([0, 150, 100]), np.array([100, 0]), 100, "decreases"),
        # the grid hint is below a valid length
        (case.cu_slots, case.valid_len, 99, "max_valid_len"),
    ]
    for cu, vl, max_len, word in malformed:
        o = torch.full_like(o_ref, 3.0)
        with pytest.raises(lib.H3Error) as ei:
            _attn_call(lib, case, cu, vl, max_len, o)
        assert ei.value.status == lib.H3_ERR_ARG and word in str(ei.value)
        torch.cuda.synchronize()
        assert torch.all(o == 3.0), "nothing may be launched after a failed check"


@pytest.mark.parametrize("entry", ["fp8", "skip", "fp8_skip"])
def test_debug_validate_on_the_other_attention_paths(lib, debug_validate, entry):
    case = W.varlen_case(seed=2, lengths=(100, 100), n_buf=256, n_heads=2, head_dim=128)
    q, k, v = (dev(a.reshape(case.n_buf, -1), "bf16") for a in (case.q, case.k, case.v))
    fn = {"fp8": lambda *a: lib.h3_varlen_attn_fp8(*a),
          "skip": lambda *a: lib.h3_varlen_attn_skip(*a, -20.0),
          "fp8_skip": lambda *a: lib.h3_varlen_attn_fp8_skip(*a, -20.0)}[entry]
    o = torch.full((256, 256), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.H3Error) as ei:   # the grid hint is below a valid length
        fn(q, k, v, o, 2, 128, dev_i32(case.cu_slots), dev_i32(case.valid_len), 99)
    assert ei.value.status == lib.H3_ERR_ARG and "max_valid_len" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(o == 3.0), "nothing may be launched after a failed check"
    fn(q, k, v, o, 2, 128, dev_i32(case.cu_slots), dev_i32(case.valid_len), 100)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


def test_debug_validate_in_the_block(lib, debug_validate):
    wl = W.TINY
    w = W.block_weights(wl, 0, "bf16")
    bi = W.block_inputs(wl, 0, "bf16")
    x = dev(bi.x, "bf16")
    x0 = x.clone()
    wd = {k: dev(getattr(w, k), "bf16") for k in ("w_qkv", "w_o", "w1", "w3", "w2", "g_q", "g_k")}
    cfg = lib.block_config(wl.dim, wl.n_heads, wl.head_dim, wl.ffn_dim, wl.sections)
    args = (cfg, wd, x, dev(bi.mod, "bf16"), dev_i32(bi.pos), dev_i32(bi.cu_slots), dev_i32(bi.valid_len))
    with pytest.raises(lib.H3Error) as ei:
        lib.h3_dit_block_forward(*args, int(bi.valid_len.max()) - 1)   # hint below the valid length
    assert ei.value.status == lib.H3_ERR_ARG and "max_valid_len" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.equal(x, x0), "nothing may be launched after a failed check"
    lib.h3_dit_block_forward(*args, int(bi.valid_len.max()))
    torch.cuda.synchronize()
    assert not torch.equal(x, x0)
