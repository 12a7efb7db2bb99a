"""The binding's tensor metadata checks (CPU: they raise before any pointer is
taken, so host tensors reach the device check only when every shape, dtype and
layout is right)."""
import pytest
import torch

bf, f32 = torch.bfloat16, torch.float32


@pytest.fixture(scope="module")
def h3():
    import audio_video_diffusion_block_amd as lib
    return lib


def _raises(fn, exc, text):
    with pytest.raises(exc) as e:
        fn()
    assert text in str(e.value), str(e.value)


def test_linear_checks(h3):
    a, w, out = torch.zeros(10, 64, dtype=bf), torch.zeros(24, 64, dtype=bf), torch.zeros(10, 24, dtype=bf)
    _raises(lambda: h3.h3_linear(a, w, out), ValueError, "device memory")  # well formed
    _raises(lambda: h3.h3_linear(a, w, out[:9]), ValueError, "addresses (10, 24)")
    _raises(lambda: h3.h3_linear(a, w[:, :32], out), ValueError, "addresses (24, 64)")
    _raises(lambda: h3.h3_linear(a, w.float(), out), TypeError, "torch.float32")
    _raises(lambda: h3.h3_linear(a, w, out.float()), TypeError, "torch.float32")
    _raises(lambda: h3.h3_linear(a, torch.zeros(64, 24, dtype=bf).t(), out), ValueError, "contiguous")
    _raises(lambda: h3.h3_linear(a, w, out, gate=torch.zeros(2, 24, dtype=bf)), ValueError, "addresses (10, 24)")
    _raises(lambda: h3.h3_linear(a, w, out, gate=torch.zeros(1, 24, dtype=bf)), ValueError, "device memory")


def test_swiglu_checks(h3):
    n, c, f = 8, 64, 96
    h, out = torch.zeros(n, c, dtype=bf), torch.zeros(n, c, dtype=bf)
    w1, w3, w2 = torch.zeros(f, c, dtype=bf), torch.zeros(f, c, dtype=bf), torch.zeros(c, f, dtype=bf)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    _raises(lambda: h3.h3_swiglu(h, w1, w3, w2, out, ws=ws), ValueError, "device memory")
    wide = torch.zeros(f, 2 * c, dtype=bf)[:, :c]  # weights are bare pointers: must be dense
    _raises(lambda: h3.h3_swiglu(h, w1, wide, w2, out, ws=ws), ValueError, "w3 must be a contiguous")
    _raises(lambda: h3.h3_swiglu(h, w1, w3, w2[:, :f - 8].contiguous(), out, ws=ws), ValueError, "w2")


def test_attention_checks(h3):
    n, H, D = 128, 2, 64
    q = torch.zeros(n, 3 * H * D, dtype=bf)
    qv, kv, vv = q[:, :H * D], q[:, H * D:2 * H * D], q[:, 2 * H * D:]
    o = torch.zeros(n, H * D, dtype=bf)
    cu = torch.tensor([0, 100, 128], dtype=torch.int32)
    for fn in (h3.h3_varlen_attn, h3.h3_varlen_attn_fp8, h3.h3_varlen_attn_noalloc):
        _raises(lambda: fn(qv, kv, vv, o, H, D, cu, None, 100), ValueError, "device memory")
        _raises(lambda: fn(qv, kv[:64], vv, o, H, D, cu, None, 100), ValueError, "k has shape")
        _raises(lambda: fn(qv, kv, vv, o[:, :64], H, D, cu, None, 100), ValueError, "o has shape")
        _raises(lambda: fn(qv, kv, vv, o, H, D, cu.long(), None, 100), ValueError, "cu_slots")
        _raises(lambda: fn(qv, kv, vv, o, H, D, cu, torch.zeros(1, dtype=torch.int32), 100),
                ValueError, "valid_len")
    _raises(lambda: h3.h3_varlen_attn_fp8(qv.float(), kv.float(), vv.float(), o.float(), H, D, cu, None, 100),
            TypeError, "bfloat16")


def test_qk_and_modulate_checks(h3):
    n, H, D, C = 16, 2, 64, 128
    t = torch.zeros(n, 3 * H * D, dtype=bf)
    g = torch.zeros(D, dtype=bf)
    pos = torch.zeros(n, 4, dtype=torch.int32)
    sec = (16, 24, 24)
    _raises(lambda: h3.h3_qk_norm_rope(t[:, :H * D], t[:, H * D:2 * H * D], H, D, g, g, pos, sec),
            ValueError, "device memory")
    _raises(lambda: h3.h3_qk_norm_rope(t[:, :H * D], t[:, H * D:2 * H * D], H, D, g, g, pos[:8], sec),
            ValueError, "pos")
    _raises(lambda: h3.h3_qk_norm_rope(t[:, :H * D], t[:, H * D:2 * H * D], H, D, g[:32], g, pos, sec),
            ValueError, "g_q")
    x = torch.zeros(n, C, dtype=bf)
    mod = torch.zeros(n, 6, C, dtype=bf)
    _raises(lambda: h3.h3_modulate_residual(x, shift=mod[:, 0], scale=mod[:, 1], h_out=x.clone()),
            ValueError, "device memory")
    # gate, shift and scale share the call's one row stride
    _raises(lambda: h3.h3_modulate_residual(x, shift=mod[:, 0], scale=torch.zeros(n, C, dtype=bf),
                                            h_out=x.clone()), ValueError, "one row stride")
    _raises(lambda: h3.h3_modulate_residual(x, shift=mod[:8, 0], scale=mod[:8, 1], h_out=x.clone()),
            ValueError, "addresses (16, 128)")


def test_block_checks(h3):
    C, H, D, F, n = 128, 4, 64, 256, 32
    cfg = h3.block_config(C, H, D, F, (16, 24, 24))
    w = {"w_qkv": torch.zeros(3 * H * D, C, dtype=bf), "w_o": torch.zeros(C, H * D, dtype=bf),
         "w1": torch.zeros(F, C, dtype=bf), "w3": torch.zeros(F, C, dtype=bf),
         "w2": torch.zeros(C, F, dtype=bf), "g_q": torch.zeros(D, dtype=bf), "g_k": torch.zeros(D, dtype=bf)}
    x, mod = torch.zeros(n, C, dtype=bf), torch.zeros(n, 6, C, dtype=bf)
    pos, cu = torch.zeros(n, 4, dtype=torch.int32), torch.tensor([0, n], dtype=torch.int32)
    ws = torch.zeros(16, dtype=torch.uint8)
    run = lambda **kw: h3.h3_dit_block_forward(cfg, {**w, **kw.pop("wd", {})}, kw.pop("x", x),
                                               kw.pop("mod", mod), pos, cu, None, n, ws=ws)
    _raises(run, ValueError, "device memory")
    _raises(lambda: run(mod=torch.zeros(n, 6, 2 * C, dtype=bf)[:, :, :C]), ValueError, "mod must be")
    _raises(lambda: run(mod=torch.zeros(2, 6, C, dtype=bf)), ValueError, "mod must be")
    _raises(lambda: run(wd={"w_o": torch.zeros(H * D, C, dtype=bf)}), ValueError, "w_o")
    _raises(lambda: run(wd={"w1": torch.zeros(F, C, dtype=f32)}), TypeError, "w1")
    _raises(lambda: run(x=torch.zeros(n, C, dtype=f32)), TypeError, "x")


def test_loop_glue_checks(h3):
    z = torch.zeros(64, dtype=bf)
    _raises(lambda: h3.h3_euler_update(z, torch.zeros(64, dtype=bf)), ValueError, "device memory")
    _raises(lambda: h3.h3_euler_update(z, torch.zeros(32, dtype=bf)), ValueError, "u must be")
    _raises(lambda: h3.h3_euler_update(z, torch.zeros(64, dtype=f32)), ValueError, "u must be")
    C, E, nb = 64, 32, 3
    tab, out = torch.zeros(nb, 6, C, dtype=bf), torch.zeros(nb, 6, C, dtype=bf)
    t1, t2 = torch.zeros(C, E, dtype=bf), torch.zeros(6 * C, C, dtype=bf)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    _raises(lambda: h3.h3_timestep_modulation(0.5, t1, t2, tab, out, ws=ws), ValueError, "device memory")
    _raises(lambda: h3.h3_timestep_modulation(0.5, t1, t2[:C], tab, out, ws=ws), ValueError, "w_t2")
    _raises(lambda: h3.h3_timestep_modulation(0.5, t1, t2, tab, out[:2], ws=ws), ValueError, "mod_out")
