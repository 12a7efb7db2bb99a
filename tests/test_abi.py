"""The C-ABI library loads, exports every symbol its header declares, and rejects
bad arguments on the host before touching the GPU (runs without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3dit.h")
LIB = os.path.join(ROOT, "audio_video_diffusion_block_amd", "libh3dit.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libh3dit.so not built")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(h3_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_block_boundary():
    syms = declared_symbols()
    for s in ("h3_qk_norm_rope", "h3_varlen_attn", "h3_modulate_residual", "h3_swiglu",
              "h3_dit_block_forward", "h3_abi_version", "h3_status_string", "h3_last_error"):
        assert s in syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [s for s in declared_symbols() if not hasattr(lib, s)]
    assert not missing, missing
    import audio_video_diffusion_block_amd as h3
    assert set(declared_symbols()) == set(h3.EXPORTED)
    declared = int(re.search(r"#define H3_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert h3.abi_version() == declared
    # the binding's struct mirrors the header's h3_block_io field for field
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{([^}]*)\} h3_block_io;", text).group(1)
    fields = re.findall(r"\b([a-z_0-9]+)\s*;", body)
    assert fields == [f[0] for f in h3.BlockIO._fields_]


def test_status_strings():
    import audio_video_diffusion_block_amd as h3
    assert h3._status_string(0) == "ok"
    assert "workspace" in h3._status_string(3)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails before any launch


def _qk(h3, **kw):
    a = dict(q=FAKE, ld_q=3 * 512, k=FAKE, ld_k=3 * 512, n=10, H=4, D=128, gq=FAKE, gk=FAKE,
             pos=FAKE, st=32, sh=48, sw=48, theta=1e4, eps=1e-6, dt=1)
    a.update(kw)
    return h3._c_qk(a["q"], a["ld_q"], a["k"], a["ld_k"], a["n"], a["H"], a["D"], a["gq"], a["gk"],
                    a["pos"], a["st"], a["sh"], a["sw"], a["theta"], a["eps"], a["dt"], None)


def test_qk_norm_rope_argument_checks():
    import audio_video_diffusion_block_amd as h3
    assert _qk(h3, q=None) == h3.H3_ERR_ARG and "q is NULL" in h3.last_error()
    assert _qk(h3, D=96) == h3.H3_ERR_UNSUPPORTED
    assert _qk(h3, st=30) == h3.H3_ERR_ARG and "sum" in h3.last_error()
    assert _qk(h3, st=31, sh=49) == h3.H3_ERR_ARG and "even" in h3.last_error()
    assert _qk(h3, q=FAKE + 8) == h3.H3_ERR_ARG and "aligned" in h3.last_error()
    assert _qk(h3, ld_q=100) == h3.H3_ERR_ARG
    assert _qk(h3, ld_q=512 + 4) == h3.H3_ERR_ARG and "16 bytes" in h3.last_error()
    assert _qk(h3, dt=7) == h3.H3_ERR_UNSUPPORTED
    assert _qk(h3, n=0, q=None, k=None) == h3.H3_OK  # empty call: nothing to do


def test_attention_argument_checks():
    import audio_video_diffusion_block_amd as h3
    ws_need = h3._c_attn_ws(8192, 8, 128, 3, 1)
    assert ws_need >= 8 * 128 * 8192 * 2

    def call(**kw):
        a = dict(n_buf=8192, H=8, D=128, cu=FAKE, n_seg=3, max_len=4032, ws=FAKE, ws_bytes=ws_need)
        a.update(kw)
        return h3._c_attn(FAKE, 1024, FAKE, 1024, FAKE, 1024, FAKE, 1024, a["n_buf"], a["H"], a["D"],
                          a["cu"], None, a["n_seg"], a["max_len"], 0.0, a["ws"], a["ws_bytes"], 1, None)

    assert call(ws_bytes=ws_need - 1) == h3.H3_ERR_WORKSPACE
    assert call(cu=None) == h3.H3_ERR_ARG
    assert call(n_seg=0) == h3.H3_ERR_ARG
    assert call(max_len=9000) == h3.H3_ERR_ARG
    assert call(D=80) == h3.H3_ERR_UNSUPPORTED
    assert call(ws=None) == h3.H3_ERR_ARG
    # the largest buffer with many segments: a head's transposed V (D rows of
    # round_up(n_buf, 64) + 128 (n_seg + 1) keys) would pass 2^31 bytes, which
    # the kernels address with 32-bit offsets; refused before any launch
    # (only refused calls here: these pointers must never reach a launch)
    big = 1 << 22
    limit = (2 ** 31 - 1) // (128 * 2)  # keys per transposed-V row at D = 128
    first_bad = -(-(limit + 1 - big) // 128) - 1  # smallest n_seg with 128 (n_seg + 1) > limit - n_buf
    for n_seg in (first_bad, 40000, 65535):
        st = call(n_buf=big, n_seg=n_seg, max_len=16, ws_bytes=1 << 40)
        assert st == h3.H3_ERR_ARG and "transposed V" in h3.last_error(), (n_seg, st)


def test_modres_and_linear_argument_checks():
    import audio_video_diffusion_block_amd as h3
    st = h3._c_modres(FAKE, 5120, None, 0, None, None, None, 0, None, 0, 4, 5120, 0, 1e-6, 1, None)
    assert st == h3.H3_ERR_ARG and "nothing to do" in h3.last_error()
    st = h3._c_modres(FAKE, 5120, None, 0, None, FAKE, FAKE, 6 * 5120, FAKE, 5120, 4, 5124, 0, 1e-6, 1, None)
    assert st == h3.H3_ERR_ARG
    st = h3._c_modres(FAKE, 5120, FAKE, 5120, None, None, None, 0, None, 0, 4, 5120, 0, 1e-6, 1, None)
    assert st == h3.H3_ERR_ARG and "gate" in h3.last_error()
    st = h3._c_linear(FAKE, 100, FAKE, 100, FAKE, 64, 10, 64, 100, None, 0, 1, None)
    assert st == h3.H3_ERR_ARG  # k_in not a multiple of 8
    st = h3._c_swiglu(FAKE, 256, FAKE, FAKE, FAKE, FAKE, 256, None, 0, 10, 256, 704, FAKE, 16, 1, None)
    assert st == h3.H3_ERR_WORKSPACE


def test_block_argument_checks():
    import audio_video_diffusion_block_amd as h3
    cfg = h3.block_config(256, 4, 64, 704, (16, 24, 24))
    need = h3.block_workspace_size(cfg, 480, 480, 1)
    assert need >= 480 * (256 + 768) * 2  # h1 and qkv at least
    w = h3.BlockWeights(*([FAKE] * 7))
    io = h3.BlockIO(FAKE, 256, FAKE, 6 * 256, FAKE, FAKE, None, 1, 480, 480, 480, 0, 0, 4, None, None, None)
    st = h3._c_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(io), FAKE, need - 256, None)
    assert st == h3.H3_ERR_WORKSPACE
    bad = h3.block_config(256, 4, 64, 704, (16, 24, 26))
    st = h3._c_block(ctypes.byref(bad), ctypes.byref(w), ctypes.byref(io), FAKE, need, None)
    assert st == h3.H3_ERR_ARG
    io2 = h3.BlockIO(FAKE, 256, FAKE, 6 * 256, FAKE, FAKE, None, 1, 480, 480, 512, 0, 0, 4, None, None, None)
    st = h3._c_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(io2), FAKE, need, None)
    assert st == h3.H3_ERR_ARG and "world-1" in h3.last_error()
    f8 = h3.block_config(256, 4, 64, 704, (16, 24, 24), attn_fp8=True)
    assert h3.block_workspace_size(f8, 480, 480, 1) != need
    import torch
    f8_f32 = h3.block_config(256, 4, 64, 704, (16, 24, 24), dtype=torch.float32, attn_fp8=True)
    st = h3._c_block(ctypes.byref(f8_f32), ctypes.byref(w), ctypes.byref(io), FAKE, 1 << 30, None)
    assert st == h3.H3_ERR_ARG and "bf16" in h3.last_error()
    f8.attn_fp8 = 2
    st = h3._c_block(ctypes.byref(f8), ctypes.byref(w), ctypes.byref(io), FAKE, 1 << 30, None)
    assert st == h3.H3_ERR_ARG and "attn_fp8" in h3.last_error()
    io3 = h3.BlockIO(FAKE, 256, FAKE, 6 * 256, FAKE, FAKE, None, 1, 480, 120, 480, 400, 3, 1, FAKE, FAKE, FAKE)
    st = h3._c_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(io3), FAKE, need, None)
    assert st == h3.H3_ERR_ARG and "local rows" in h3.last_error()
    # ffn_dim and n_heads*head_dim become GEMM widths and row strides: at most 2^22
    for big in (h3.block_config(256, 4, 64, (1 << 22) + 8, (16, 24, 24)),
                h3.block_config(256, (1 << 22) // 64 + 1, 64, 704, (16, 24, 24))):
        st = h3._c_block(ctypes.byref(big), ctypes.byref(w), ctypes.byref(io), FAKE, 1 << 40, None)
        assert st == h3.H3_ERR_ARG and "2^22" in h3.last_error()


def test_frames_argument_checks():
    import audio_video_diffusion_block_amd as h3
    st = h3._c_frames(FAKE, 1, 2, 4, 16, FAKE + (1 << 20), 2, None)
    assert st == h3.H3_ERR_ARG and "layout" in h3.last_error()
    st = h3._c_frames(FAKE, 1, 2, 4, 16, FAKE + 8 + (1 << 20), 0, None)
    assert st == h3.H3_ERR_ARG and "aligned" in h3.last_error()
    st = h3._c_frames(FAKE, 1, 2, 4, 16, FAKE + 64, 0, None)
    assert st == h3.H3_ERR_ARG and "overlap" in h3.last_error()
    st = h3._c_frames(FAKE, -1, 2, 4, 16, FAKE + (1 << 20), 0, None)
    assert st == h3.H3_ERR_ARG
    assert h3._c_frames(None, 1, 0, 4, 16, None, 0, None) == h3.H3_OK  # empty: nothing launched


def test_peer_major_layout_argument_checks():
    import audio_video_diffusion_block_amd as h3
    cfg = h3.BlockConfig(256, 4, 64, 704, 16, 24, 24, 1e4, 1e-6, 1e-6, 0, h3.H3_BF16)
    w = h3.BlockWeights(*([FAKE] * 7))

    def io(**kw):
        base = dict(x=FAKE, ld_x=256, mod=FAKE, ld_mod=0, pos=FAKE, cu_slots=FAKE, valid_len=FAKE,
                    n_seg=1, max_valid_len=64, n_tok_local=16, n_buf=64, tok_begin=32,
                    head_begin=2, head_count=1, qkv_attn=FAKE, o_attn=FAKE, o_local=None,
                    qkv_send=FAKE, o_recv=FAKE)
        base.update(kw)
        return h3.BlockIO(**base)

    ws = h3.block_workspace_size(cfg, 16, 64, 1)

    def run(i, c=cfg):
        return h3._c_block(ctypes.byref(c), ctypes.byref(w), ctypes.byref(i), FAKE, ws, None)

    assert run(io(tok_begin=16)) == h3.H3_ERR_ARG and "tok_begin" in h3.last_error()
    assert run(io(o_recv=None)) == h3.H3_ERR_ARG and "o_recv" in h3.last_error()
    assert run(io(qkv_attn=None, n_buf=16, tok_begin=0, head_begin=0, head_count=4)) == h3.H3_ERR_ARG
    f32 = h3.BlockConfig(256, 4, 64, 704, 16, 24, 24, 1e4, 1e-6, 1e-6, 0, h3.H3_F32)
    assert run(io(), f32) == h3.H3_ERR_ARG and "bf16" in h3.last_error()



def test_fp8_projection_argument_checks():
    import audio_video_diffusion_block_amd as h3
    M = h3.MxOperand
    # quantize: bf16 only, cols a multiple of 32, padded row length
    assert h3._c_mxq(FAKE, 256, 10, 256, FAKE, 256, FAKE, 8, h3.H3_F32, None) == h3.H3_ERR_UNSUPPORTED
    st = h3._c_mxq(FAKE, 256, 10, 200, FAKE, 256, FAKE, 8, h3.H3_BF16, None)
    assert st == h3.H3_ERR_ARG and "32" in h3.last_error()
    st = h3._c_mxq(FAKE, 704, 10, 704, FAKE, 704, FAKE, 24, h3.H3_BF16, None)
    assert st == h3.H3_ERR_ARG and "ld" in h3.last_error()  # needs round_up(704, 128) = 768
    st = h3._c_mxq(FAKE, 704, 10, 704, FAKE, 768, FAKE, 22, h3.H3_BF16, None)
    assert st == h3.H3_ERR_ARG and "ld_scale" in h3.last_error()
    assert h3._c_mxq(None, 704, 0, 704, None, 768, None, 24, h3.H3_BF16, None) == h3.H3_OK
    # linear: k a multiple of 32; scale alignment and stride
    a = M(FAKE, 256, FAKE, 8)
    w = M(FAKE, 256, FAKE, 8)
    st = h3._c_lin8(ctypes.byref(a), ctypes.byref(w), FAKE, 64, 10, 64, 250, None, 0, None)
    assert st == h3.H3_ERR_ARG
    bad = M(FAKE, 256, FAKE + 2, 8)
    st = h3._c_lin8(ctypes.byref(bad), ctypes.byref(w), FAKE, 64, 10, 64, 256, None, 0, None)
    assert st == h3.H3_ERR_ARG and "scale" in h3.last_error()
    bad = M(FAKE, 256, FAKE, 6)
    st = h3._c_lin8(ctypes.byref(a), ctypes.byref(bad), FAKE, 64, 10, 64, 256, None, 0, None)
    assert st == h3.H3_ERR_ARG and "ld_scale" in h3.last_error()
    bad = M(FAKE + 8, 256, FAKE, 8)
    st = h3._c_lin8(ctypes.byref(bad), ctypes.byref(w), FAKE, 64, 10, 64, 256, None, 0, None)
    assert st == h3.H3_ERR_ARG and "aligned" in h3.last_error()
    # swiglu: w1 and w3 share strides; workspace size
    h = M(FAKE, 256, FAKE, 8)
    w13 = M(FAKE, 256, FAKE, 8)
    w3b = M(FAKE, 384, FAKE, 12)
    w2 = M(FAKE, 768, FAKE, 24)
    args = lambda w3_, ws: [ctypes.byref(h), ctypes.byref(w13), ctypes.byref(w3_), ctypes.byref(w2),
                            FAKE, 256, None, 0, 10, 256, 704, FAKE, ws, None]
    st = h3._c_sw8(*args(w3b, 1 << 30))
    assert st == h3.H3_ERR_ARG and "share" in h3.last_error()
    need = h3._c_sw8_ws(10, 704)
    assert need >= 10 * 704 * 2 + 10 * 768 + 10 * 24
    st = h3._c_sw8(*args(w13, need - 16))
    assert st == h3.H3_ERR_WORKSPACE


def _struct_fields(name):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{([^}]*)\} " + name + ";", text).group(1)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        first, *rest = decl.split(",")
        names.append(re.findall(r"[A-Za-z_0-9]+", first)[-1])
        names += [r.strip() for r in rest]
    return names


def test_binding_structs_mirror_the_header():
    import audio_video_diffusion_block_amd as h3
    for name, cls in (("h3_block_config", h3.BlockConfig), ("h3_block_weights", h3.BlockWeights),
                      ("h3_block_io", h3.BlockIO), ("h3_mx_operand", h3.MxOperand)):
        assert _struct_fields(name) == [f[0] for f in cls._fields_], name


def test_block_gemm_fp8_argument_checks():
    import audio_video_diffusion_block_amd as h3
    import torch
    w = h3.BlockWeights(*([FAKE] * 7))
    io = h3.BlockIO(FAKE, 256, FAKE, 6 * 256, FAKE, FAKE, None, 1, 480, 480, 480, 0, 0, 4, None, None, None)
    cfg = h3.block_config(256, 4, 64, 704, (16, 24, 24), gemm_fp8=True)
    need = h3.block_workspace_size(cfg, 480, 480, 1)
    assert need != h3.block_workspace_size(h3.block_config(256, 4, 64, 704, (16, 24, 24)), 480, 480, 1)
    st = h3._c_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(io), FAKE, need, None)
    assert st == h3.H3_ERR_ARG and "weights.mx" in h3.last_error()
    f32 = h3.block_config(256, 4, 64, 704, (16, 24, 24), dtype=torch.float32, gemm_fp8=True)
    st = h3._c_block(ctypes.byref(f32), ctypes.byref(w), ctypes.byref(io), FAKE, 1 << 30, None)
    assert st == h3.H3_ERR_ARG and "bf16" in h3.last_error()
    mx = (h3.MxOperand * 5)(h3.MxOperand(FAKE, 256, FAKE, 8), h3.MxOperand(FAKE, 256, FAKE, 8),
                            h3.MxOperand(FAKE, 256, FAKE, 8), h3.MxOperand(FAKE, 384, FAKE, 12),
                            h3.MxOperand(FAKE, 768, FAKE, 24))
    w.mx = ctypes.cast(mx, ctypes.POINTER(h3.MxOperand))
    st = h3._c_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(io), FAKE, need, None)
    assert st == h3.H3_ERR_ARG and "share" in h3.last_error()  # w1 / w3 strides differ


def test_skip_softmax_argument_checks():
    import audio_video_diffusion_block_amd as h3
    args = lambda t, dt: (FAKE, 256, FAKE, 256, FAKE, 256, FAKE, 256, 64, 4, 64, FAKE, None, 1, 64,
                          0.0, t, FAKE, 1 << 20, dt, None)
    assert h3._c_attn_skip(*args(-10.0, h3.H3_F32)) == h3.H3_ERR_UNSUPPORTED
    assert h3._c_attn_skip(*args(0.0, h3.H3_BF16)) == h3.H3_ERR_ARG
    assert "negative" in h3.last_error()
    assert h3._c_attn_skip(*args(float("nan"), h3.H3_BF16)) == h3.H3_ERR_ARG


def test_block_skip_softmax_argument_checks():
    import torch
    import audio_video_diffusion_block_amd as h3
    w = h3.BlockWeights(*([FAKE] * 7))
    io = h3.BlockIO(FAKE, 256, FAKE, 6 * 256, FAKE, FAKE, None, 1, 480, 480, 480, 0, 0, 4, None, None, None)
    cases = [(dict(attn_skip_log2=1.0), "attn_skip_log2"),
             (dict(attn_skip_log2=float("nan")), "attn_skip_log2"),
             (dict(attn_skip_log2=-3.0, dtype=torch.float32), "bf16")]
    for kw, word in cases:
        cfg = h3.block_config(256, 4, 64, 704, (16, 24, 24), **kw)
        st = h3._c_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(io), FAKE, 1 << 30, None)
        assert st == h3.H3_ERR_ARG and word in h3.last_error(), (kw, h3.last_error())
    # the option leaves the workspace size unchanged (the exact kernel's workspace)
    on = h3.block_config(256, 4, 64, 704, (16, 24, 24), attn_skip_log2=-3.0)
    off = h3.block_config(256, 4, 64, 704, (16, 24, 24))
    assert h3.block_workspace_size(on, 480, 480, 1) == h3.block_workspace_size(off, 480, 480, 1)


def test_fp8_skip_softmax_argument_checks():
    import audio_video_diffusion_block_amd as h3
    args = lambda t, dt: (FAKE, 256, FAKE, 256, FAKE, 256, FAKE, 256, 64, 4, 64, FAKE, None, 1, 64,
                          0.0, t, FAKE, 1 << 24, dt, None)
    assert h3._c_attn8_skip(*args(-10.0, h3.H3_F32)) == h3.H3_ERR_UNSUPPORTED
    assert h3._c_attn8_skip(*args(0.0, h3.H3_BF16)) == h3.H3_ERR_ARG
    assert "negative" in h3.last_error()
    assert h3._c_attn8_skip(*args(float("nan"), h3.H3_BF16)) == h3.H3_ERR_ARG


def test_check_segments_rules():
    """The host segment checker accepts well-formed metadata and names each rule it rejects."""
    import numpy as np
    import audio_video_diffusion_block_amd as h3
    ok = dict(cu_slots=[0, 4032, 5600, 5700], valid_len=[4032, 1500, 17], n_buf=8192, max_valid_len=4032)
    h3.h3_check_segments(**ok)
    h3.h3_check_segments([0, 10, 10, 30], None, 30, 20)         # empty slot, full slots
    h3.h3_check_segments(np.array([0, 64]), np.array([0]), 64, 0)  # zero valid rows
    bad = [
        (dict(ok, cu_slots=[-1, 4032, 5600, 5700]), "negative"),
        (dict(ok, cu_slots=[0, 5600, 4032, 5700]), "decreases"),
        (dict(ok, cu_slots=[0, 4032, 5600, 8193]), "exceeds n_buf"),
        (dict(ok, valid_len=[4033, 1500, 17]), "outside"),
        (dict(ok, valid_len=[4032, -1, 17]), "outside"),
        (dict(ok, max_valid_len=4031), "max_valid_len"),
        (dict(ok, cu_slots=[0, 70], valid_len=None, n_buf=70, max_valid_len=64), "max_valid_len"),
    ]
    for args, word in bad:
        with pytest.raises(h3.H3Error) as ei:
            h3.h3_check_segments(**args)
        assert ei.value.status == h3.H3_ERR_ARG and word in str(ei.value), (args, str(ei.value))
    assert h3._c_check_segments(None, None, 1, 10, 10) == h3.H3_ERR_ARG
    cu = np.array([0, 10], dtype=np.int32)
    assert h3._c_check_segments(cu.ctypes.data, None, 0, 10, 10) == h3.H3_ERR_ARG


def test_modulate_mx_argument_checks():
    """The modulated norm to an MX operand: dim a multiple of 128, operand strides, pointers."""
    import audio_video_diffusion_block_amd as h3
    # x, ld_x, shift, scale, ld_mod, q, ld_q, q_scale, ld_scale, n, dim, norm_kind, eps, stream
    ok = [FAKE, 256, FAKE, FAKE, 6 * 256, FAKE, 256, FAKE, 8, 10, 256, 0, 1e-6, None]

    def call(**kw):
        a = list(ok)
        names = ["x", "ld_x", "shift", "scale", "ld_mod", "q", "ld_q", "qs", "ld_s", "n", "dim", "nk", "eps", "st"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return h3._c_modmx(*a)

    st = call(dim=192, ld_x=192, ld_q=256)
    assert st == h3.H3_ERR_ARG and "128" in h3.last_error()
    assert call(ld_q=128) == h3.H3_ERR_ARG and "ld" in h3.last_error()
    assert call(ld_s=6) == h3.H3_ERR_ARG and "ld_scale" in h3.last_error()
    assert call(q=None) == h3.H3_ERR_ARG
    assert call(shift=None) == h3.H3_ERR_ARG
    assert call(nk=2) == h3.H3_ERR_ARG
    assert call(x=FAKE + 8) == h3.H3_ERR_ARG
    assert call(n=0, x=None, q=None) == h3.H3_OK


def test_noalloc_attention_argument_checks():
    """The no-allocation attention validates like h3_varlen_attn and refuses, on
    the host, a call whose transposed v exceeds its fixed scratch."""
    import audio_video_diffusion_block_amd as h3

    def call(n_buf=8192, H=8, D=128, q=FAKE, n_seg=3, dt=1):
        return h3._c_attn_na(q, H * D, FAKE, H * D, FAKE, H * D, FAKE, H * D, n_buf, H, D, FAKE,
                             None, n_seg, min(n_buf, 4032), 0.0, dt, None)
    assert call(q=None) == h3.H3_ERR_ARG and "q is NULL" in h3.last_error()
    assert call(D=96) == h3.H3_ERR_UNSUPPORTED
    big = h3.NOALLOC_SCRATCH_BYTES // (8 * 128 * 2) + 64
    assert call(n_buf=big) == h3.H3_ERR_WORKSPACE and "scratch" in h3.last_error()
    assert call(n_buf=0) == h3.H3_OK                     # empty call: nothing to do


def test_block_workspace_size_by_head_slice():
    """The size query: a rank share's workspace follows its head slice, 0 covers
    world 1 and every share, and the forward refuses 256 bytes less than the
    query for the mode it runs in."""
    import audio_video_diffusion_block_amd as h3
    for kw in ({}, dict(attn_fp8=True), dict(gemm_fp8=True), dict(attn_fp8=True, gemm_fp8=True)):
        cfg = h3.block_config(256, 8, 64, 768, (16, 24, 24), **kw)
        n, n_buf = 480, 3840
        sizes = [h3.block_workspace_size(cfg, n, n_buf, 1, hc) for hc in (1, 2, 4, 8)]
        assert all(a < b for a, b in zip(sizes, sizes[1:])), (kw, sizes)
        anyc = h3.block_workspace_size(cfg, n, n_buf, 1)
        assert anyc >= sizes[-1] and anyc >= h3.block_workspace_size(cfg, n, n, 1), kw
        assert h3.block_workspace_size(cfg, n, n_buf, 1, -1) == 0
        # a share with 2 of 8 heads: refused 256 bytes short of its own size
        w = h3.BlockWeights(*([FAKE] * 7))
        if kw.get("gemm_fp8"):
            mx = (h3.MxOperand * 5)(h3.MxOperand(FAKE, 256, FAKE, 8), h3.MxOperand(FAKE, 512, FAKE, 16),
                                    h3.MxOperand(FAKE, 256, FAKE, 8), h3.MxOperand(FAKE, 256, FAKE, 8),
                                    h3.MxOperand(FAKE, 768, FAKE, 24))
            w.mx = ctypes.cast(mx, ctypes.POINTER(h3.MxOperand))
        io = h3.BlockIO(FAKE, 256, FAKE, 6 * 256, FAKE, FAKE, None, 1, n_buf, n, n_buf, 0, 2, 2,
                        FAKE, FAKE, FAKE)
        st = h3._c_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(io), FAKE, sizes[1] - 256, None)
        assert st == h3.H3_ERR_WORKSPACE, (kw, h3.last_error())


def test_block_workspace_stages_share_bytes():
    """qkv, the attention workspace and o are dead before the SwiGLU writes g:
    the workspace is the larger stage, not the sum (bf16, world 1)."""
    import audio_video_diffusion_block_amd as h3
    C, H, D, F, n = 256, 4, 64, 2048, 1024
    cfg = h3.block_config(C, H, D, F, (16, 24, 24))
    need = h3.block_workspace_size(cfg, n, n, 1, 0)
    h1, qkv, o, g = n * C * 2, n * 3 * H * D * 2, n * H * D * 2, n * F * 2
    assert g > qkv + o  # the FFN stage is the larger one here
    assert need < h1 + qkv + o + g
    assert need >= h1 + g
