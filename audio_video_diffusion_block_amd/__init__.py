"""Python binding of libh3dit.so: one DiT block forward on a packed
audio-video token sequence, hand-written HIP for MI355X (gfx950).

Argument marshalling only.  Every function takes torch tensors that already
live in device memory (torch is the allocator and the stream provider) and
passes raw pointers, strides and sizes to the C ABI declared in
``include/h3dit.h``; all arithmetic happens in the library's kernels.  There
is no CPU fallback: if the library is missing, importing the binding raises.

Names mirror the C entry points (``h3_qk_norm_rope`` ...); tensors' row
strides are taken from the tensors themselves.  Since the C ABI sees only
pointers and sizes, each entry first checks every tensor against the call:
its dtype, that it holds at least the rows and columns the call addresses,
contiguous columns (dense layout for operands passed as bare pointers), int32
segment and position metadata; a mismatch raises ValueError or TypeError
before anything reaches the library.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libh3dit.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python audio_video_diffusion_block_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

H3_OK, H3_ERR_ARG, H3_ERR_UNSUPPORTED, H3_ERR_WORKSPACE, H3_ERR_HIP = range(5)
H3_F32, H3_BF16 = 0, 1
POS_VIDEO, POS_AUDIO, POS_PAD = 0, 1, 2

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f = ctypes.c_float
_sz = ctypes.c_size_t


class H3Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"h3dit status {status} ({_status_string(status)}): {detail}")
        self.status = status


class BlockConfig(ctypes.Structure):
    _fields_ = [("dim", _i32), ("n_heads", _i32), ("head_dim", _i32), ("ffn_dim", _i32),
                ("sec_t", _i32), ("sec_h", _i32), ("sec_w", _i32), ("theta", _f),
                ("eps_qk", _f), ("eps_mod", _f), ("norm_kind", _i32), ("dtype", _i32),
                ("attn_fp8", _i32), ("gemm_fp8", _i32), ("attn_skip_log2", _f)]


class MxOperand(ctypes.Structure):
    _fields_ = [("data", _p), ("ld", _i64), ("scale", _p), ("ld_scale", _i64)]


class BlockWeights(ctypes.Structure):
    _fields_ = [("w_qkv", _p), ("w_o", _p), ("w1", _p), ("w3", _p), ("w2", _p), ("g_q", _p),
                ("g_k", _p), ("mx", ctypes.POINTER(MxOperand))]


class BlockIO(ctypes.Structure):
    _fields_ = [("x", _p), ("ld_x", _i64), ("mod", _p), ("ld_mod", _i64), ("pos", _p),
                ("cu_slots", _p), ("valid_len", _p), ("n_seg", _i32), ("max_valid_len", _i32),
                ("n_tok_local", _i64), ("n_buf", _i64), ("tok_begin", _i64),
                ("head_begin", _i32), ("head_count", _i32), ("qkv_attn", _p), ("o_attn", _p),
                ("o_local", _p), ("qkv_send", _p), ("o_recv", _p)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_lib.h3_abi_version.restype = ctypes.c_int
# the ctypes structures below mirror this version of include/h3dit.h
ABI_VERSION = 7
if _lib.h3_abi_version() != ABI_VERSION:
    raise ImportError(f"{LIB_PATH} has ABI version {_lib.h3_abi_version()}, the binding "
                      f"expects {ABI_VERSION}: rebuild it")
_lib.h3_status_string.restype = ctypes.c_char_p
_lib.h3_status_string.argtypes = [ctypes.c_int]
_lib.h3_last_error.restype = ctypes.c_char_p

_c_qk = _sig("h3_qk_norm_rope", ctypes.c_int,
             [_p, _i64, _p, _i64, _i64, _i32, _i32, _p, _p, _p, _i32, _i32, _i32, _f, _f, _i32, _p])
_c_attn_ws = _sig("h3_varlen_attn_workspace_size", _sz, [_i64, _i32, _i32, _i32, _i32])
_c_attn = _sig("h3_varlen_attn", ctypes.c_int,
               [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i32, _i32, _p, _p, _i32, _i32, _f,
                _p, _sz, _i32, _p])
_c_attn_na = _sig("h3_varlen_attn_noalloc", ctypes.c_int,
                  [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i32, _i32, _p, _p, _i32, _i32, _f,
                   _i32, _p])
_c_modres = _sig("h3_modulate_residual", ctypes.c_int,
                 [_p, _i64, _p, _i64, _p, _p, _p, _i64, _p, _i64, _i64, _i32, _i32, _f, _i32, _p])
_c_linear = _sig("h3_linear", ctypes.c_int,
                 [_p, _i64, _p, _i64, _p, _i64, _i64, _i32, _i32, _p, _i64, _i32, _p])
_c_swiglu_ws = _sig("h3_swiglu_workspace_size", _sz, [_i64, _i32, _i32])
_c_swiglu = _sig("h3_swiglu", ctypes.c_int,
                 [_p, _i64, _p, _p, _p, _p, _i64, _p, _i64, _i64, _i32, _i32, _p, _sz, _i32, _p])
_c_block_ws = _sig("h3_dit_block_workspace_size", _sz,
                   [ctypes.POINTER(BlockConfig), _i64, _i64, _i32, _i32])
_c_block = _sig("h3_dit_block_forward", ctypes.c_int,
                [ctypes.POINTER(BlockConfig), ctypes.POINTER(BlockWeights), ctypes.POINTER(BlockIO),
                 _p, _sz, _p])
_c_temb_ws = _sig("h3_timestep_workspace_size", _sz, [_i32])
_c_temb = _sig("h3_timestep_modulation", ctypes.c_int,
               [_f, _p, _p, _p, _p, _i32, _i32, _i32, _p, _sz, _i32, _p])
_c_euler = _sig("h3_euler_update", ctypes.c_int, [_p, _p, _p, _i64, _f, _f, _i32, _p])
_c_frames = _sig("h3_frames_to_u8", ctypes.c_int, [_p, _i64, _i64, _i64, _i64, _p, _i32, _p])
_c_attn8_ws = _sig("h3_varlen_attn_fp8_workspace_size", _sz, [_i64, _i32, _i32, _i32])
_c_attn8 = _sig("h3_varlen_attn_fp8", ctypes.c_int,
                [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i32, _i32, _p, _p, _i32, _i32, _f,
                 _p, _sz, _i32, _p])

_c_attn_skip = _sig("h3_varlen_attn_skip", ctypes.c_int,
                    [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i32, _i32, _p, _p, _i32, _i32,
                     _f, _f, _p, _sz, _i32, _p])
_c_attn8_skip = _sig("h3_varlen_attn_fp8_skip", ctypes.c_int,
                     [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i32, _i32, _p, _p, _i32, _i32,
                      _f, _f, _p, _sz, _i32, _p])
_c_check_segments = _sig("h3_check_segments", ctypes.c_int, [_p, _p, _i32, _i64, _i32])
_c_modmx = _sig("h3_modulate_mx", ctypes.c_int,
                [_p, _i64, _p, _p, _i64, _p, _i64, _p, _i64, _i64, _i32, _i32, _f, _p])
_c_mxq = _sig("h3_mx_quantize", ctypes.c_int,
              [_p, _i64, _i64, _i32, _p, _i64, _p, _i64, _i32, _p])
_c_lin8 = _sig("h3_linear_fp8", ctypes.c_int,
               [ctypes.POINTER(MxOperand), ctypes.POINTER(MxOperand), _p, _i64, _i64, _i32, _i32,
                _p, _i64, _p])
_c_sw8_ws = _sig("h3_swiglu_fp8_workspace_size", _sz, [_i64, _i32])
_c_sw8 = _sig("h3_swiglu_fp8", ctypes.c_int,
              [ctypes.POINTER(MxOperand)] * 4 + [_p, _i64, _p, _i64, _i64, _i32, _i32, _p, _sz, _p])

EXPORTED = ("h3_abi_version", "h3_status_string", "h3_last_error", "h3_qk_norm_rope",
            "h3_varlen_attn_workspace_size", "h3_varlen_attn", "h3_modulate_residual",
            "h3_linear", "h3_swiglu_workspace_size", "h3_swiglu", "h3_dit_block_workspace_size",
            "h3_dit_block_forward", "h3_timestep_workspace_size", "h3_timestep_modulation",
            "h3_euler_update", "h3_frames_to_u8", "h3_varlen_attn_fp8_workspace_size",
            "h3_varlen_attn_fp8", "h3_mx_quantize", "h3_linear_fp8", "h3_swiglu_fp8_workspace_size",
            "h3_swiglu_fp8", "h3_varlen_attn_skip", "h3_varlen_attn_fp8_skip",
            "h3_check_segments", "h3_modulate_mx", "h3_varlen_attn_noalloc")


def _status_string(st: int) -> str:
    return _lib.h3_status_string(st).decode()


def last_error() -> str:
    return _lib.h3_last_error().decode()


def abi_version() -> int:
    return _lib.h3_abi_version()


def _check(st: int):
    if st != H3_OK:
        raise H3Error(st, last_error())


# --------------------------------------------------------------- marshalling

def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return H3_BF16
    if t.dtype == torch.float32:
        return H3_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError("tensors must live in device memory")
    return t.data_ptr()


def _ld(t: torch.Tensor) -> int:
    """Row stride (elements) of a 2-D view whose rows may be strided, columns contiguous."""
    if t.dim() == 1:
        return t.shape[0]
    if t.stride(-1) != 1:
        raise ValueError("innermost dimension must be contiguous")
    return t.stride(0)


# Tensor metadata checks.  The C ABI sees pointers and sizes only, so the
# binding checks that every tensor holds what the call will touch: the call's
# dtype, at least the rows and columns it addresses (views of larger buffers
# are fine), contiguous columns.  They raise before any pointer is taken (the
# device check comes with the pointer).
_TDT = {H3_BF16: torch.bfloat16, H3_F32: torch.float32}


def _mat(t, name: str, rows: int, cols: int, dtype: torch.dtype):
    """t: 2-D view of at least rows x cols elements of dtype, columns contiguous."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} is {t.dtype}; this call needs {dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} has shape {tuple(t.shape)}; the call addresses ({rows}, {cols})")
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: columns must be contiguous")


def _dense(t, name: str, shape: tuple, dtype: torch.dtype):
    """t: a contiguous tensor of exactly `shape` (passed to the library as a bare pointer)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} is {t.dtype}; this call needs {dtype}")
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor of shape {tuple(shape)}, "
                         f"got {tuple(t.shape)}{'' if t.is_contiguous() else ' (strided)'}")


def _ints(t, name: str, n: int):
    """t: contiguous int32 tensor of at least n elements."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name} must be a contiguous int32 tensor of >= {n} elements, "
                         f"got {t.dtype} {tuple(t.shape)}")


def _gate_rows(gate, ld_gate, m: int) -> int:
    """Rows a gate view must hold: 1 when broadcast (ld_gate 0), else m."""
    if ld_gate not in (0, None) and ld_gate != _ld(gate):
        raise ValueError("ld_gate must be 0 (broadcast) or the gate's own row stride")
    return 1 if (ld_gate == 0 or (ld_gate is None and gate.shape[0] == 1)) else m


def _segments(cu_slots, valid_len) -> int:
    """n_seg from cu_slots [n_seg + 1]; checks both are int32 device metadata."""
    if cu_slots is None or cu_slots.dim() != 1 or cu_slots.numel() < 2:
        raise ValueError("cu_slots must be a 1-D int32 tensor of n_seg + 1 >= 2 entries")
    n_seg = cu_slots.shape[0] - 1
    _ints(cu_slots, "cu_slots", n_seg + 1)
    if valid_len is not None:
        _ints(valid_len, "valid_len", n_seg)
    return n_seg


def _attn_operands(q, k, v, o, n_heads: int, head_dim: int, dtype=None) -> int:
    """q, k, v, o: [n_buf, >= n_heads*head_dim] views of one dtype; returns n_buf."""
    n_buf, width = q.shape[0], n_heads * head_dim
    dtype = dtype or q.dtype
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _mat(t, name, n_buf, width, dtype)
    return n_buf


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _bytes_ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entries

def h3_qk_norm_rope(q: torch.Tensor, k: torch.Tensor, n_heads: int, head_dim: int,
                    g_q: torch.Tensor, g_k: torch.Tensor, pos: torch.Tensor,
                    sections: Sequence[int], theta: float = 1e4, eps: float = 1e-6, stream=None):
    """In place on q, k (views [n_tok, >= H*D] with row strides)."""
    n = q.shape[0]
    _mat(q, "q", n, n_heads * head_dim, q.dtype)
    _mat(k, "k", n, n_heads * head_dim, q.dtype)
    _dense(g_q, "g_q", (head_dim,), q.dtype)
    _dense(g_k, "g_k", (head_dim,), q.dtype)
    _ints(pos, "pos", 4 * n)
    _check(_c_qk(_ptr(q), _ld(q), _ptr(k), _ld(k), q.shape[0], n_heads, head_dim, _ptr(g_q),
                 _ptr(g_k), _ptr(pos), sections[0], sections[1], sections[2], theta, eps, _dt(q),
                 _stream(stream)))


def varlen_attn_workspace_size(n_buf: int, n_heads: int, head_dim: int, n_seg: int, dtype) -> int:
    return _c_attn_ws(n_buf, n_heads, head_dim, n_seg, H3_BF16 if dtype == torch.bfloat16 else H3_F32)


def h3_varlen_attn(q, k, v, o, n_heads: int, head_dim: int, cu_slots: torch.Tensor,
                   valid_len: Optional[torch.Tensor], max_valid_len: int,
                   softmax_scale: float = 0.0, ws: Optional[torch.Tensor] = None, stream=None):
    n_buf = _attn_operands(q, k, v, o, n_heads, head_dim)
    n_seg = _segments(cu_slots, valid_len)
    need = varlen_attn_workspace_size(n_buf, n_heads, head_dim, n_seg, q.dtype)
    if ws is None:
        ws = _bytes_ws(need, q.device)
    _check(_c_attn(_ptr(q), _ld(q), _ptr(k), _ld(k), _ptr(v), _ld(v), _ptr(o), _ld(o), n_buf,
                   n_heads, head_dim, _ptr(cu_slots), _ptr(valid_len), n_seg, max_valid_len,
                   softmax_scale, _ptr(ws), ws.numel() * ws.element_size(), _dt(q),
                   _stream(stream)))


def h3_varlen_attn_noalloc(q, k, v, o, n_heads: int, head_dim: int, cu_slots: torch.Tensor,
                           valid_len: Optional[torch.Tensor], max_valid_len: int,
                           softmax_scale: float = 0.0, stream=None):
    """h3_varlen_attn with the library's own fixed scratch (no workspace, no
    allocation; NOALLOC_SCRATCH_BYTES per device, shared by every call)."""
    n_buf = _attn_operands(q, k, v, o, n_heads, head_dim)
    n_seg = _segments(cu_slots, valid_len)
    _check(_c_attn_na(_ptr(q), _ld(q), _ptr(k), _ld(k), _ptr(v), _ld(v), _ptr(o), _ld(o), n_buf,
                      n_heads, head_dim, _ptr(cu_slots), _ptr(valid_len), n_seg, max_valid_len,
                      softmax_scale, _dt(q), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20


def h3_varlen_attn_skip(q, k, v, o, n_heads: int, head_dim: int, cu_slots, valid_len,
                        max_valid_len: int, skip_log2: float, softmax_scale: float = 0.0,
                        ws: Optional[torch.Tensor] = None, stream=None):
    """bf16 attention with Skip-Softmax: key blocks of 64 whose scores are all
    more than |skip_log2| (log2 units) below a query group's running max are
    skipped (workspace as h3_varlen_attn)."""
    n_buf = _attn_operands(q, k, v, o, n_heads, head_dim)
    n_seg = _segments(cu_slots, valid_len)
    if ws is None:
        ws = _bytes_ws(varlen_attn_workspace_size(n_buf, n_heads, head_dim, n_seg, q.dtype), q.device)
    _check(_c_attn_skip(_ptr(q), _ld(q), _ptr(k), _ld(k), _ptr(v), _ld(v), _ptr(o), _ld(o), n_buf,
                        n_heads, head_dim, _ptr(cu_slots), _ptr(valid_len), n_seg, max_valid_len,
                        softmax_scale, skip_log2, _ptr(ws), ws.numel() * ws.element_size(), _dt(q),
                        _stream(stream)))


def varlen_attn_fp8_workspace_size(n_buf: int, n_heads: int, head_dim: int, n_seg: int) -> int:
    return _c_attn8_ws(n_buf, n_heads, head_dim, n_seg)


def h3_varlen_attn_fp8(q, k, v, o, n_heads: int, head_dim: int, cu_slots: torch.Tensor,
                       valid_len: Optional[torch.Tensor], max_valid_len: int,
                       softmax_scale: float = 0.0, ws: Optional[torch.Tensor] = None, stream=None):
    """h3_varlen_attn with MX-scaled e4m3 operands (bf16 in, bf16 out)."""
    n_buf = _attn_operands(q, k, v, o, n_heads, head_dim, torch.bfloat16)
    n_seg = _segments(cu_slots, valid_len)
    need = varlen_attn_fp8_workspace_size(n_buf, n_heads, head_dim, n_seg)
    if ws is None:
        ws = _bytes_ws(need, q.device)
    _check(_c_attn8(_ptr(q), _ld(q), _ptr(k), _ld(k), _ptr(v), _ld(v), _ptr(o), _ld(o), n_buf,
                    n_heads, head_dim, _ptr(cu_slots), _ptr(valid_len), n_seg, max_valid_len,
                    softmax_scale, _ptr(ws), ws.numel() * ws.element_size(), _dt(q),
                    _stream(stream)))


def h3_varlen_attn_fp8_skip(q, k, v, o, n_heads: int, head_dim: int, cu_slots, valid_len,
                            max_valid_len: int, skip_log2: float, softmax_scale: float = 0.0,
                            ws: Optional[torch.Tensor] = None, stream=None):
    """h3_varlen_attn_fp8 with the Skip-Softmax rule of h3_varlen_attn_skip."""
    n_buf = _attn_operands(q, k, v, o, n_heads, head_dim, torch.bfloat16)
    n_seg = _segments(cu_slots, valid_len)
    if ws is None:
        ws = _bytes_ws(varlen_attn_fp8_workspace_size(n_buf, n_heads, head_dim, n_seg), q.device)
    _check(_c_attn8_skip(_ptr(q), _ld(q), _ptr(k), _ld(k), _ptr(v), _ld(v), _ptr(o), _ld(o), n_buf,
                         n_heads, head_dim, _ptr(cu_slots), _ptr(valid_len), n_seg, max_valid_len,
                         softmax_scale, skip_log2, _ptr(ws), ws.numel() * ws.element_size(),
                         _dt(q), _stream(stream)))


def h3_modulate_residual(x, y=None, gate=None, shift=None, scale=None, h_out=None,
                         ld_mod: Optional[int] = None, norm_kind: int = 0, eps: float = 1e-6,
                         stream=None):
    """x [n, C] in place; gate/shift/scale [n or 1, C] row views (ld_mod 0 = broadcast)."""
    mod_ref = next((t for t in (gate, shift, scale) if t is not None), None)
    if ld_mod is None:
        ld_mod = 0 if mod_ref is None or mod_ref.shape[0] == 1 else _ld(mod_ref)
    n, c = x.shape
    _mat(x, "x", n, c, x.dtype)
    if y is not None:
        _mat(y, "y", n, c, x.dtype)
    if h_out is not None:
        _mat(h_out, "h_out", n, c, x.dtype)
    for t, name in ((gate, "gate"), (shift, "shift"), (scale, "scale")):
        if t is not None:
            # the three share one row stride in the call
            _mat(t, name, 1 if ld_mod == 0 else n, c, x.dtype)
            if ld_mod != 0 and _ld(t) != ld_mod:
                raise ValueError("gate, shift and scale must share one row stride (ld_mod)")
    _check(_c_modres(_ptr(x), _ld(x), _ptr(y), _ld(y) if y is not None else 0, _ptr(gate),
                     _ptr(shift), _ptr(scale), ld_mod, _ptr(h_out),
                     _ld(h_out) if h_out is not None else 0, x.shape[0], x.shape[1], norm_kind, eps,
                     _dt(x), _stream(stream)))


def h3_linear(a, w, out, gate=None, ld_gate: Optional[int] = None, stream=None):
    """out = a @ w^T, or out += gate * (a @ w^T) if gate is given."""
    m, k = a.shape
    n = w.shape[0]
    _mat(a, "a", m, k, a.dtype)
    _mat(w, "w", n, k, a.dtype)
    _mat(out, "out", m, n, a.dtype)
    if gate is not None:
        _mat(gate, "gate", _gate_rows(gate, ld_gate, m), n, a.dtype)
        if ld_gate is None:
            ld_gate = 0 if gate.shape[0] == 1 else _ld(gate)
    _check(_c_linear(_ptr(a), _ld(a), _ptr(w), _ld(w), _ptr(out), _ld(out), a.shape[0],
                     w.shape[0], a.shape[1], _ptr(gate), ld_gate or 0, _dt(a), _stream(stream)))


def swiglu_workspace_size(n_tok: int, ffn_dim: int, dtype) -> int:
    return _c_swiglu_ws(n_tok, ffn_dim, H3_BF16 if dtype == torch.bfloat16 else H3_F32)


def h3_swiglu(h, w1, w3, w2, out, gate=None, ld_gate: Optional[int] = None,
              ws: Optional[torch.Tensor] = None, stream=None):
    n, c = h.shape
    f = w1.shape[0]
    _mat(h, "h", n, c, h.dtype)
    _dense(w1, "w1", (f, c), h.dtype)
    _dense(w3, "w3", (f, c), h.dtype)
    _dense(w2, "w2", (c, f), h.dtype)
    _mat(out, "out", n, c, h.dtype)
    if gate is not None:
        _mat(gate, "gate", _gate_rows(gate, ld_gate, n), c, h.dtype)
        if ld_gate is None:
            ld_gate = 0 if gate.shape[0] == 1 else _ld(gate)
    if ws is None:
        ws = _bytes_ws(swiglu_workspace_size(n, f, h.dtype), h.device)
    _check(_c_swiglu(_ptr(h), _ld(h), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out), _ld(out),
                     _ptr(gate), ld_gate or 0, n, c, f, _ptr(ws), ws.numel() * ws.element_size(),
                     _dt(h), _stream(stream)))


class MxTensor:
    """An MX-e4m3 operand on the device: q uint8 [rows, >= round_up(k, 128)]
    (e4m3 bytes, zeros past k) and s uint8 [rows, >= round_up(k, 128) / 32]
    (E8M0 bytes), k logical columns."""

    def __init__(self, q: torch.Tensor, s: torch.Tensor, k: int):
        self.q, self.s, self.k = q, s, k

    @staticmethod
    def empty(rows: int, k: int, device="cuda") -> "MxTensor":
        kp = -(-k // 128) * 128
        return MxTensor(torch.empty((rows, kp), dtype=torch.uint8, device=device),
                        torch.empty((rows, kp // 32), dtype=torch.uint8, device=device), k)

    def check(self, name: str, rows: int, k: Optional[int] = None):
        """Holds rows x round_up(k, 128) e4m3 bytes and their scale bytes."""
        k = self.k if k is None else k
        if self.k != k:
            raise ValueError(f"{name} holds k = {self.k} columns; the call needs {k}")
        kp = -(-k // 128) * 128
        _mat(self.q, f"{name}.q", rows, kp, torch.uint8)
        _mat(self.s, f"{name}.s", rows, kp // 32, torch.uint8)

    def c(self) -> MxOperand:
        return MxOperand(_ptr(self.q), _ld(self.q), _ptr(self.s), _ld(self.s))


def h3_mx_quantize(x, out: Optional[MxTensor] = None, stream=None) -> MxTensor:
    """bf16 x [rows, cols] -> MxTensor (allocated when out is None)."""
    rows, cols = x.shape
    _mat(x, "x", rows, cols, torch.bfloat16)
    if out is None:
        out = MxTensor.empty(rows, cols, x.device)
    out.check("out", rows, cols)
    _check(_c_mxq(_ptr(x), _ld(x), rows, cols, _ptr(out.q), _ld(out.q), _ptr(out.s), _ld(out.s),
                  _dt(x), _stream(stream)))
    return out


def h3_modulate_mx(x, shift, scale, out: Optional[MxTensor] = None, ld_mod: Optional[int] = None,
                   norm_kind: int = 0, eps: float = 1e-6, stream=None) -> MxTensor:
    """Modulated norm of bf16 x [n, C] written as an MxTensor (C % 128 == 0); the
    same bytes as h3_mx_quantize of h3_modulate_residual's bf16 h."""
    n, c = x.shape
    _mat(x, "x", n, c, torch.bfloat16)
    if out is None:
        out = MxTensor.empty(n, c, x.device)
    out.check("out", n, c)
    if ld_mod is None:
        ld_mod = 0 if shift.shape[0] == 1 else _ld(shift)
    for t, name in ((shift, "shift"), (scale, "scale")):
        _mat(t, name, 1 if ld_mod == 0 else n, c, torch.bfloat16)
        if ld_mod != 0 and _ld(t) != ld_mod:
            raise ValueError("shift and scale must share one row stride (ld_mod)")
    _check(_c_modmx(_ptr(x), _ld(x), _ptr(shift), _ptr(scale), ld_mod, _ptr(out.q), _ld(out.q),
                    _ptr(out.s), _ld(out.s), n, c, norm_kind, eps, _stream(stream)))
    return out


def h3_linear_fp8(a: MxTensor, w: MxTensor, out, gate=None, ld_gate: Optional[int] = None,
                  stream=None):
    """out = a @ w^T over MX operands, or out += gate * (a @ w^T)."""
    m, n = a.q.shape[0], w.q.shape[0]
    a.check("a", m)
    w.check("w", n, a.k)
    _mat(out, "out", m, n, torch.bfloat16)
    if gate is not None:
        _mat(gate, "gate", _gate_rows(gate, ld_gate, m), n, torch.bfloat16)
        if ld_gate is None:
            ld_gate = 0 if gate.shape[0] == 1 else _ld(gate)
    ca, cw = a.c(), w.c()
    _check(_c_lin8(ctypes.byref(ca), ctypes.byref(cw), _ptr(out), _ld(out), a.q.shape[0],
                   w.q.shape[0], a.k, _ptr(gate), ld_gate or 0, _stream(stream)))


def swiglu_fp8_workspace_size(n_tok: int, ffn_dim: int) -> int:
    return _c_sw8_ws(n_tok, ffn_dim)


def h3_swiglu_fp8(h: MxTensor, w1: MxTensor, w3: MxTensor, w2: MxTensor, out, gate=None,
                  ld_gate: Optional[int] = None, ws: Optional[torch.Tensor] = None, stream=None):
    n, c, f = h.q.shape[0], h.k, w1.q.shape[0]
    h.check("h", n)
    w1.check("w1", f, c)
    w3.check("w3", f, c)
    w2.check("w2", c, f)
    _mat(out, "out", n, c, torch.bfloat16)
    if gate is not None:
        _mat(gate, "gate", _gate_rows(gate, ld_gate, n), c, torch.bfloat16)
        if ld_gate is None:
            ld_gate = 0 if gate.shape[0] == 1 else _ld(gate)
    if ws is None:
        ws = _bytes_ws(swiglu_fp8_workspace_size(n, f), h.q.device)
    ops = [x.c() for x in (h, w1, w3, w2)]
    _check(_c_sw8(*[ctypes.byref(o) for o in ops], _ptr(out), _ld(out), _ptr(gate), ld_gate or 0,
                  n, c, f, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def block_config(dim, n_heads, head_dim, ffn_dim, sections, theta=1e4, eps_qk=1e-6,
                 eps_mod=1e-6, norm_kind=0, dtype=torch.bfloat16,
                 attn_fp8=False, gemm_fp8=False, attn_skip_log2=0.0) -> BlockConfig:
    return BlockConfig(dim, n_heads, head_dim, ffn_dim, sections[0], sections[1], sections[2],
                       theta, eps_qk, eps_mod, norm_kind,
                       H3_BF16 if dtype == torch.bfloat16 else H3_F32, int(bool(attn_fp8)),
                       int(bool(gemm_fp8)), attn_skip_log2)


def block_weights_mx(weights: dict, stream=None) -> list:
    """MX copies (MxTensor) of a block's bf16 projection weights, in the order
    h3_block_weights.mx takes them: w_qkv, w_o, w1, w3, w2."""
    return [h3_mx_quantize(weights[k], stream=stream) for k in ("w_qkv", "w_o", "w1", "w3", "w2")]


def block_workspace_size(cfg: BlockConfig, n_tok_local: int, n_buf: int, n_seg: int,
                         head_count: int = 0) -> int:
    """head_count > 0: a rank share with that head slice; 0: world 1 or any share."""
    return _c_block_ws(ctypes.byref(cfg), n_tok_local, n_buf, n_seg, head_count)


def h3_dit_block_forward(cfg: BlockConfig, weights: dict, x, mod, pos, cu_slots, valid_len,
                         max_valid_len: int, ws=None, n_buf: Optional[int] = None,
                         tok_begin: int = 0, head_begin: int = 0, head_count: Optional[int] = None,
                         qkv_attn=None, o_attn=None, o_local=None, qkv_send=None, o_recv=None,
                         stream=None):
    """One block, x [n, C] updated in place.  mod is [n, 6, C] or [1, 6, C] (broadcast).

    Rank share: qkv_attn/o_attn with either o_local (heads of the other ranks
    pre-filled) or the peer-major exchange buffers qkv_send [P, n, 3, hc, D]
    and o_recv [P, n, hc, D] (blocks of the other ranks pre-filled)."""
    n = x.shape[0]
    share = qkv_attn is not None
    n_buf = n_buf if n_buf is not None else (qkv_attn.shape[0] if share else n)
    n_seg = _segments(cu_slots, valid_len)
    C, H, D, F = cfg.dim, cfg.n_heads, cfg.head_dim, cfg.ffn_dim
    dt = _TDT.get(cfg.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype code {cfg.dtype}")
    _mat(x, "x", n, C, dt)
    if mod.dim() != 3 or mod.shape[1:] != (6, C) or mod.dtype != dt or mod.shape[0] not in (1, n) \
            or mod.stride(2) != 1 or mod.stride(1) != C:
        raise ValueError(f"mod must be [n_tok or 1, 6, {C}] of {dt} with contiguous [6, C] rows, "
                         f"got {mod.dtype} {tuple(mod.shape)}")
    _ints(pos, "pos", 4 * n)
    for key, shape in (("w_qkv", (3 * H * D, C)), ("w_o", (C, H * D)), ("w1", (F, C)),
                       ("w3", (F, C)), ("w2", (C, F)), ("g_q", (D,)), ("g_k", (D,))):
        if key in ("g_q", "g_k") or not cfg.gemm_fp8 or weights.get(key) is not None:
            _dense(weights.get(key), key, shape, dt)
    hc = head_count if head_count is not None else H
    for t, name, shape in ((qkv_attn, "qkv_attn", (n_buf, 3 * hc * D)), (o_attn, "o_attn", (n_buf, hc * D)),
                           (o_local, "o_local", (n, H * D))):
        if t is not None:
            if t.numel() < shape[0] * shape[1] or not t.is_contiguous() or t.dtype != dt:
                raise ValueError(f"{name} must be a contiguous {dt} buffer of {shape[0]} x {shape[1]} elements")
    P = H // hc if hc else 0
    for t, name, per in ((qkv_send, "qkv_send", 3 * hc * D), (o_recv, "o_recv", hc * D)):
        if t is not None:
            if t.numel() < P * n * per or not t.is_contiguous() or t.dtype != dt:
                raise ValueError(f"{name} must be a contiguous {dt} buffer of {P} x {n} x {per} elements")
    mx = None
    if weights.get("mx") is not None:
        # MX copies of w_qkv, w_o, w1, w3, w2 (MxTensor each) for cfg.gemm_fp8
        shapes = ((3 * H * D, C), (C, H * D), (F, C), (F, C), (C, F))
        for name, m, (rows, k) in zip(("w_qkv", "w_o", "w1", "w3", "w2"), weights["mx"], shapes):
            m.check(f"mx[{name}]", rows, k)
        mx = (MxOperand * 5)(*[m.c() for m in weights["mx"]])
    w = BlockWeights(*(_ptr(weights.get(k)) for k in ("w_qkv", "w_o", "w1", "w3", "w2", "g_q", "g_k")),
                     ctypes.cast(mx, ctypes.POINTER(MxOperand)) if mx is not None else None)
    ld_mod = 0 if mod.shape[0] == 1 else mod.stride(0)
    io = BlockIO(_ptr(x), _ld(x), _ptr(mod), ld_mod, _ptr(pos), _ptr(cu_slots), _ptr(valid_len),
                 n_seg, max_valid_len, n, n_buf, tok_begin, head_begin,
                 head_count if head_count is not None else cfg.n_heads, _ptr(qkv_attn),
                 _ptr(o_attn), _ptr(o_local), _ptr(qkv_send), _ptr(o_recv))
    need = block_workspace_size(cfg, n, n_buf, n_seg, (head_count or cfg.n_heads) if share else 0)
    if ws is None:
        ws = _bytes_ws(need, x.device)
    _check(_c_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(io), _ptr(ws),
                    ws.numel() * ws.element_size(), _stream(stream)))


def timestep_workspace_size(dim: int) -> int:
    return _c_temb_ws(dim)


def h3_timestep_modulation(sigma: float, w_t1, w_t2, table, mod_out, ws=None, stream=None):
    nb, six, c = table.shape
    if six != 6:
        raise ValueError("table must be [n_blocks, 6, C]")
    e = w_t1.shape[1] if w_t1.dim() == 2 else -1
    _dense(table, "table", (nb, 6, c), table.dtype)
    _dense(mod_out, "mod_out", (nb, 6, c), table.dtype)
    _dense(w_t1, "w_t1", (c, e), table.dtype)
    _dense(w_t2, "w_t2", (6 * c, c), table.dtype)
    if ws is None:
        ws = _bytes_ws(timestep_workspace_size(c), table.device)
    _check(_c_temb(sigma, _ptr(w_t1), _ptr(w_t2), _ptr(table), _ptr(mod_out), nb, c,
                   w_t1.shape[1], _ptr(ws), ws.numel() * ws.element_size(), _dt(table),
                   _stream(stream)))


def h3_euler_update(z, u, x_next=None, sigma_from: float = 0.0, sigma_to: float = 0.0,
                    stream=None):
    """z <- z + (sigma_to - sigma_from) * u over every element; x_next <- z."""
    for t, name in ((z, "z"), (u, "u"), (x_next, "x_next")):
        if t is not None and (t.dtype != z.dtype or t.numel() != z.numel() or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous with z's dtype and element count")
    _check(_c_euler(_ptr(z), _ptr(u), _ptr(x_next), z.numel(), sigma_from, sigma_to, _dt(z),
                    _stream(stream)))


def h3_frames_to_u8(frames, out, layout: int = 0, stream=None):
    """frames: float32 [B, 3, T, H, W] (contiguous); out: uint8 [B, T, H, W, 3]
    (layout 0) or [B, T, 3, H, W] (layout 1), contiguous."""
    if frames.dtype != torch.float32 or out.dtype != torch.uint8:
        raise TypeError("frames must be float32 and out uint8")
    if not (frames.is_contiguous() and out.is_contiguous()):
        raise ValueError("frames and out must be contiguous")
    if frames.dim() != 5 or frames.shape[1] != 3:
        raise ValueError("frames must be [B, 3, T, H, W]")
    B, _, T, H, W = frames.shape
    want = (B, T, H, W, 3) if layout == 0 else (B, T, 3, H, W)
    if tuple(out.shape) != want:
        raise ValueError(f"out must have shape {want}")
    _check(_c_frames(_ptr(frames), B, T, H, W, _ptr(out), layout, _stream(stream)))


def h3_check_segments(cu_slots, valid_len, n_buf: int, max_valid_len: int) -> None:
    """Check segment metadata given as host int32 arrays (numpy or CPU tensors);
    raises H3Error (H3_ERR_ARG) naming the first violated rule."""
    import numpy as np
    cu = np.ascontiguousarray(np.asarray(cu_slots), dtype=np.int32)
    vl = None if valid_len is None else np.ascontiguousarray(np.asarray(valid_len), dtype=np.int32)
    n_seg = cu.size - 1
    if vl is not None and vl.size != n_seg:
        raise ValueError("valid_len must have one entry per segment")
    _check(_c_check_segments(cu.ctypes.data, None if vl is None else vl.ctypes.data, n_seg, n_buf,
                             max_valid_len))
