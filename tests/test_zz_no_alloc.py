"""The no-allocation attention entry point (GPU): h3_varlen_attn_noalloc,
through the C ABI, against h3_varlen_attn with a caller workspace.

Both launch the same kernels, the first with the library's fixed per-device
scratch for the transposed v, so the outputs must be byte-identical; they are
also held to the oracle at the bf16 bar.  Two calls in a row, the second on a
smaller input (the scratch keeps the first call's bytes), then a call too
large for the scratch, which must be refused with nothing launched."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _util import assert_close, dev, dev_i32, host

pytestmark = pytest.mark.gpu


def _case_tensors(c):
    H, D = c.n_heads, c.head_dim
    q, k, v = (dev(a.reshape(c.n_buf, H * D), "bf16") for a in (c.q, c.k, c.v))
    return q, k, v, dev_i32(c.cu_slots), dev_i32(c.valid_len)


def _valid(c):
    m = np.zeros(c.n_buf, bool)
    for s in range(len(c.valid_len)):
        m[c.cu_slots[s]:c.cu_slots[s] + c.valid_len[s]] = True
    return m


def test_noalloc_attention_matches_workspace_entry(lib):
    cases = [W.varlen_case(seed=0, dtype="bf16", pad_fill="nan"),          # 4032/1500/17 in 8192, 8 x 128
             W.varlen_case(seed=5, lengths=(300, 45, 17), n_buf=512, n_heads=2, head_dim=64,
                           dtype="bf16")]                                   # smaller, D = 64
    for i, c in enumerate(cases):
        print(f"noalloc call {i}: n_buf={c.n_buf} heads={c.n_heads} D={c.head_dim}", flush=True)
        H, D = c.n_heads, c.head_dim
        assert H * D * (-(-c.n_buf // 64) * 64 + 128 * (len(c.valid_len) + 1)) * 2 <= lib.NOALLOC_SCRATCH_BYTES
        q, k, v, cu, vl = _case_tensors(c)
        ml = int(c.valid_len.max())
        o_ws = torch.full((c.n_buf, H * D), float("nan"), dtype=torch.bfloat16, device="cuda")
        o_na = torch.full_like(o_ws, float("nan"))
        lib.h3_varlen_attn(q, k, v, o_ws, H, D, cu, vl, ml)
        lib.h3_varlen_attn_noalloc(q, k, v, o_na, H, D, cu, vl, ml)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws), f"call {i}: differs from the workspace entry"
        got = host(o_na).reshape(c.n_buf, H, D)
        m = _valid(c)
        assert np.all(got[~m] == 0)
        ref = O.varlen_attention(c.q, c.k, c.v, c.cu_slots, c.valid_len)
        assert_close(got[m], ref[m], "bf16", f"noalloc call {i} vs oracle")


def test_noalloc_attention_refuses_oversize(lib):
    """A call whose transposed v would not fit the fixed scratch is refused on
    the host (H3_ERR_WORKSPACE) and launches nothing: o keeps its bytes."""
    H, D = 8, 128
    n_buf = lib.NOALLOC_SCRATCH_BYTES // (H * D * 2) + 64      # one tile over the limit
    q = torch.zeros((n_buf, H * D), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    cu = dev_i32(np.array([0, n_buf]))
    with pytest.raises(lib.H3Error) as e:
        lib.h3_varlen_attn_noalloc(q, q, q, o, H, D, cu, None, n_buf)
    assert e.value.status == lib.H3_ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
