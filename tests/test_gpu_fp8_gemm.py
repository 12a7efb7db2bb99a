"""FP8 (MX-scaled e4m3) projections against the oracle (GPU).

The quantized operands are compared element for element with the oracle's MX
quantizer; the products with the oracle's exact product of the dequantized
operands.  Both sides multiply the same e4m3 values, so the kernel differs
only by the matrix pipe's accumulation and the final bf16 rounding:
elementwise |got - ref| <= 2^-8 |ref| + 2^-14 S, with S = |a| |w|^T the sum of
product magnitudes.  The bf16 rounding is at most 2^-8 relative; the fp8
MFMA's dot products are not exact to fp32 (measured: about 2^-17 of the
product magnitudes one 64-deep instruction sums), and 2^-14 S bounds that
with margin at every K used here."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _util import E4M3_DECODE, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _bf16(seed, name, shape, std=1.0):
    return W.round_to_bf16(W.normal(seed, name, shape, std=std))


def _mx_values(m):
    """Device MxTensor -> (dequantized values [rows, kp] float64, exponents [rows, kp/32])."""
    q = m.q.cpu().numpy()
    e = m.s.cpu().numpy().astype(np.int64) - 127
    kp = -(-m.k // 128) * 128
    vals = E4M3_DECODE[q[:, :kp]] * np.ldexp(1.0, np.repeat(e[:, :kp // 32], 32, axis=1))
    return vals, e[:, :kp // 32]


def _abs_products(x, w):
    """S = |x^| |w^|^T over the dequantized MX operands."""
    xd = np.abs(O.mx_dequantize(*O.mx_quantize(x)))
    wd = np.abs(O.mx_dequantize(*O.mx_quantize(w)))
    return xd @ wd.T


def _close_bf16_product(got, ref, S, what):
    bad = np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * S
    assert np.all(np.isfinite(got)), what
    assert not bad.any(), f"{what}: {bad.sum()} elements off, worst {np.abs(got - ref).max():.3g}"


@pytest.mark.parametrize("rows,cols", [(300, 704), (1, 128), (257, 5120)])
def test_mx_quantize_matches_oracle(lib, rows, cols):
    x = _bf16(1, "mxq", (rows, cols))
    # wide dynamic range across rows, a zero row, and a block with one large element
    x *= np.ldexp(1.0, W.uniform_ints(1, "mxq-exp", -20, 20, rows)).astype(np.float32)[:, None]
    x[0] = 0.0
    if rows > 2:
        x[2, 33] = 3.0e4
    x = W.round_to_bf16(x)
    m = lib.h3_mx_quantize(dev(x, "bf16"))
    torch.cuda.synchronize()
    vals, e = _mx_values(m)
    q_ref, e_ref = O.mx_quantize(x)
    np.testing.assert_array_equal(e[:, :cols // 32], e_ref)
    np.testing.assert_array_equal(vals[:, :cols], O.mx_dequantize(q_ref, e_ref))
    # padding columns up to a multiple of 128: zeros with scale byte 127
    assert not m.q[:, cols:].any()
    assert (m.s[:, cols // 32:] == 127).all()


@pytest.mark.parametrize("M,N,K", [(300, 200, 256), (513, 520, 768), (64, 96, 704), (1, 8, 128),
                                   (1000, 264, 5120), (77, 40, 224), (5, 24, 32), (4000, 5120, 128)])
@pytest.mark.parametrize("residual", [False, True])
def test_linear_fp8_parity(lib, M, N, K, residual):
    a = _bf16(2, f"a{M}", (M, K))
    w = _bf16(2, f"w{N}", (N, K), std=K ** -0.5)
    am, wm = lib.h3_mx_quantize(dev(a, "bf16")), lib.h3_mx_quantize(dev(w, "bf16"))
    ref = O.linear_fp8_operands(a, w)
    S = _abs_products(a, w)
    if residual:
        x = _bf16(3, "x", (M, N))
        g = _bf16(3, "g", (M, N), std=0.5)
        out = dev(x, "bf16")
        lib.h3_linear_fp8(am, wm, out, gate=dev(g, "bf16"))
        ref = x.astype(np.float64) + g.astype(np.float64) * ref
        S = np.abs(g) * S
    else:
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        lib.h3_linear_fp8(am, wm, out)
    torch.cuda.synchronize()
    _close_bf16_product(host(out), ref, S, f"linear_fp8 {M}x{N}x{K} residual={residual}")


def test_linear_fp8_strided_out_and_rerun(lib):
    """Output written into a column slice of a wider buffer, nothing else touched;
    reruns are bit-identical."""
    M, N, K = 290, 136, 384
    a = _bf16(4, "a", (M, K))
    w = _bf16(4, "w", (N, K), std=K ** -0.5)
    am, wm = lib.h3_mx_quantize(dev(a, "bf16")), lib.h3_mx_quantize(dev(w, "bf16"))
    buf = torch.full((M, 400), 7.0, dtype=torch.bfloat16, device="cuda")
    lib.h3_linear_fp8(am, wm, buf[:, 64:64 + N])
    torch.cuda.synchronize()
    got = host(buf)
    _close_bf16_product(got[:, 64:64 + N], O.linear_fp8_operands(a, w), _abs_products(a, w), "strided")
    assert (got[:, :64] == 7.0).all() and (got[:, 64 + N:] == 7.0).all()
    again = buf.clone()
    lib.h3_linear_fp8(am, wm, again[:, 64:64 + N])
    torch.cuda.synchronize()
    assert torch.equal(again, buf)


def _swiglu_ref(h, w1, w3, w2, rows=None):
    """The oracle's MLP over MX operands, with g rounded to bf16 before it is
    quantized (the storage type g has between the two projections)."""
    hs = h if rows is None else h[rows]
    a = O.linear_fp8_operands(hs, w1)
    b = O.linear_fp8_operands(hs, w3)
    g = W.round_to_bf16(O.swiglu_gate(a, b).astype(np.float32))
    return O.linear_fp8_operands(g, w2)


@pytest.mark.parametrize("n,C,F", [(480, 256, 704), (300, 512, 1408), (4000, 256, 2816)])
def test_swiglu_fp8_parity(lib, n, C, F):
    h = _bf16(5, "h", (n, C))
    w1 = _bf16(5, "w1", (F, C), std=C ** -0.5)
    w3 = _bf16(5, "w3", (F, C), std=C ** -0.5)
    w2 = _bf16(5, "w2", (C, F), std=F ** -0.5)
    x = _bf16(5, "x", (n, C))
    g = _bf16(5, "gate", (n, C), std=0.5)
    mx = [lib.h3_mx_quantize(dev(t, "bf16")) for t in (h, w1, w3, w2)]
    out = dev(x, "bf16")
    ws = torch.empty(lib.swiglu_fp8_workspace_size(n, F), dtype=torch.uint8, device="cuda")
    lib.h3_swiglu_fp8(*mx, out, gate=dev(g, "bf16"), ws=ws)
    torch.cuda.synchronize()
    a, b = O.linear_fp8_operands(h, w1), O.linear_fp8_operands(h, w3)
    g_ref = O.swiglu_gate(a, b)
    # g = silu(a) b: errors in a and b enter through |silu'(a)| <= 1.1 and |silu(a)|
    S = 1.1 * np.abs(b) * _abs_products(h, w1) + np.abs(O.silu(a)) * _abs_products(h, w3)
    fp = -(-F // 128) * 128
    up = lambda b: -(-b // 256) * 256
    if F % 128:
        # g = bf16(silu(h w1^T) * (h w3^T)) sits at the start of the workspace,
        # and a separate pass quantizes it: its MX operand is the MX
        # quantization of the stored bf16 g, byte for byte
        g_got = host(ws[:n * F * 2].view(torch.bfloat16).reshape(n, F))
        _close_bf16_product(g_got, g_ref, S, f"swiglu_fp8 gate product {n}x{C}x{F}")
        gq_off = up(n * F * 2)
        gs_off = gq_off + up(n * fp)
        g_dev = ws[:n * F * 2].view(torch.bfloat16).reshape(n, F)
        ref_mx = lib.h3_mx_quantize(g_dev.clone())
        torch.cuda.synchronize()
        assert torch.equal(ws[gq_off:gq_off + n * fp].reshape(n, fp), ref_mx.q)
        assert torch.equal(ws[gs_off:gs_off + n * (fp // 32)].reshape(n, fp // 32), ref_mx.s)
    else:
        # F % 128 == 0: the up-projection's epilogue writes g only as its MX
        # operand (the quantization of bf16 g), at the start of the workspace
        gs_off = up(n * fp)
        q = ws[:n * fp].reshape(n, fp).cpu().numpy()
        e = ws[gs_off:gs_off + n * (fp // 32)].reshape(n, fp // 32).cpu().numpy().astype(np.int64) - 127
        e_full = np.repeat(e, 32, axis=1)
        vals = E4M3_DECODE[q] * np.ldexp(1.0, e_full)
        assert np.all(np.isfinite(vals))
        # bound: the e4m3 half step at the element's binade (2^-4 relative, or
        # half the subnormal quantum 2^-10 of the block scale) on top of the
        # bf16 gate product's own bound
        bound = (2.0 ** -4 * (1 + 2.0 ** -3) + 2.0 ** -8) * np.abs(g_ref) + 2.0 ** -14 * S \
            + 2.0 ** -10 * np.ldexp(1.0, e_full)
        bad = np.abs(vals - g_ref) > bound
        assert not bad.any(), f"swiglu_fp8 g (mx): {bad.sum()} elements off"
        # decisions: the oracle's g rounded to bf16 and quantized the same way
        # gives the same scales and codes wherever the two bf16 g agree (they
        # differ only in last bits of the fp32 accumulation)
        q_ref, e_ref = O.mx_quantize(W.round_to_bf16(g_ref.astype(np.float32)))
        assert np.abs(e - e_ref).max() <= 1 and (e != e_ref).mean() < 1e-3
        assert (vals != O.mx_dequantize(q_ref, e_ref)).mean() < 1e-2
    ref = x.astype(np.float64) + g.astype(np.float64) * _swiglu_ref(h, w1, w3, w2)
    got = host(out)
    # g is rounded to bf16 on both sides from values that differ in the last
    # fp32 bits (accumulation order), so a few g elements sit one bf16 ulp
    # apart and some of those round to neighbouring e4m3 values (a 2^-4
    # step) before the down-projection; on these inputs that moves single
    # outputs by up to ~0.016, on top of the final bf16 rounding of |x| <= 4.7
    # (up to 2^-6): max-abs 4e-2, mean and relative L2 at the bf16 bar.
    assert_close(got, ref, "bf16", f"swiglu_fp8 {n}x{C}x{F}", max_abs=4e-2)
    # the update itself (x is O(1), the MLP branch O(0.5))
    assert_close(got - x, ref - x, "bf16", "swiglu_fp8 update", max_abs=4e-2, rel_l2=2e-2)


@pytest.mark.parametrize("n", [30776, 45912], ids=["share10s", "loop15s"])
def test_fp8_projections_share_shapes_sampled(lib, n):
    """The block's projection shapes at the 10 s share (30,776 rows) and the
    15 s share (45,912 rows, the loop benchmark's), C = 5120, F = 13,824: QKV
    and the SwiGLU MLP, full launches; sampled rows (and, for QKV, sampled
    output columns, each a weight row quantized on its own) checked."""
    print(f"fp8 projections n={n}", flush=True)
    C, F = 5120, 13824
    rows = np.sort(W.uniform_ints(6, "rows", 0, n - 1, 24))
    rows[-1] = n - 1
    h = _bf16(6, "h", (n, C))
    hm = lib.h3_mx_quantize(dev(h, "bf16"))
    wq = _bf16(6, "wqkv", (3 * C, C), std=C ** -0.5)
    wqm = lib.h3_mx_quantize(dev(wq, "bf16"))
    qkv = torch.empty((n, 3 * C), dtype=torch.bfloat16, device="cuda")
    lib.h3_linear_fp8(hm, wqm, qkv)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([W.uniform_ints(6, "cols", 0, 3 * C - 1, 600), [0, 3 * C - 1]]))
    got = host(qkv[torch.from_numpy(rows).cuda()])[:, cols]
    _close_bf16_product(got, O.linear_fp8_operands(h[rows], wq[cols]), _abs_products(h[rows], wq[cols]),
                        f"qkv n={n} sampled")
    del qkv, wqm
    w1 = _bf16(6, "w1", (F, C), std=C ** -0.5)
    w3 = _bf16(6, "w3", (F, C), std=C ** -0.5)
    w2 = _bf16(6, "w2", (C, F), std=F ** -0.5)
    mx = [lib.h3_mx_quantize(dev(t, "bf16")) for t in (w1, w3, w2)]
    out = torch.empty((n, C), dtype=torch.bfloat16, device="cuda")
    lib.h3_swiglu_fp8(hm, *mx, out)
    torch.cuda.synchronize()
    got = host(out[torch.from_numpy(rows).cuda()])
    assert_close(got, _swiglu_ref(h, w1, w3, w2, rows), "bf16", f"swiglu_fp8 n={n} sampled", max_abs=4e-2)


@pytest.mark.parametrize("rows,dim,per_token,norm_kind", [(333, 256, True, 0), (70, 384, False, 0),
                                                         (129, 5120, True, 0), (65, 1024, True, 1),
                                                         # every other launch tier, whole and partial
                                                         # (16, 144, 272, 512, 528, 656, 1040 and 2048
                                                         # chunks of 8)
                                                         (9, 128, True, 0), (17, 1152, True, 1),
                                                         (17, 2176, True, 0), (9, 4096, False, 0),
                                                         (9, 4224, True, 1), (9, 5248, True, 0),
                                                         (5, 8320, True, 1), (5, 16384, True, 0)])
def test_modulate_mx_equals_norm_then_quantize(lib, rows, dim, per_token, norm_kind):
    """The fused modulated norm -> MX operand gives the bytes of the two passes it
    replaces: the bf16 modulated norm, then the MX quantizer (each pinned to the
    oracle on its own); per-token and broadcast modulation, LayerNorm and RMSNorm,
    ragged row counts."""
    g = torch.Generator(device="cuda").manual_seed(rows + dim)
    bf = torch.bfloat16
    x = (3 * torch.randn((rows, dim), generator=g, device="cuda")).to(bf)
    mod = (0.5 * torch.randn((rows if per_token else 1, 6, dim), generator=g, device="cuda")).to(bf)
    x[rows // 2] = 0  # a constant row: zero variance
    h = torch.empty_like(x)
    xs = x.clone()
    lib.h3_modulate_residual(xs, shift=mod[:, 0], scale=mod[:, 1], h_out=h, norm_kind=norm_kind)
    ref = lib.h3_mx_quantize(h)
    got = lib.h3_modulate_mx(x, mod[:, 0], mod[:, 1], norm_kind=norm_kind)
    torch.cuda.synchronize()
    assert torch.equal(x, xs), "x is read only"
    assert torch.equal(got.q, ref.q) and torch.equal(got.s, ref.s)
