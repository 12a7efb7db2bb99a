"""Skip-Softmax attention (GPU) against the oracle's Skip-Softmax rule.

Inputs are built so that every skip decision has a wide margin (on these
seeds the closest skipped block sits 2.2 log2 units below the threshold and
the closest kept one 1.7 above, far beyond the ~1e-5 by which the kernel's
fp32 scores differ from the oracle's float64 ones), so both take the same
decisions; the kept blocks then go through the exact attention path."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _util import assert_close, dev, dev_i32, host

pytestmark = pytest.mark.gpu


def _blocky(lengths, n_buf, H, D, far_frac, seed, v_far=None):
    """q = 4 e0 + N(0, 0.05^2); keys N(0, 1), except in a seeded subset of each
    segment's 64-key blocks (never the first), whose keys are -c e0 + N(0,
    0.05^2) with c set so that their scores sit at -4.5 log2 units.  The kept
    blocks' maxima are near +1.3, so with t = -3 the far blocks are skipped
    with a margin of ~3 and the others kept with a margin of ~4, while the
    skipped weight (2^-4.5 per key relative to the row max) is large enough to
    see in the output.  v_far: the far blocks' values are v_far + N(0, 0.05^2),
    which makes the skipped weight move the output by far more than the FP8
    path's rounding."""
    g = np.random.default_rng(seed)
    e0 = np.zeros(D, np.float32)
    e0[0] = 1.0
    c = 4.5 / (4.0 * np.log2(np.e) / np.sqrt(D))
    q = (4.0 * e0 + 0.05 * g.standard_normal((n_buf, H, D))).astype(np.float32)
    k = g.standard_normal((n_buf, H, D)).astype(np.float32)
    v = g.standard_normal((n_buf, H, D)).astype(np.float32)
    # each segment's slot: its length rounded up to 32 plus 16 padding rows,
    # the last slot running to the end of the buffer
    cu = np.zeros(len(lengths) + 1, np.int64)
    for s, n in enumerate(lengths):
        cu[s + 1] = cu[s] + 32 * (-(-n // 32)) + 16
    assert cu[-1] <= n_buf
    cu[-1] = n_buf
    far_blocks = 0
    for s, n in enumerate(lengths):
        for b in range(1, -(-n // 64)):
            if g.random() < far_frac:
                lo = cu[s] + 64 * b
                hi = min(lo + 64, cu[s] + n)
                k[lo:hi] = -c * e0 + 0.05 * g.standard_normal((hi - lo, H, D))
                if v_far is not None:
                    v[lo:hi] = v_far + 0.05 * g.standard_normal((hi - lo, H, D))
                far_blocks += 1
    r = lambda a: W.round_to_bf16(a)
    return r(q), r(k), r(v), cu, np.asarray(lengths), far_blocks


def _run(lib, q, k, v, cu, vl, H, D, skip_log2):
    n_buf = q.shape[0]
    qd, kd, vd = (dev(a.reshape(n_buf, H * D), "bf16") for a in (q, k, v))
    o = torch.full((n_buf, H * D), float("nan"), dtype=torch.bfloat16, device="cuda")
    if skip_log2 is None:
        lib.h3_varlen_attn(qd, kd, vd, o, H, D, dev_i32(cu), dev_i32(vl), int(vl.max()))
    else:
        lib.h3_varlen_attn_skip(qd, kd, vd, o, H, D, dev_i32(cu), dev_i32(vl), int(vl.max()), skip_log2)
    torch.cuda.synchronize()
    return host(o).reshape(n_buf, H, D)


@pytest.mark.parametrize("lengths,n_buf,H,D", [((700, 333, 64), 1200, 2, 128), ((500, 40), 640, 3, 64)])
def test_skip_matches_oracle_rule(lib, lengths, n_buf, H, D):
    q, k, v, cu, vl, far = _blocky(lengths, n_buf, H, D, 0.5, seed=3)
    assert far > 0
    got = _run(lib, q, k, v, cu, vl, H, D, -3.0)
    ref = O.varlen_attention_skip(q, k, v, cu, vl, -3.0)
    exact = O.varlen_attention(q, k, v, cu, vl)
    valid = np.zeros(n_buf, bool)
    for s in range(len(vl)):
        valid[cu[s]:cu[s] + vl[s]] = True
    assert_close(got[valid], ref[valid], "bf16", f"skip {lengths}")
    assert np.all(got[~valid] == 0)
    # the kernel took the skips: it sits on the Skip-Softmax result, several
    # times closer to it than to exact attention
    to_ref = np.abs(got[valid] - ref[valid]).mean()
    to_exact = np.abs(got[valid] - exact[valid]).mean()
    assert to_exact > 3 * to_ref, (to_ref, to_exact)


@pytest.mark.parametrize("lengths,n_buf,H,D", [((700, 333, 64), 1200, 2, 128), ((500, 40), 640, 3, 64)])
def test_skip_without_skips_is_the_exact_kernel(lib, lengths, n_buf, H, D):
    """-inf threshold, and a finite one with nothing below it: bit for bit the exact path."""
    q, k, v, cu, vl, _ = _blocky(lengths, n_buf, H, D, 0.0, seed=4)
    base = _run(lib, q, k, v, cu, vl, H, D, None)
    assert np.array_equal(_run(lib, q, k, v, cu, vl, H, D, float("-inf")), base)
    assert np.array_equal(_run(lib, q, k, v, cu, vl, H, D, -30.0), base)


def test_skip_10s_share_random_inputs_skip_nothing(lib):
    """On the 10 s share's random operands no key block is far enough below the
    running max for t = -20: the Skip-Softmax path equals the exact one."""
    wl = W.SHARE_10S
    N, hc, D = wl.n_pad_total, wl.head_count, wl.head_dim
    g = torch.Generator(device="cuda").manual_seed(5)
    qa = torch.randn((N, 3 * hc * D), generator=g, device="cuda").to(torch.bfloat16)
    q, k, v = qa[:, :hc * D], qa[:, hc * D:2 * hc * D], qa[:, 2 * hc * D:]
    cu = torch.tensor([0, N], dtype=torch.int32, device="cuda")
    vl = torch.tensor([wl.n_valid], dtype=torch.int32, device="cuda")
    o1 = torch.empty((N, hc * D), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    lib.h3_varlen_attn(q, k, v, o1, hc, D, cu, vl, wl.n_valid)
    lib.h3_varlen_attn_skip(q, k, v, o2, hc, D, cu, vl, wl.n_valid, -20.0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ------------------------------------------------------------ FP8 path

# the FP8 attention bar against the quantized-operand oracle: the e4m3 rounding
# of 256 p (up to 2^-4 relative per weight) leaves a few percent relative L2
# FP8 path: against the oracle's FP8 attention with the rule (same e4m3
# weights on the same grid), the bf16 bar; a CPU emulation of the kernel's
# arithmetic on these cases gives max-abs 1.5e-3 - 5e-3, relative L2 0.18%
TOL_Q = dict(max_abs=2e-2, mean_abs=2e-3, rel_l2=1e-2)


def _run8(lib, q, k, v, cu, vl, H, D, skip_log2):
    n_buf = q.shape[0]
    qd, kd, vd = (dev(a.reshape(n_buf, H * D), "bf16") for a in (q, k, v))
    o = torch.full((n_buf, H * D), float("nan"), dtype=torch.bfloat16, device="cuda")
    if skip_log2 is None:
        lib.h3_varlen_attn_fp8(qd, kd, vd, o, H, D, dev_i32(cu), dev_i32(vl), int(vl.max()))
    else:
        lib.h3_varlen_attn_fp8_skip(qd, kd, vd, o, H, D, dev_i32(cu), dev_i32(vl), int(vl.max()),
                                    skip_log2)
    torch.cuda.synchronize()
    return host(o).reshape(n_buf, H, D)


@pytest.mark.parametrize("lengths,n_buf,H,D", [((700, 333, 64), 1200, 2, 128), ((500, 40), 640, 3, 64)])
def test_fp8_skip_matches_oracle_rule(lib, lengths, n_buf, H, D):
    """FP8 attention with the rule, against the oracle's FP8 attention with the
    rule applied to the scores of its quantized operands (margins of >= 1.8
    log2 units on those scores on these seeds).  The far blocks' values are
    offset by 8, so dropping them moves the output by 0.07-0.28 on average,
    far above the FP8 path's own rounding."""
    q, k, v, cu, vl, far = _blocky(lengths, n_buf, H, D, 0.5, seed=3, v_far=8.0)
    assert far > 0
    got = _run8(lib, q, k, v, cu, vl, H, D, -3.0)
    ref = O.varlen_attention_fp8_operands(q, k, v, cu, vl, skip_log2=-3.0)
    plain = O.varlen_attention_fp8_operands(q, k, v, cu, vl)
    valid = np.zeros(n_buf, bool)
    for s in range(len(vl)):
        valid[cu[s]:cu[s] + vl[s]] = True
    assert_close(got[valid], ref[valid], "bf16", f"fp8 skip {lengths}", **TOL_Q)
    assert np.all(got[~valid] == 0)
    to_ref = np.abs(got[valid] - ref[valid]).mean()
    to_plain = np.abs(got[valid] - plain[valid]).mean()
    assert to_plain > 10 * to_ref, (to_ref, to_plain)


@pytest.mark.parametrize("lengths,n_buf,H,D", [((700, 333, 64), 1200, 2, 128), ((500, 40), 640, 3, 64)])
def test_fp8_skip_without_skips_is_the_fp8_kernel(lib, lengths, n_buf, H, D):
    q, k, v, cu, vl, _ = _blocky(lengths, n_buf, H, D, 0.0, seed=4)
    base = _run8(lib, q, k, v, cu, vl, H, D, None)
    assert np.array_equal(_run8(lib, q, k, v, cu, vl, H, D, float("-inf")), base)
    assert np.array_equal(_run8(lib, q, k, v, cu, vl, H, D, -30.0), base)


def test_fp8_skip_10s_share_random_inputs_skip_nothing(lib):
    wl = W.SHARE_10S
    N, hc, D = wl.n_pad_total, wl.head_count, wl.head_dim
    g = torch.Generator(device="cuda").manual_seed(6)
    qa = torch.randn((N, 3 * hc * D), generator=g, device="cuda").to(torch.bfloat16)
    q, k, v = qa[:, :hc * D], qa[:, hc * D:2 * hc * D], qa[:, 2 * hc * D:]
    cu = torch.tensor([0, N], dtype=torch.int32, device="cuda")
    vl = torch.tensor([wl.n_valid], dtype=torch.int32, device="cuda")
    o1 = torch.empty((N, hc * D), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    lib.h3_varlen_attn_fp8(q, k, v, o1, hc, D, cu, vl, wl.n_valid)
    lib.h3_varlen_attn_fp8_skip(q, k, v, o2, hc, D, cu, vl, wl.n_valid, -20.0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("D,seed", [(128, 7), (64, 8)])
def test_skip_edge_segments(lib, D, seed, fp8):
    """Segments of 65 (a one-key tail block), 0, 1, 129 and 300 keys with 70% far
    blocks: on these seeds the rule skips 66 (D = 128) and 106 (D = 64) group
    blocks with margins >= 1.9 log2 units below the threshold and keeps the rest
    >= 1.08 above it, on exact and on FP8-quantized scores."""
    lengths, n_buf, H = (65, 0, 1, 129, 300), 720, 2
    q, k, v, cu, vl, far = _blocky(lengths, n_buf, H, D, 0.7, seed=seed, v_far=8.0)
    assert far > 0
    valid = np.zeros(n_buf, bool)
    for s in range(len(vl)):
        valid[cu[s]:cu[s] + vl[s]] = True
    if fp8:
        got = _run8(lib, q, k, v, cu, vl, H, D, -3.0)
        ref = O.varlen_attention_fp8_operands(q, k, v, cu, vl, skip_log2=-3.0)
        plain = O.varlen_attention_fp8_operands(q, k, v, cu, vl)
        assert_close(got[valid], ref[valid], "bf16", f"fp8 skip edges D={D}", **TOL_Q)
    else:
        got = _run(lib, q, k, v, cu, vl, H, D, -3.0)
        ref = O.varlen_attention_skip(q, k, v, cu, vl, -3.0)
        plain = O.varlen_attention(q, k, v, cu, vl)
        assert_close(got[valid], ref[valid], "bf16", f"skip edges D={D}")
    assert np.all(got[~valid] == 0)
    # the length-1 segment attends to itself only: its row is its (quantized) value, exactly
    one = cu[2]
    np.testing.assert_array_equal(got[one], W.round_to_bf16(ref[one].astype(np.float32)))
    assert np.abs(got[valid] - plain[valid]).mean() > 10 * np.abs(got[valid] - ref[valid]).mean()


# ------------------------------------------------ full size, sampled groups

def _concentrated_10s(seed=11, v_far=8.0):
    """The 10 s share's head slice with concentrated attention: q = 4 e0 +
    N(0, 0.05^2); keys N(0, 1) except in 75% of the 64-key blocks after the
    first, whose keys are -c e0 + N(0, 0.05^2) (scores near -4.5 log2 units)
    and whose values are v_far + N(0, 0.05^2).  Device bf16 [N, 5 * 128]."""
    wl = W.SHARE_10S
    N, hc, D = wl.n_pad_total, wl.head_count, wl.head_dim
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn((N, hc, D), generator=g, device="cuda") * 0.05
    q[:, :, 0] += 4.0
    k = torch.randn((N, hc, D), generator=g, device="cuda")
    v = torch.randn((N, hc, D), generator=g, device="cuda")
    far = torch.rand((N + 63) // 64, generator=g, device="cuda") < 0.75
    far[0] = False
    rows = far.repeat_interleave(64)[:N]
    nf = int(rows.sum())
    k[rows] = torch.randn((nf, hc, D), generator=g, device="cuda") * 0.05
    k[rows, :, 0] -= 4.5 / (4.0 * np.log2(np.e) / np.sqrt(D))
    v[rows] = v_far + torch.randn((nf, hc, D), generator=g, device="cuda") * 0.05
    bf = torch.bfloat16
    return wl, (q.reshape(N, -1).to(bf), k.reshape(N, -1).to(bf), v.reshape(N, -1).to(bf))


def _min_margin(sc, t, q_group=32, k_block=64):
    """Smallest distance (log2 units) between a group's decision statistic
    max_row(block max - running max) and the threshold t, over the blocks
    after the first, following the decisions as they fall."""
    r, n = sc.shape
    best = np.inf
    for g0 in range(0, r, q_group):
        rows = sc[g0:g0 + q_group]
        m = rows[:, :k_block].max(axis=1)
        for b0 in range(k_block, n, k_block):
            bm = rows[:, b0:b0 + k_block].max(axis=1)
            d = (bm - m - t).max()
            best = min(best, abs(d))
            if d >= 0:
                m = np.maximum(m, bm)
    return best


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_skip_10s_share_concentrated_sampled(lib, fp8):
    """Full size, in the bench's launch configuration: the concentrated operands
    of breakdown.attention_skip with t = -3, three sampled query groups (the
    first, one in the middle and the shorter last one) against the oracle's
    rule, whose decisions on these rows are checked to lie >= 0.3 log2 units
    from the threshold."""
    wl, (qd, kd, vd) = _concentrated_10s()
    N, hc, D, nv = wl.n_pad_total, wl.head_count, wl.head_dim, wl.n_valid
    cu = torch.tensor([0, N], dtype=torch.int32, device="cuda")
    vl = torch.tensor([nv], dtype=torch.int32, device="cuda")
    o = torch.full_like(qd, float("nan"))
    t = -3.0
    if fp8:
        lib.h3_varlen_attn_fp8_skip(qd, kd, vd, o, hc, D, cu, vl, nv, t)
    else:
        lib.h3_varlen_attn_skip(qd, kd, vd, o, hc, D, cu, vl, nv, t)
    torch.cuda.synchronize()
    last = (nv // 32) * 32
    rows = np.r_[0:32, 123008:123040, last:nv]
    ridx = torch.from_numpy(rows).cuda()
    got = host(o[ridx]).reshape(len(rows), hc, D)
    h = lambda x: x.float().cpu().numpy().reshape(N, hc, D)
    k, v = h(kd), h(vd)
    q = qd[ridx].float().cpu().numpy().reshape(len(rows), hc, D)
    cu_h, vl_h = np.array([0, N]), np.array([nv])
    if fp8:
        c = O.fp8_fold(D)
        qq = O.mx_dequantize(*O.mx_quantize(q, fold=c))
        kq = O.mx_dequantize(*O.mx_quantize(k[:nv]))
        margins = [_min_margin(qq[a:b, hh] @ kq[:, hh].T, t)
                   for a, b in ((0, 32), (32, 64), (64, len(rows))) for hh in range(hc)]
        ref = O.varlen_attention_fp8_operands(q, k, v, cu_h, vl_h, q_rows=rows, skip_log2=t)
        plain = O.varlen_attention_fp8_operands(q, k, v, cu_h, vl_h, q_rows=rows)
        assert min(margins) >= 0.3, margins
        assert_close(got, ref, "bf16", "fp8 skip 10s sampled", **TOL_Q)
    else:
        cl = np.log2(np.e) / np.sqrt(D)
        margins = [_min_margin((q[a:b, hh].astype(np.float64) @ k[:nv, hh].T.astype(np.float64)) * cl, t)
                   for a, b in ((0, 32), (32, 64), (64, len(rows))) for hh in range(hc)]
        ref = O.varlen_attention_skip(q, k, v, cu_h, vl_h, t, q_rows=rows)
        plain = O.varlen_attention(q, k, v, cu_h, vl_h, q_rows=rows)
        assert min(margins) >= 0.3, margins
        assert_close(got, ref, "bf16", "skip 10s sampled")
    # the skips were taken: far from attention without the rule
    assert np.abs(got - plain).mean() > 10 * np.abs(got - ref).mean()
