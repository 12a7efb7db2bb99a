"""Pins of the CPU oracle against what the pages and the mathematics fix.

No test here re-types the oracle's own formula: each checks a closed form, an
invariant, a special case that reduces to a library routine (torch CPU in
float64), a hand-derived fixture, or brute force on tiny inputs.
"""
import hashlib
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ----------------------------------------------------------------- inputs (O0)

def test_bf16_rounding_ties_to_even():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8) * 4,
                  2 ** -133, np.inf, -np.inf], dtype=np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -4.0, 2 ** -133, np.inf, -np.inf], dtype=np.float32)
    got = W.round_to_bf16(a)
    assert np.array_equal(got, want)
    assert np.isnan(W.round_to_bf16(np.array([np.nan], np.float32)))[0]
    # agrees with torch's own float32 -> bfloat16 conversion (round to nearest even)
    x = rng.standard_normal(100000).astype(np.float32) * 7
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(W.round_to_bf16(x), ref)


def test_seeded_draws_are_byte_identical():
    a = W.normal(0, "x", (3000, 5000), threads=1)
    b = W.normal(0, "x", (3000, 5000), threads=8)
    c = W.normal(1, "x", (3000, 5000))
    assert hashlib.sha256(a.tobytes()).digest() == hashlib.sha256(b.tobytes()).digest()
    assert not np.array_equal(a, c)
    assert abs(a.mean()) < 1e-2 and abs(a.std() - 1) < 1e-2


def test_positions_layout():
    wl = W.TINY
    pos = W.positions(wl)
    assert pos.shape == (480, 4)
    assert (pos[:384, 0] == 0).all() and (pos[384:, 0] == 1).all()
    # t slowest, then h, then w
    assert tuple(pos[0, 1:]) == (0, 0, 0) and tuple(pos[1, 1:]) == (0, 0, 1)
    assert tuple(pos[12, 1:]) == (0, 1, 0) and tuple(pos[96, 1:]) == (1, 0, 0)
    assert tuple(pos[383, 1:]) == (3, 7, 11)
    assert (pos[384:, 1] == np.arange(96)).all()
    w10 = W.SHARE_10S
    assert w10.n_valid == 246206 and w10.n_pad_total == 246208 and w10.n_loc == 30776
    p10 = W.positions(w10)
    assert (p10[-2:, 0] == W.POS_PAD).all() and p10[245952, 0] == W.POS_AUDIO


def test_varlen_case_layout():
    c = W.varlen_case(seed=0, n_heads=2, head_dim=8)
    assert c.cu_slots[0] == 0 and c.cu_slots[-1] == 8192
    slots = np.diff(c.cu_slots)
    assert (slots >= c.valid_len).all()
    assert c.valid_len.tolist() == [4032, 1500, 17]


# ------------------------------------------------------------------- O1 modnorm

def test_modnorm_closed_form_moments():
    x = rng.standard_normal((64, 256)) * 3 + 1.5
    eps = 1e-6
    z = np.zeros_like(x)
    n = O.modulated_norm(x, z, z, eps)
    var = x.var(axis=1)
    assert np.allclose(n.mean(axis=1), 0, atol=1e-12)
    assert np.allclose((n ** 2).mean(axis=1), var / (var + eps), rtol=1e-12)


def test_modnorm_matches_library_layer_norm():
    x = rng.standard_normal((32, 96))
    z = np.zeros_like(x)
    got = O.modulated_norm(x, z, z, 1e-6)
    ref = F.layer_norm(t64(x), (96,), eps=1e-6).numpy()
    assert np.allclose(got, ref, atol=1e-12)
    got = O.modulated_norm(x, z, z, 1e-6, kind="rms")
    ref = F.rms_norm(t64(x), (96,), eps=1e-6).numpy()
    assert np.allclose(got, ref, atol=1e-12)


def test_modnorm_modulation_special_cases():
    x = rng.standard_normal((16, 40))
    shift = rng.standard_normal((16, 40))
    # scale = -1 removes the normalised term entirely: output is shift
    assert np.allclose(O.modulated_norm(x, shift, -np.ones_like(x)), shift, atol=1e-14)
    # scale = c with no shift scales the plain norm by (1 + c)
    c = 0.37
    base = F.layer_norm(t64(x), (40,), eps=1e-6).numpy()
    assert np.allclose(O.modulated_norm(x, 0 * x, c + 0 * x), (1 + c) * base, atol=1e-12)
    # shift adds after scaling
    assert np.allclose(O.modulated_norm(x, shift, 0 * x) - base, shift, atol=1e-12)
    # constant rows normalise to 0 (var 0, eps keeps it finite)
    assert np.allclose(O.modulated_norm(np.full((2, 8), 5.0), np.zeros((2, 8)), np.zeros((2, 8))), 0)


def test_gated_residual_zero_gate_is_identity():
    x = rng.standard_normal((8, 16))
    y = rng.standard_normal((8, 16))
    assert np.array_equal(O.gated_residual(x, np.zeros_like(x), y), x)
    g = rng.standard_normal((8, 16))
    # linear in the gate
    d1 = O.gated_residual(x, g, y) - x
    d2 = O.gated_residual(x, 2 * g, y) - x
    assert np.allclose(d2, 2 * d1)


# ------------------------------------------------------------- O3 Q/K RMSNorm

def test_qk_rmsnorm_unit_rms_before_gain():
    q = rng.standard_normal((50, 4, 64)) * 2.5
    g = 1 + 0.02 * rng.standard_normal(64)
    eps = 1e-6
    out = O.rms_norm_heads(q, g, eps)
    ms = (q ** 2).mean(axis=-1)
    assert np.allclose(((out / g) ** 2).mean(axis=-1), ms / (ms + eps), rtol=1e-12)
    ref = F.rms_norm(t64(q), (64,), weight=t64(g), eps=eps).numpy()
    assert np.allclose(out, ref, atol=1e-12)


# ---------------------------------------------------------------------- O4 RoPE

def _golden_rope():
    with open(os.path.join(GOLDEN, "rope_closed_form.json")) as f:
        return json.load(f)


def test_rope_hand_derived_angles():
    g = _golden_rope()
    d, secs, theta = g["head_dim"], tuple(g["sections"]), g["theta"]
    for case in g["cases"]:
        pos = np.array([case["pos"]], dtype=np.int32)
        ang = O.rope_angles(pos, d, secs, theta)[0]
        if case["angles"] is None:
            assert np.all(ang == 0)
            continue
        assert np.allclose(ang, case["angles"], rtol=1e-13, atol=1e-15), case["note"]
        # rotating the unit vector e0 of each pair yields (cos, sin) of that angle,
        # and e1 yields (-sin, cos)
        for unit, want in (((1.0, 0.0), lambda a: (math.cos(a), math.sin(a))),
                           ((0.0, 1.0), lambda a: (-math.sin(a), math.cos(a)))):
            x = np.tile(np.array(unit), d // 2).reshape(1, 1, d)
            y = O.apply_rope(x, ang[None])[0, 0]
            for j, a in enumerate(case["angles"]):
                assert np.allclose(y[2 * j:2 * j + 2], want(a), atol=1e-14)


def test_rope_matches_complex_rotation():
    # pairs as complex numbers a + ib, multiplied by e^{i phi}
    pos = W.positions(W.TINY)
    x = rng.standard_normal((480, 4, 64))
    ang = O.rope_angles(pos, 64, (16, 24, 24), 1e4)
    got = O.apply_rope(x, ang)
    z = torch.complex(t64(x[..., 0::2]), t64(x[..., 1::2])) * torch.polar(
        torch.ones_like(t64(ang)), t64(ang))[:, None, :]
    ref = np.stack([z.real.numpy(), z.imag.numpy()], axis=-1).reshape(x.shape)
    assert np.allclose(got, ref, atol=1e-12)


def test_rope_preserves_norm_and_composes():
    d, secs = 128, (32, 48, 48)
    x = rng.standard_normal((20, 3, d))
    p1 = np.zeros((20, 4), np.int32)
    p1[:, 1:] = rng.integers(0, 300, (20, 3))
    p1[10:, 0] = W.POS_AUDIO
    p2 = p1.copy()
    p2[:, 1:] = rng.integers(0, 300, (20, 3))
    a1 = O.rope_angles(p1, d, secs, 1e4)
    a2 = O.rope_angles(p2, d, secs, 1e4)
    p12 = p1.copy()
    p12[:, 1:] = p1[:, 1:] + p2[:, 1:]
    a12 = O.rope_angles(p12, d, secs, 1e4)
    y = O.apply_rope(x, a1)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    assert np.allclose(O.apply_rope(y, a2), O.apply_rope(x, a12), atol=1e-10)
    zero = np.zeros((20, 4), np.int32)
    zero[10:, 0] = W.POS_AUDIO
    assert np.array_equal(O.apply_rope(x, O.rope_angles(zero, d, secs, 1e4)), x)


@pytest.mark.parametrize("axis", [1, 2, 3])
def test_rope_scores_depend_only_on_relative_position(axis):
    d, secs = 128, (32, 48, 48)
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    kind = W.POS_VIDEO if axis else W.POS_AUDIO

    def score(pq, pk):
        a = np.zeros((1, 4), np.int32)
        b = np.zeros((1, 4), np.int32)
        a[0, 0] = b[0, 0] = kind
        a[0, axis], b[0, axis] = pq, pk
        rq = O.apply_rope(q, O.rope_angles(a, d, secs, 1e4))
        rk = O.apply_rope(k, O.rope_angles(b, d, secs, 1e4))
        return float((rq * rk).sum())

    s0 = score(3, 10)
    assert abs(score(3 + 57, 10 + 57) - s0) < 1e-10
    assert abs(score(0, 7) - s0) < 1e-10
    assert abs(score(10, 3) - s0) > 1e-6  # not symmetric: direction matters


def test_rope_audio_uses_full_width_single_section():
    d, secs = 128, (32, 48, 48)
    pos = np.array([[W.POS_AUDIO, 37, 5, 9]], np.int32)
    ang = O.rope_angles(pos, d, secs, 1e4)[0]
    # the h and w columns are ignored for audio; pair j turns by 37 * 1e4^(-2j/128)
    assert np.allclose(ang[0], 37) and np.allclose(ang[-1], 37 * 1e4 ** (-126 / 128))
    assert np.allclose(np.diff(np.log(ang)), -2 / 128 * math.log(1e4))


def test_qk_norm_rope_pad_rows_untouched():
    pos = W.positions(W.TINY.replace(pad_to=512))
    q = rng.standard_normal((512, 4, 64))
    k = rng.standard_normal((512, 4, 64))
    g = np.ones(64)
    qo, ko = O.qk_norm_rope(q, k, pos, g, g, (16, 24, 24))
    assert np.array_equal(qo[480:], q[480:]) and np.array_equal(ko[480:], k[480:])
    assert np.allclose(np.sqrt((qo[:480] ** 2).mean(-1)), 1, atol=1e-5)


# ------------------------------------------------------------ O5 attention

def _brute_attention(q, k, v, cu, vl, scale):
    n, h, d = q.shape
    out = [[[0.0] * d for _ in range(h)] for _ in range(n)]
    for s in range(len(cu) - 1):
        lo, hi = int(cu[s]), int(cu[s]) + int(vl[s])
        for i in range(lo, hi):
            for hh in range(h):
                sc = []
                for j in range(lo, hi):
                    sc.append(sum(float(q[i, hh, c]) * float(k[j, hh, c]) for c in range(d)) * scale)
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                z = sum(e)
                for c in range(d):
                    out[i][hh][c] = sum(e[j - lo] / z * float(v[j, hh, c]) for j in range(lo, hi))
    return np.array(out)


def test_attention_brute_force_tiny():
    cu = np.array([0, 7, 12, 13, 16], np.int32)
    vl = np.array([5, 5, 0, 2], np.int32)
    q, k, v = (rng.standard_normal((16, 2, 4)) for _ in range(3))
    got = O.varlen_attention(q, k, v, cu, vl)
    ref = _brute_attention(q, k, v, cu, vl, 0.5)
    assert np.allclose(got, ref, atol=1e-13)


def test_attention_matches_library_sdpa_per_segment():
    c = W.varlen_case(seed=3, lengths=(300, 77, 1), n_buf=512, n_heads=3, head_dim=64, dtype="f32")
    got = O.varlen_attention(c.q, c.k, c.v, c.cu_slots, c.valid_len)
    for s in range(3):
        lo = c.cu_slots[s]
        hi = lo + c.valid_len[s]
        ref = F.scaled_dot_product_attention(t64(c.q[lo:hi]).transpose(0, 1), t64(c.k[lo:hi]).transpose(0, 1),
                                             t64(c.v[lo:hi]).transpose(0, 1)).transpose(0, 1).numpy()
        assert np.allclose(got[lo:hi], ref, atol=1e-12)
        assert np.all(got[hi:c.cu_slots[s + 1]] == 0)


def test_attention_special_cases():
    d = 16
    # single-row segment returns its own v
    q, k, v = (rng.standard_normal((4, 1, d)) for _ in range(3))
    o = O.varlen_attention(q, k, v, np.array([0, 1, 4]), np.array([1, 3]))
    assert np.allclose(o[0], v[0])
    # identical keys: uniform weights, output = mean of the valid values
    kk = np.tile(rng.standard_normal((1, 1, d)), (10, 1, 1))
    vv = rng.standard_normal((10, 1, d))
    o = O.varlen_attention(rng.standard_normal((10, 1, d)), kk, vv, np.array([0, 10]), np.array([6]))
    assert np.allclose(o[:6], vv[:6].mean(axis=0, keepdims=True))
    assert np.all(o[6:] == 0)
    # two keys, closed form: weights e^{a}/(e^a+e^b)
    qq = np.array([[[1.0, 0.0]]])
    k2 = np.array([[[2.0, 0.0]], [[0.0, 5.0]]])
    v2 = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    o = O.varlen_attention(qq.repeat(2, 0), k2, v2, np.array([0, 2]), np.array([2]), scale=1.0)
    w0 = math.exp(2) / (math.exp(2) + 1)
    assert np.allclose(o[0, 0], [w0, 1 - w0], atol=1e-15)


def test_attention_packed_equals_each_segment_alone_and_pads_poisoned():
    c = W.varlen_case(seed=5, lengths=(200, 45, 1, 17), n_buf=400, n_heads=2, head_dim=32,
                      dtype="f32", pad_fill="nan")
    got = O.varlen_attention(c.q, c.k, c.v, c.cu_slots, c.valid_len)
    for s in range(4):
        lo = c.cu_slots[s]
        hi = lo + c.valid_len[s]
        alone = O.varlen_attention(c.q[lo:hi], c.k[lo:hi], c.v[lo:hi], np.array([0, hi - lo]),
                                   np.array([hi - lo]))
        assert np.array_equal(got[lo:hi], alone)
    assert np.isfinite(got).all()


def test_attention_permutation_equivariance():
    q, k, v = (rng.standard_normal((50, 2, 8)) for _ in range(3))
    perm = rng.permutation(50)
    cu, vl = np.array([0, 50]), np.array([50])
    a = O.varlen_attention(q, k, v, cu, vl)
    b = O.varlen_attention(q[perm], k[perm], v[perm], cu, vl)
    assert np.allclose(a[perm], b, atol=1e-13)


def test_attention_invariant_to_shifting_all_positions_of_a_segment():
    wl = W.TINY
    pos = W.positions(wl)
    q, k, v = (rng.standard_normal((480, 4, 64)) for _ in range(3))
    g = 1 + 0.02 * rng.standard_normal(64)
    cu, vl = np.array([0, 480]), np.array([480])
    q1, k1 = O.qk_norm_rope(q, k, pos, g, g, wl.sections)
    shifted = pos.copy()
    shifted[:, 1:] += np.array([5, 3, 11])            # video t/h/w shift, audio index shift by 5
    q2, k2 = O.qk_norm_rope(q, k, shifted, g, g, wl.sections)
    # video and audio tokens sit in one segment; a shift that is the same for
    # every token of each kind keeps scores within each kind, not across kinds,
    # so compare per-kind segments
    segs = (np.array([0, 384]), np.array([384]))
    a = O.varlen_attention(q1[:384], k1[:384], v[:384], *segs)
    b = O.varlen_attention(q2[:384], k2[:384], v[:384], *segs)
    assert np.allclose(a, b, atol=1e-10)
    a = O.varlen_attention(q1[384:], k1[384:], v[384:], np.array([0, 96]), np.array([96]))
    b = O.varlen_attention(q2[384:], k2[384:], v[384:], np.array([0, 96]), np.array([96]))
    assert np.allclose(a, b, atol=1e-10)


# ------------------------------------------------------- O2 / O6 / O8 GEMMs, SwiGLU

def test_linear_brute_force_and_identity():
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    got = O.linear(x, w)
    for i in range(3):
        for o in range(4):
            assert abs(got[i, o] - sum(x[i, c] * w[o, c] for c in range(5))) < 1e-13
    assert np.array_equal(O.linear(x, np.eye(5)), x)


def test_silu_and_swiglu():
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(40.0) - 40.0) < 1e-12 and abs(O.silu(-40.0)) < 1e-15
    a = rng.standard_normal((6, 7)) * 3
    assert np.allclose(O.silu(a), F.silu(t64(a)).numpy(), atol=1e-14)
    h = rng.standard_normal((5, 16))
    w1, w3 = rng.standard_normal((24, 16)), rng.standard_normal((24, 16))
    w2 = rng.standard_normal((16, 24))
    ref = (F.silu(t64(h) @ t64(w1).T) * (t64(h) @ t64(w3).T)) @ t64(w2).T
    assert np.allclose(O.swiglu_mlp(h, w1, w3, w2), ref.numpy(), atol=1e-10)
    # W3 = 0 turns the branch off
    assert np.all(O.swiglu_mlp(h, w1, 0 * w3, w2) == 0)


# ------------------------------------------------------------------ whole block

def _tiny(dtype="f32", seed=0, wl=W.TINY):
    w = W.block_weights(wl, seed, dtype)
    bi = W.block_inputs(wl, seed, dtype)
    return wl, w, bi


def test_block_zero_gates_and_zero_outputs_are_identity():
    wl, w, bi = _tiny()
    sh = O.BlockShape.of(wl)
    mod = bi.mod.copy()
    mod[:, O.GATE1] = 0
    mod[:, O.GATE2] = 0
    out = O.dit_block(bi.x, mod, w, bi.pos, bi.cu_slots, bi.valid_len, sh)
    assert np.array_equal(out, bi.x.astype(np.float64))
    import dataclasses
    w0 = dataclasses.replace(w, w_o=0 * w.w_o, w2=0 * w.w2)
    out = O.dit_block(bi.x, bi.mod, w0, bi.pos, bi.cu_slots, bi.valid_len, sh)
    assert np.array_equal(out, bi.x.astype(np.float64))


def test_block_slot_roles():
    import dataclasses
    wl, w, bi = _tiny()
    sh = O.BlockShape.of(wl)
    w_mlp_off = dataclasses.replace(w, w2=0 * w.w2)
    x = bi.x.astype(np.float64)
    # with the MLP off, the update is gate1 * y1 and is linear in gate1 only
    base = O.dit_block(bi.x, bi.mod, w_mlp_off, bi.pos, bi.cu_slots, bi.valid_len, sh) - x
    m2 = bi.mod.copy()
    m2[:, O.GATE1] *= 2
    assert np.allclose(O.dit_block(bi.x, m2, w_mlp_off, bi.pos, bi.cu_slots, bi.valid_len, sh) - x, 2 * base)
    m3 = bi.mod.copy()
    m3[:, O.SHIFT2:] = rng.standard_normal(m3[:, O.SHIFT2:].shape)
    assert np.allclose(O.dit_block(bi.x, m3, w_mlp_off, bi.pos, bi.cu_slots, bi.valid_len, sh) - x, base)
    # scale1 = -1 makes the first norm output shift1: the attention branch no
    # longer sees x, so the update is the same for two different x
    m4 = bi.mod.copy()
    m4[:, O.SCALE1] = -1
    x_other = rng.standard_normal(x.shape)
    d1 = O.dit_block(bi.x, m4, w_mlp_off, bi.pos, bi.cu_slots, bi.valid_len, sh) - x
    d2 = O.dit_block(x_other, m4, w_mlp_off, bi.pos, bi.cu_slots, bi.valid_len, sh) - x_other
    assert np.allclose(d1, d2, atol=1e-12)


def test_block_padding_invariance_with_poisoned_pad_rows():
    wl, w, bi = _tiny()
    wlp = wl.replace(pad_to=512)
    bip = W.block_inputs(wlp, 0, "f32")
    x = np.full((512, wl.dim), np.nan, np.float32)
    x[:480] = bi.x
    x[480::2] = np.inf
    mod = np.full((512, 6, wl.dim), np.nan, np.float32)
    mod[:480] = bi.mod
    sh = O.BlockShape.of(wl)
    a = O.dit_block(bi.x, bi.mod, w, bi.pos, bi.cu_slots, bi.valid_len, sh)
    b = O.dit_block(x, mod, w, bip.pos, bip.cu_slots, bip.valid_len, sh)
    assert np.array_equal(a, b[:480])


def test_block_rank_share_matches_world_one():
    """A rank's share, fed what the other ranks would send, equals the world-1
    block on those rows (sequence parallel over tokens, head-parallel attention)."""
    wl, w, bi = _tiny()
    sh1 = O.BlockShape.of(wl)
    full = O.dit_block(bi.x, bi.mod, w, bi.pos, bi.cu_slots, bi.valid_len, sh1, intermediates=True)
    P = 4
    for rank in (1, 3):
        wr = wl.replace(sp_degree=P, rank=rank)
        n = wr.n_loc
        tb, hb, hc = wr.tok_begin, wr.head_begin, wr.head_count
        # what the exchange delivers: every rank's post-norm/RoPE q, k, v of heads [hb, hb+hc)
        qkv_fill = np.stack([full["q"][:, hb:hb + hc], full["k"][:, hb:hb + hc], full["v"][:, hb:hb + hc]], 1)
        o_fill = full["o"][tb:tb + n].copy()
        qkv_fill[tb:tb + n] = 1e30   # local rows must be overwritten by the rank's own values
        o_fill[:, hb:hb + hc] = 1e30
        shr = O.BlockShape.of(wr)
        got = O.dit_block(bi.x[tb:tb + n], bi.mod[tb:tb + n], w, bi.pos[tb:tb + n], bi.cu_slots,
                          bi.valid_len, shr, qkv_attn_fill=qkv_fill, o_local_fill=o_fill)
        assert np.allclose(got, full["x2"][tb:tb + n], atol=1e-12)


def test_block_sampled_rows_equal_full():
    wl, w, bi = _tiny()
    sh = O.BlockShape.of(wl)
    full = O.dit_block(bi.x, bi.mod, w, bi.pos, bi.cu_slots, bi.valid_len, sh)
    rows = np.array([0, 5, 383, 384, 479])
    part = O.dit_block(bi.x, bi.mod, w, bi.pos, bi.cu_slots, bi.valid_len, sh, rows=rows)
    assert np.allclose(part, full[rows], atol=1e-13)


# ------------------------------------------------------------- O9 student loop

def test_timestep_embedding_closed_form():
    e0 = O.timestep_embedding(0.0)
    assert np.array_equal(e0, np.concatenate([np.ones(128), np.zeros(128)]))
    e = O.timestep_embedding(0.75)
    assert np.allclose(e[:128] ** 2 + e[128:] ** 2, 1)
    assert math.isclose(e[0], math.cos(750.0)) and math.isclose(e[128], math.sin(750.0))
    assert math.isclose(e[127], math.cos(750.0 * 1e4 ** (-127 / 128)))


def test_student_loop_special_cases():
    wl = W.TINY.replace(n_blocks=1)
    w = W.block_weights(wl, 0, "f32")
    tw = W.timestep_weights(wl, 0, "f32")
    bi = W.block_inputs(wl, 0, "f32")
    sh = O.BlockShape.of(wl)
    # equal sigmas: no motion
    z = O.student_loop(bi.x, [w], tw, bi.pos, bi.cu_slots, bi.valid_len, sh, (0.5, 0.5, 0.5))
    assert np.array_equal(z, bi.x.astype(np.float64))
    # one step from sigma 1 to 0 with one block: z - block(z)
    z = O.student_loop(bi.x, [w], tw, bi.pos, bi.cu_slots, bi.valid_len, sh, (1.0, 0.0))
    mod = O.timestep_modulation(1.0, tw)[0][None]
    u = O.dit_block(bi.x, mod, w, bi.pos, bi.cu_slots, bi.valid_len, sh)
    assert np.allclose(z, bi.x - u, atol=1e-12)


def test_timestep_modulation_closed_form():
    """W_t2 silu(W_t1 e(sigma)) + table on weights chosen so every value has a
    closed form.  At sigma = 0 the embedding is 128 ones then 128 zeros, so a
    W_t1 row holding a/128 on the cosine half gives the pre-activation a; with
    a = ln 3 the SiLU is ln 3 * sigmoid(ln 3) = (3/4) ln 3, with a = -ln 3 it
    is -(1/4) ln 3, and silu(0) = 0.  W_t2 row (k, c) holds b[k, c] at column c
    only, so slot k of channel c is b[k, c] silu(a_c) + table[block, k, c]."""
    C = 6
    ln3 = math.log(3.0)
    a = np.array([ln3, -ln3, 0.0, ln3, -ln3, 2 * ln3])
    silu_a = np.array([0.75 * ln3, -0.25 * ln3, 0.0, 0.75 * ln3, -0.25 * ln3, 2 * ln3 * 9 / 10])
    w_t1 = np.zeros((C, 256))
    w_t1[:, :128] = a[:, None] / 128.0
    b = (np.arange(6 * C).reshape(6, C) + 1.0) * np.where(np.arange(C) % 2, -0.5, 0.25)
    w_t2 = np.zeros((6 * C, C))
    for k in range(6):
        for c in range(C):
            w_t2[k * C + c, c] = b[k, c]
    table = rng.standard_normal((2, 6, C))
    tw = W.TimestepWeights(w_t1=w_t1, w_t2=w_t2, table=table)
    got = O.timestep_modulation(0.0, tw)
    assert got.shape == (2, 6, C)
    want = b[None] * silu_a[None, None, :] + table
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)
    # at sigma = 0.75 a unit W_t1 row reads one embedding entry, cos(750) or
    # sin(750); the SiLU is then torch's (a library routine)
    w_t1 = np.zeros((C, 256))
    w_t1[np.arange(C), [0, 128, 1, 129, 0, 128]] = [1.0, 1.0, 1.0, 1.0, -2.0, 3.0]
    pre = np.array([math.cos(750.0), math.sin(750.0), math.cos(750.0 * 1e4 ** (-1 / 128)),
                    math.sin(750.0 * 1e4 ** (-1 / 128)), -2 * math.cos(750.0), 3 * math.sin(750.0)])
    tw = W.TimestepWeights(w_t1=w_t1, w_t2=w_t2, table=table)
    got = O.timestep_modulation(0.75, tw)
    want = b[None] * F.silu(t64(pre)).numpy()[None, None, :] + table
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)


def test_block_gated_branch_enters_linearly():
    """Doubling W3 doubles the MLP update exactly (silu sits on the W1 branch)."""
    import dataclasses
    wl, w, bi = _tiny()
    sh = O.BlockShape.of(wl)
    w_att_off = dataclasses.replace(w, w_o=0 * w.w_o)
    x = bi.x.astype(np.float64)
    d1 = O.dit_block(bi.x, bi.mod, w_att_off, bi.pos, bi.cu_slots, bi.valid_len, sh) - x
    w_twice = dataclasses.replace(w_att_off, w3=2 * w.w3)
    d2 = O.dit_block(bi.x, bi.mod, w_twice, bi.pos, bi.cu_slots, bi.valid_len, sh) - x
    assert np.allclose(d2, 2 * d1, atol=1e-12)
    w_w1 = dataclasses.replace(w_att_off, w1=2 * w.w1)
    d3 = O.dit_block(bi.x, bi.mod, w_w1, bi.pos, bi.cu_slots, bi.valid_len, sh) - x
    assert not np.allclose(d3, 2 * d1, atol=1e-6)


def test_block_value_rows_drive_the_attention_update():
    """Zero value projection rows (the last third of Wqkv) silence attention."""
    import dataclasses
    wl, w, bi = _tiny()
    sh = O.BlockShape.of(wl)
    hd = wl.n_heads * wl.head_dim
    wq = w.w_qkv.copy()
    wq[2 * hd:] = 0
    w_v0 = dataclasses.replace(w, w_qkv=wq, w2=0 * w.w2)
    out = O.dit_block(bi.x, bi.mod, w_v0, bi.pos, bi.cu_slots, bi.valid_len, sh)
    assert np.array_equal(out, bi.x.astype(np.float64))


def _brute_block(x, mod, w, pos, n_valid, C, H, D, secs, theta, eps):
    """Direct loops over tokens, heads and dims: one segment [0, n), first n_valid valid."""
    n = len(x)
    E = math.exp

    def modnorm(row, sh, sc):
        mu = sum(row) / C
        var = sum((a - mu) ** 2 for a in row) / C
        return [(a - mu) / math.sqrt(var + eps) * (1 + sc[c]) + sh[c] for c, a in enumerate(row)]

    def mv(wm, vec):  # wm [out][in]
        return [sum(wm[o][c] * vec[c] for c in range(len(vec))) for o in range(len(wm))]

    def angle(p, i):  # pair i of a head row
        if p[0] == 1:
            return p[1] * theta ** (-2 * i / D)
        off = 0
        for ax, d in enumerate(secs):
            if i < off + d // 2:
                return p[1 + ax] * theta ** (-2 * (i - off) / d)
            off += d // 2

    h1 = [modnorm(list(x[t]), mod[t][0], mod[t][1]) for t in range(n)]
    qkv = [mv(w.w_qkv.tolist(), h1[t]) for t in range(n)]
    q = [[[qkv[t][hh * D + c] for c in range(D)] for hh in range(H)] for t in range(n)]
    k = [[[qkv[t][H * D + hh * D + c] for c in range(D)] for hh in range(H)] for t in range(n)]
    v = [[[qkv[t][2 * H * D + hh * D + c] for c in range(D)] for hh in range(H)] for t in range(n)]
    for t in range(n):
        if pos[t][0] == 2:
            continue
        for arr, g in ((q, w.g_q), (k, w.g_k)):
            for hh in range(H):
                r = arr[t][hh]
                rms = math.sqrt(sum(a * a for a in r) / D + eps)
                r = [r[c] / rms * g[c] for c in range(D)]
                out = []
                for i in range(D // 2):
                    a, b = r[2 * i], r[2 * i + 1]
                    phi = angle(pos[t], i)
                    out += [a * math.cos(phi) - b * math.sin(phi), a * math.sin(phi) + b * math.cos(phi)]
                arr[t][hh] = out
    o = [[0.0] * (H * D) for _ in range(n)]
    for t in range(n_valid):
        for hh in range(H):
            s = [sum(q[t][hh][c] * k[j][hh][c] for c in range(D)) / math.sqrt(D) for j in range(n_valid)]
            m = max(s)
            e = [E(a - m) for a in s]
            z = sum(e)
            for c in range(D):
                o[t][hh * D + c] = sum(e[j] * v[j][hh][c] for j in range(n_valid)) / z
    res = []
    for t in range(n):
        y1 = mv(w.w_o.tolist(), o[t])
        x1 = [x[t][c] + mod[t][2][c] * y1[c] for c in range(C)]
        h2 = modnorm(x1, mod[t][3], mod[t][4])
        a = mv(w.w1.tolist(), h2)
        b = mv(w.w3.tolist(), h2)
        g = [a[i] / (1 + E(-a[i])) * b[i] for i in range(len(a))]
        y2 = mv(w.w2.tolist(), g)
        res.append([x1[c] + mod[t][5][c] * y2[c] for c in range(C)])
    return np.array(res)


def test_block_brute_force_tiny():
    C, H, D, Fd, secs = 12, 2, 8, 10, (2, 2, 4)
    r = np.random.default_rng(7)
    w = W.BlockWeights(w_qkv=r.standard_normal((3 * H * D, C)) * 0.5, w_o=r.standard_normal((C, H * D)) * 0.5,
                       w1=r.standard_normal((Fd, C)), w3=r.standard_normal((Fd, C)),
                       w2=r.standard_normal((C, Fd)) * 0.5, g_q=1 + 0.3 * r.standard_normal(D),
                       g_k=1 + 0.3 * r.standard_normal(D))
    pos = np.array([[0, 0, 0, 0], [0, 0, 1, 2], [0, 1, 0, 3], [0, 2, 1, 1], [1, 4, 0, 0], [2, 0, 0, 0]], np.int32)
    x = r.standard_normal((6, C))
    mod = r.standard_normal((6, 6, C)) * 0.3
    sh = O.BlockShape(dim=C, n_heads=H, head_dim=D, ffn_dim=Fd, sections=secs)
    got = O.dit_block(x, mod, w, pos, np.array([0, 6]), np.array([5]), sh)
    ref = _brute_block(x, mod, w, pos, 5, C, H, D, secs, 1e4, 1e-6)
    assert np.allclose(got, ref, atol=1e-11)


# ----------------------------------------------------- output frames (f)

def _u8_exact(x32):
    """The value rule evaluated independently: every step in float64 (where
    each intermediate is exact), rounded to float32 explicitly, and the final
    half-to-even rounding done by hand on the exact float32 product."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    v = (x / 2.0 + 0.5).astype(np.float32).astype(np.float64)   # exact in f64, one f32 rounding
    v = np.where(np.isnan(v), 0.0, v)
    v = np.clip(v, 0.0, 1.0)
    w = (v * 255.0).astype(np.float32).astype(np.float64)        # exact in f64, one f32 rounding
    r = np.floor(w)
    frac = w - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2.0) == 1.0))
    return (r + up).astype(np.uint8)


def test_frames_closed_form_values():
    x = np.array([-1.0, 1.0, 0.0, 3.0, -7.0, np.nan, np.inf, -np.inf, 0.5, -0.5],
                 dtype=np.float32)
    want = [0, 255, 128, 255, 0, 0, 255, 0, 191, 64]  # 0 -> 127.5 -> 128 (even); 0.5 -> 191.25
    got = O.frames_to_u8(np.repeat(x.reshape(1, 1, 1, 1, -1), 3, axis=1), 0)[0, 0, 0, :, 0]
    assert got.tolist() == want


def test_frames_against_exact_evaluation():
    # every bf16 value in [-2, 2] plus random float32 values
    bits = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    xs = bits.view(np.float32)
    xs = xs[np.isfinite(xs) & (np.abs(xs) <= 2.0)]
    xs = np.concatenate([xs, rng.uniform(-1.2, 1.2, 200_000).astype(np.float32)])
    got = O.frames_to_u8(np.repeat(xs.reshape(1, 1, 1, 1, -1), 3, axis=1), 1)[0, 0, 0, 0]
    np.testing.assert_array_equal(got, _u8_exact(xs))


def test_frames_ties_round_to_even():
    # float32 inputs whose product v * 255 is exactly k + 0.5 exist; each must go to the even side
    k = np.arange(255, dtype=np.float64)
    cand = []
    for d in range(-64, 65):
        x = (2.0 * (k + 0.5) / 255.0 - 1.0).astype(np.float32)
        x = np.nextafter(x, np.float32(np.inf) if d > 0 else np.float32(-np.inf)) if d else x
        cand.append(x)
    xs = np.unique(np.concatenate(cand))
    v = (xs.astype(np.float64) / 2 + 0.5).astype(np.float32)
    w = (v.astype(np.float64) * 255).astype(np.float32).astype(np.float64)
    ties = xs[(w - np.floor(w)) == 0.5]
    assert ties.size > 0
    u = O.frames_to_u8(np.repeat(ties.reshape(1, 1, 1, 1, -1), 3, axis=1), 0)[0, 0, 0, :, 0]
    assert np.all(u % 2 == 0)


def test_frames_monotone_and_layouts_agree():
    x = W.frames(3, 2, 3, 4, 24)
    a = O.frames_to_u8(x, 0)
    p = O.frames_to_u8(x, 1)
    B, _, T, H, Wd = x.shape
    for b, c, t, h, w in [(0, 0, 0, 0, 0), (1, 2, 2, 3, 23), (1, 1, 0, 2, 7), (0, 2, 1, 1, 16)]:
        assert a[b, t, h, w, c] == p[b, t, c, h, w] == _u8_exact(x[b, c, t, h, w:w + 1])[0]
    s = np.sort(rng.uniform(-1.5, 1.5, 4096).astype(np.float32))
    u = O.frames_to_u8(np.repeat(s.reshape(1, 1, 1, 1, -1), 3, axis=1), 0)[0, 0, 0, :, 0]
    assert np.all(np.diff(u.astype(np.int32)) >= 0)
    # uint8 BTHWC is the contiguous, interleaved layout
    assert a.flags["C_CONTIGUOUS"] and a.shape == (B, T, H, Wd, 3)


# ----------------------------------------- FP8 (MX e4m3) operands (f)

def _e4m3_decode(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1 + m / 8) * 2.0 ** (e - 7)


def test_e4m3_grid_fixed_points_and_ties():
    vals = sorted({_e4m3_decode(c) for c in range(256) if (c & 0x7F) != 0x7F})
    assert max(vals) == 448.0 and min(v for v in vals if v > 0) == 2.0 ** -9
    v = np.array(vals)
    np.testing.assert_array_equal(O.e4m3_round(v), v)
    pos = v[v >= 0]
    mids = (pos[:-1] + pos[1:]) / 2
    got = O.e4m3_round(mids)
    # each midpoint goes to the neighbour whose code (mantissa) is even
    codes = {_e4m3_decode(c): c for c in range(0x7F)}
    for m, lo, hi, g in zip(mids, pos[:-1], pos[1:], got):
        even = lo if codes[lo] % 2 == 0 else hi
        assert g == even, (m, lo, hi, g)
    assert O.e4m3_round(np.array([460.0, 464.0]))[1] == 448.0


def test_e8m0_rule_against_search():
    a = np.concatenate([rng.uniform(0, 1, 500) * 10.0 ** rng.integers(-6, 6, 500),
                        [448.0, 448.0 * 2 ** -3, np.nextafter(448.0, 1e9), 1.0, 0.0]])
    got = O.e8m0_exponent(a)
    for ai, gi in zip(a, got):
        want = 0 if ai == 0 else min(e for e in range(-127, 128) if ai <= 448.0 * 2.0 ** e)
        assert gi == want, (ai, gi, want)


def test_mx_quantize_error_bound_and_top_binade():
    x = (rng.standard_normal((8, 128)) * 10.0 ** rng.integers(-3, 3, (8, 1))).astype(np.float32)
    q, e = O.mx_quantize(x)
    d = O.mx_dequantize(q, e)
    xb = x.astype(np.float64).reshape(8, 4, 32)
    amax = np.abs(xb).max(-1)
    # the block's largest magnitude lands in the top binade of e4m3 (224..448]
    assert np.all(amax / np.ldexp(1.0, e) > 224.0) and np.all(amax / np.ldexp(1.0, e) <= 448.0)
    # rounding error: half a quantum of the element's binade (relative 2^-4), or 2^-10 * 2^e below normals
    err = np.abs(d - x).reshape(8, 4, 32)
    bound = np.maximum(np.abs(xb) * 2.0 ** -4, np.ldexp(1.0, e)[..., None] * 2.0 ** -10)
    assert np.all(err <= bound + 1e-300)


def test_fp8_operand_attention_close_to_exact():
    case = W.varlen_case(seed=5, lengths=(100, 37), n_buf=160, n_heads=2, head_dim=64, dtype="bf16")
    ref = O.varlen_attention(case.q, case.k, case.v, case.cu_slots, case.valid_len)
    got = O.varlen_attention_fp8_operands(case.q, case.k, case.v, case.cu_slots, case.valid_len)
    valid = np.zeros(case.q.shape[0], bool)
    for s in range(len(case.valid_len)):
        valid[case.cu_slots[s]:case.cu_slots[s] + case.valid_len[s]] = True
    diff = np.abs(got[valid] - ref[valid])
    assert diff.max() < 0.1 and diff.mean() < 0.01
    # the quantization changes the result (this is not the exact path)
    assert diff.max() > 1e-4


def test_fp8_weights_hand_derived():
    """The FP8 path's softmax weights, e4m3(2^(8 + s - M)) with M = ceil(row
    max), on scores whose values are worked out by hand: max 0.5 gives M = 1,
    2^7.5 = 181.02 -> 176 (grid step 16 in [128, 256)), 2^6.5 = 90.51 -> 88
    (step 8), 2^4.75 = 26.91 -> 26 (step 2); integer scores give exact powers
    of two (the row max 256); a score 24 below an integer max lands in the
    subnormal range (2^-16 -> 0)."""
    np.testing.assert_array_equal(O.fp8_weights([[0.5, -0.5, -2.25]]), [[176.0, 88.0, 26.0]])
    np.testing.assert_array_equal(O.fp8_weights([[0.0, -1.0, -3.0, 2.0]]), [[64.0, 32.0, 8.0, 256.0]])
    np.testing.assert_array_equal(O.fp8_weights([[3.0, -5.0, -13.0, -14.0, -21.0]]),
                                  [[256.0, 1.0, 2.0 ** -8, 2.0 ** -9, 0.0]])


def test_fp8_weights_grid_and_shift_rules():
    """Every weight is an e4m3 value (decoded from the byte definition) and the
    nearest one to 2^(8 + s - M); the row's largest weight lies in [128, 256]
    (2^(8 + max - M) is in (128, 256], and rounding can reach 128);
    adding an integer to a row leaves its weights unchanged."""
    grid = np.array(sorted({_e4m3_decode(c) for c in range(0x7F)}))
    sc = rng.uniform(-12, 6, (40, 50))
    w = O.fp8_weights(sc)
    assert np.all(np.isin(w, grid))
    x = np.exp2(sc - np.ceil(sc.max(1, keepdims=True)) + 8.0)
    dist = np.abs(grid[None, None, :] - x[..., None])
    assert np.all(np.abs(w - x) <= dist.min(-1) + 1e-12)
    assert np.all((w.max(1) >= 128) & (w.max(1) <= 256))
    np.testing.assert_array_equal(O.fp8_weights(sc + 3.0), w)
    assert not np.array_equal(O.fp8_weights(sc + 0.37), w)


def test_fp8_rounded_weights_attention_bound():
    """Rounding the weights moves each output by at most
    2 * 2^-4 / (1 - 2^-4) * max|v| when every weight is an e4m3 normal (each is
    off by at most 2^-4 relative), and it does move it; the weights of a row
    whose scores are integers are exact, so there the output is the
    unrounded one."""
    case = W.varlen_case(seed=5, lengths=(100, 37), n_buf=160, n_heads=2, head_dim=64, dtype="bf16")
    args = (case.q, case.k, case.v, case.cu_slots, case.valid_len)
    r = O.varlen_attention_fp8_operands(*args)
    e = O.varlen_attention_fp8_operands(*args, round_p=False)
    bound = 2 * 2.0 ** -4 / (1 - 2.0 ** -4) * np.abs(case.v).max()
    assert np.abs(r - e).max() <= bound and np.abs(r - e).max() > 1e-4
    # one query whose folded grid value meets each key in an integer score
    g = np.random.default_rng(3)
    d = 64
    c = float(O.fp8_fold(d))
    qd = np.zeros((1, 1, d))
    qd[0, 0, 0] = 1.0
    kd = np.zeros((9, 1, d))
    kd[:, 0, 0] = [0, -1, 2, -3, 1, -6, 3, -2, 2]
    vd = O.mx_dequantize(*O.mx_quantize(g.standard_normal((1, d, 32)).astype(np.float32)))[..., :9].transpose(2, 0, 1)
    qin = (qd / c).astype(np.float32)
    assert O.mx_dequantize(*O.mx_quantize(qin, fold=c))[0, 0, 0] == 1.0
    qb = np.zeros((9, 1, d), np.float32)
    qb[0] = qin[0]
    cu, vl = np.array([0, 9]), np.array([9])
    got = O.varlen_attention_fp8_operands(qb, kd.astype(np.float32), vd.astype(np.float32), cu, vl)
    np.testing.assert_array_equal(got[0], O.varlen_attention_fp8_operands(
        qb, kd.astype(np.float32), vd.astype(np.float32), cu, vl, round_p=False)[0])


def test_fp8_operands_ignore_pad_rows():
    """NaN and Inf in pad rows of q, k, v change nothing (only valid rows are
    quantized), and no invalid cast happens on the way."""
    case = W.varlen_case(seed=9, lengths=(70, 33), n_buf=128, n_heads=1, head_dim=64, dtype="bf16")
    args = (case.cu_slots, case.valid_len)
    base = O.varlen_attention_fp8_operands(case.q, case.k, case.v, *args)
    valid = np.zeros(case.q.shape[0], bool)
    for s in range(len(case.valid_len)):
        valid[case.cu_slots[s]:case.cu_slots[s] + case.valid_len[s]] = True
    q, k, v = (a.copy() for a in (case.q, case.k, case.v))
    q[~valid], k[~valid], v[~valid] = np.nan, np.inf, -np.inf
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        got = O.varlen_attention_fp8_operands(q, k, v, *args)
    np.testing.assert_array_equal(got, base)


def test_mx_quantize_exact_on_representable_blocks():
    """Blocks already of the form e4m3 value x 2^E, with the largest magnitude in
    the top binade (224..448], come back unchanged, exponent and all."""
    grid = np.array([_e4m3_decode(c) for c in range(0x7F)])
    top = grid[grid > 224.0]
    e = rng.integers(-20, 10, (6, 4))
    codes = rng.choice(np.concatenate([grid, -grid]), (6, 4, 32))
    codes[..., 5] = rng.choice(top, (6, 4)) * rng.choice([-1.0, 1.0], (6, 4))
    x = (codes * np.ldexp(1.0, e)[..., None]).reshape(6, 128).astype(np.float32)
    q, got_e = O.mx_quantize(x)
    np.testing.assert_array_equal(got_e, e)
    np.testing.assert_array_equal(O.mx_dequantize(q, got_e), x)


# ------------------------------------------------- FP8 (MX e4m3) GEMM operands

def test_fp8_linear_exact_on_grid_and_power_of_two_equivariant():
    """Operands already on the MX grid pass through unchanged, so the product is
    the plain matmul; scaling an operand by 2^j scales the result by 2^j exactly
    (the block exponent absorbs it)."""
    grid = np.array([_e4m3_decode(c) for c in range(0x7F)])
    top = grid[grid > 224.0]

    def on_grid(rows, k):
        e = rng.integers(-12, 4, (rows, k // 32))
        c = rng.choice(np.concatenate([grid, -grid]), (rows, k // 32, 32))
        c[..., 0] = rng.choice(top, (rows, k // 32))
        return (c * np.ldexp(1.0, e)[..., None]).reshape(rows, k).astype(np.float32)

    x, w = on_grid(7, 96), on_grid(5, 96)
    np.testing.assert_array_equal(O.linear_fp8_operands(x, w), x.astype(np.float64) @ w.astype(np.float64).T)
    # both operands are quantized: one off-grid operand alone moves the result
    xo = rng.standard_normal((7, 96)).astype(np.float32)
    wo = (rng.standard_normal((5, 96)) * 0.02).astype(np.float32)
    assert not np.array_equal(O.linear_fp8_operands(xo, w), xo.astype(np.float64) @ w.astype(np.float64).T)
    assert not np.array_equal(O.linear_fp8_operands(x, wo), x.astype(np.float64) @ wo.astype(np.float64).T)
    xr = rng.standard_normal((6, 128)).astype(np.float32)
    wr = (rng.standard_normal((9, 128)) * 0.02).astype(np.float32)
    base = O.linear_fp8_operands(xr, wr)
    for j in (-5, 3):
        np.testing.assert_array_equal(O.linear_fp8_operands(np.ldexp(xr, j), wr), np.ldexp(base, j))
        np.testing.assert_array_equal(O.linear_fp8_operands(xr, np.ldexp(wr, j)), np.ldexp(base, j))


def test_fp8_linear_error_bound_and_zero_padding():
    """Each operand element is off by at most 2^-4 relative (normal range), so
    |y - y_exact| <= sum_k |x_k w_k| (2 * 2^-4 + 2^-8); appending zero columns
    to both operands changes nothing."""
    x = rng.standard_normal((11, 192)).astype(np.float32)
    w = (rng.standard_normal((13, 192)) * 0.02).astype(np.float32)
    got = O.linear_fp8_operands(x, w)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    bound = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T * (2 * 2.0 ** -4 + 2.0 ** -8)
    assert np.all(np.abs(got - exact) <= bound)
    assert np.abs(got - exact).max() > 0  # the quantization is applied
    xp = np.concatenate([x, np.zeros((11, 64), np.float32)], axis=1)
    wp = np.concatenate([w, np.zeros((13, 64), np.float32)], axis=1)
    np.testing.assert_array_equal(O.linear_fp8_operands(xp, wp), got)
    # each row of x is quantized on its own: the result for a row does not depend on the others
    np.testing.assert_array_equal(O.linear_fp8_operands(x[3:4], w), got[3:4])


# ------------------------------------------------------------ Skip-Softmax

def _blocky_case(n=320, h=1, d=64, far=(1, 3), seed=7):
    """Every query is 4 e0 + N(0, 0.3^2) noise; keys are N(0, 1) except in the
    64-key blocks listed in `far`, whose keys are -55 e0 + N(0, 1): their scores
    sit near -40 (log2 units, scale 1/8) while the others are O(1), so with
    t = -10 exactly the far blocks fall below the threshold."""
    g = np.random.default_rng(seed)
    e0 = np.zeros(d)
    e0[0] = 1.0
    q = 4.0 * e0 + 0.3 * g.standard_normal((n, h, d))
    k = g.standard_normal((n, h, d))
    v = g.standard_normal((n, h, d))
    for b in far:
        k[b * 64:(b + 1) * 64] -= 55.0 * e0
    return q, k, v


def test_skip_softmax_reduces_to_exact_and_to_kept_blocks():
    q, k, v = _blocky_case()
    n = q.shape[0]
    cu, vl = np.array([0, n]), np.array([n])
    exact = O.varlen_attention(q, k, v, cu, vl)
    # no threshold to cross: identical to exact attention
    np.testing.assert_allclose(O.varlen_attention_skip(q, k, v, cu, vl, -1e9), exact, rtol=0, atol=1e-12)
    # t = -10: the far blocks are skipped, so each row is exact attention over the kept keys
    got = O.varlen_attention_skip(q, k, v, cu, vl, -10.0)
    keep = np.ones(n, bool)
    keep[64:128] = keep[192:256] = False
    scale = 1 / np.sqrt(q.shape[-1])
    want = np.stack([O.attention_dense(q[:, 0], k[keep, 0], v[keep, 0], scale)], axis=1)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # the skipped weight is tiny: the result stays within 2^-10 * 128 * max|v| of exact
    assert np.abs(got - exact).max() <= 2.0 ** -10 * 128 * np.abs(v).max()
    assert np.abs(got - exact).max() > 0


def test_skip_softmax_first_block_and_group_rule():
    """The first block is always kept, and one row of a group that still needs a
    block keeps it for the whole group."""
    q, k, v = _blocky_case(far=(0,))
    n = q.shape[0]
    cu, vl = np.array([0, n]), np.array([n])
    got = O.varlen_attention_skip(q, k, v, cu, vl, -10.0)
    np.testing.assert_allclose(got, O.varlen_attention(q, k, v, cu, vl), rtol=1e-10, atol=1e-12)
    q2, k2, v2 = _blocky_case(far=(2,))
    q2[5] = -q2[5]          # row 5 of group 0 now prefers block 2
    got2 = O.varlen_attention_skip(q2, k2, v2, cu, vl, -10.0)
    exact2 = O.varlen_attention(q2, k2, v2, cu, vl)
    np.testing.assert_allclose(got2[:32], exact2[:32], rtol=1e-10, atol=1e-12)   # group 0 keeps block 2
    assert np.abs(got2[32:64] - exact2[32:64]).max() > 0                     # group 1 skips it


def test_fp8_skip_softmax_on_grid_operands_is_the_skip_rule():
    """On operands already on the MX-e4m3 grid the FP8 oracle quantizes nothing
    away, so with a threshold it must be the Skip-Softmax oracle itself."""
    q, k, v = _blocky_case()
    n, h, d = q.shape
    # far blocks at ~-12 log2 units (not -40), so that dropping them shows at t = -6
    k[64:128, :, 0] += 38.0
    k[192:256, :, 0] += 38.0
    cu, vl = np.array([0, n]), np.array([n])
    c = O.fp8_fold(d)
    # grid values of the folded Q (scores in log2 units), and a Q that folds onto them
    qd = O.mx_dequantize(*O.mx_quantize(q.astype(np.float32), fold=c))
    qin = (qd / np.float64(c)).astype(np.float32)
    # folding the scale back in lands on the same grid values
    assert np.array_equal(O.mx_dequantize(*O.mx_quantize(qin, fold=c)), qd)
    kd = O.mx_dequantize(*O.mx_quantize(k.astype(np.float32)))
    vq, ve = O.mx_quantize(v.astype(np.float32).transpose(1, 2, 0))   # blocks of 32 keys
    vd = O.mx_dequantize(vq, ve).transpose(2, 0, 1)
    got = O.varlen_attention_fp8_operands(qin, kd, vd, cu, vl, skip_log2=-6.0, round_p=False)
    # scores q.k in log2 units: scale 1/log2(e) undoes the oracle's own log2(e)
    want = O.varlen_attention_skip(qd, kd, vd, cu, vl, -6.0, scale=1.0 / np.log2(np.e))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-9)
    plain = O.varlen_attention_fp8_operands(qin, kd, vd, cu, vl, round_p=False)
    assert np.abs(got - plain).max() > 1e-6          # the far blocks were dropped
    np.testing.assert_allclose(O.varlen_attention_fp8_operands(qin, kd, vd, cu, vl, skip_log2=-1e9,
                                                               round_p=False), plain, rtol=0, atol=1e-12)
    # with the weights rounded as the FP8 path stores them: the same rule, on the
    # kept keys only, each row's weights e4m3(2^(8 + s - M)) of its kept scores
    got_r = O.varlen_attention_fp8_operands(qin, kd, vd, cu, vl, skip_log2=-6.0)
    keep = np.ones(n, bool)
    keep[64:128] = keep[192:256] = False
    sc = qd[:, 0] @ kd[keep, 0].T
    wts = O.fp8_weights(sc)
    np.testing.assert_allclose(got_r[:, 0], (wts @ vd[keep, 0]) / wts.sum(1, keepdims=True), rtol=0, atol=1e-12)


def test_skip_softmax_sampled_groups_equal_the_full_result():
    q, k, v = _blocky_case(n=400)
    k[64:128, :, 0] += 38.0            # far blocks near -12 log2 units, skipped at t = -6
    cu, vl = np.array([0, 400]), np.array([400])
    full = O.varlen_attention_skip(q, k, v, cu, vl, -6.0)
    rows = np.r_[32:96, 384:400]        # groups 1-2 and the last, shorter group
    part = O.varlen_attention_skip(q[rows], k, v, cu, vl, -6.0, q_rows=rows)
    np.testing.assert_allclose(part, full[rows], rtol=0, atol=1e-13)
    with pytest.raises(AssertionError):
        O.varlen_attention_skip(q[40:60], k, v, cu, vl, -6.0, q_rows=np.arange(40, 60))
