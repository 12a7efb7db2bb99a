#!/usr/bin/env python3
"""Benchmark: one DiT block forward on one GPU's share of a packed audio-video
sequence (default: the 10 s request at 1344x768, 24 FPS), bf16, on MI355X.

A "step" is one h3_dit_block_forward call (all steps of the block: modulated
norm, QKV projection, Q/K RMSNorm+RoPE, head-slice exchange copies, varlen
attention over the full sequence, output projection with gated residual,
modulated norm, SwiGLU with gated residual) over inputs already resident in
HBM.  Prints ONE JSON line.

Per-kernel figures (attention TFLOP/s, fused-op GB/s) come from HIP events
around each C entry point on the stream it is launched on.  The CPU baseline
is the float64 oracle, timed on this host on a bounded row sample and
extrapolated by row count.

The default run then frees the 10 s share and adds the other configurations
of the request sweep as extra keys: the 8k varlen attention case (bf16 and
FP8), one block on the 5 s share, and the four-forward 15 s student loop
(bf16, then FP8 with only the MX weights resident, with peak device bytes of
both).

  python bench.py [--steps K] [--warmup W] [--config share10s|share5s|loop15s|tiny]
                  [--no-cpu-baseline] [--no-extra] [--only attn|attn_fp8|copy|block]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published
METRIC = "varlen attn TFLOP/s + fused-op HBM GB/s; DiT-block ms, 10 s shape, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")
ATTN_SRC = os.path.join(ROOT, "audio_video_diffusion_block_amd", "csrc", "k_attn.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="share10s")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", choices=["", "attn", "attn_fp8", "attn8k", "copy", "block"])
    ap.add_argument("--op-reps", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other configs (8k varlen attention, 5 s block, 15 s loop)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workload

def algorithmic_work(wl):
    """Per-launch algorithmic FLOPs and bytes of every step (each input read once,
    each output written once; bf16 = 2 bytes)."""
    n, c, h, d, f = wl.n_loc, wl.dim, wl.n_heads, wl.head_dim, wl.ffn_dim
    hc = wl.head_count if wl.share_mode else h
    nv = wl.n_valid
    es = 2
    mod_rows = n if wl.mod_per_token else 1
    return {
        "attn_flop": 4.0 * d * hc * nv * nv,
        "qkv_flop": 2.0 * n * c * 3 * h * d,
        "out_flop": 2.0 * n * h * d * c,
        "w13_flop": 2.0 * n * c * 2 * f,
        "w2_flop": 2.0 * n * f * c,
        # modulated norm: read x, shift, scale; write h
        "modnorm_bytes": es * (2 * n * c + 2 * mod_rows * c),
        # Q/K RMSNorm + RoPE: read and write q and k (positions: 16 B/token)
        "qknorm_bytes": es * 2 * 2 * n * h * d + 16 * n,
    }


def make_inputs(wl, seed):
    import numpy as np
    import workloads as W
    t0 = time.time()
    w = W.block_weights(wl, seed, "bf16")
    bi = W.block_inputs(wl, seed, "bf16")
    log(f"generated inputs in {time.time() - t0:.1f}s")
    return w, bi


def to_dev(a, dtype=None):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        return t.to("cuda").to(dtype)
    return t.to("cuda")


# ----------------------------------------------------------------- timing

class EventTimer:
    """HIP events on the stream the kernels are launched on."""

    def __init__(self, stream):
        import torch
        self.torch = torch
        self.stream = stream

    def time(self, fn, reps, warm=0):
        torch = self.torch
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        for _ in range(warm):
            fn()
        s.record(self.stream)
        for _ in range(reps):
            fn()
        e.record(self.stream)
        e.synchronize()
        return s.elapsed_time(e) / reps  # ms per call


def copy_rate(timer):
    """HBM rate of a plain 1 GiB device-to-device copy (torch's copy kernel):
    the practical ceiling the elementwise passes are read against; bytes =
    read + written."""
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    ms = timer.time(lambda: b.copy_(a), 20, warm=2)
    del a, b
    return 2.0 * (1 << 30) / ms / 1e6


def traffic_record():
    """HBM bytes per attention launch from committed rocprof counters, if they were
    taken on the current attention source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    src_hash = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    if rec.get("k_attn_sha256") != src_hash:
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------- cpu baseline

def cpu_baseline(wl, w, bi, work, attn_rows=2048, local_rows=4096):
    """The float64 oracle on this host, on a bounded sample of the same workload:
    attention for `attn_rows` query rows of the head slice against every key
    (scaled by N / attn_rows), and the row-local steps (modulated norms, QKV
    projection, Q/K RMSNorm+RoPE, output projection, residuals, SwiGLU) for
    `local_rows` token rows (scaled by n_loc / local_rows).  Both scalings are
    exact in work."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    import oracle as O
    rng = np.random.default_rng(0)
    hc = wl.head_count if wl.share_mode else wl.n_heads
    D = wl.head_dim
    # attention sample
    if wl.share_mode:
        qkv = bi.qkv_attn
        q_all, k_all, v_all = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    else:
        g = np.random.default_rng(1)
        q_all, k_all, v_all = (g.standard_normal((wl.n_loc, hc, D)).astype(np.float32) for _ in range(3))
    qrows = np.sort(rng.choice(wl.n_valid, size=attn_rows, replace=False))
    t0 = time.perf_counter()
    O.varlen_attention(q_all[qrows], k_all, v_all, bi.cu_slots, bi.valid_len, q_rows=qrows)
    t_attn = time.perf_counter() - t0
    # row-local sample
    rows = np.sort(rng.choice(wl.n_loc, size=local_rows, replace=False))
    mod = bi.mod[rows] if bi.mod.shape[0] > 1 else bi.mod
    H = wl.n_heads
    t0 = time.perf_counter()
    h1 = O.modulated_norm(bi.x[rows], mod[:, 0], mod[:, 1], wl.eps_mod)
    qkv_r = O.linear(h1, w.w_qkv).reshape(len(rows), 3, H, D)
    O.qk_norm_rope(qkv_r[:, 0], qkv_r[:, 1], bi.pos[rows], w.g_q, w.g_k, wl.sections, wl.theta, wl.eps_qk)
    o = bi.o_local[rows].reshape(len(rows), -1) if bi.o_local is not None else qkv_r[:, 2].reshape(len(rows), -1)
    x1 = O.gated_residual(bi.x[rows], mod[:, 2], O.linear(o, w.w_o))
    h2 = O.modulated_norm(x1, mod[:, 3], mod[:, 4], wl.eps_mod)
    O.gated_residual(x1, mod[:, 5], O.swiglu_mlp(h2, w.w1, w.w3, w.w2))
    t_local = time.perf_counter() - t0
    full_s = t_attn * wl.n_valid / attn_rows + t_local * wl.n_loc / local_rows
    flop = work["attn_flop"] + work["qkv_flop"] + work["out_flop"] + work["w13_flop"] + work["w2_flop"]
    log(f"oracle: attention {attn_rows} rows {t_attn:.1f}s, row-local {local_rows} rows {t_local:.1f}s, "
        f"full block extrapolated {full_s:.0f}s")
    return {"value": flop / full_s / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"float64 numpy oracle: attention for {attn_rows} query rows x {hc} heads against "
                       f"all {wl.n_valid} keys ({t_attn:.1f}s, scaled by N/{attn_rows}) + row-local steps "
                       f"for {local_rows} of {wl.n_loc} token rows ({t_local:.1f}s, scaled by "
                       f"n_loc/{local_rows}); extrapolated full block {full_s:.0f}s")}



# ------------------------------------------------------------ student loop

def loop_measure(h3, torch, W, seed, steps, warmup):
    """Four-forward student loop on the 15 s share: 8 blocks with their own weights,
    modulation regenerated per sigma from the timestep embedding, Euler update.
    Timed in bf16, then with FP8 attention and FP8 projections with only the MX
    weights resident (the bf16 copies freed first).  Peak device bytes are the
    caching allocator's high-water mark over each run, counted from what was
    allocated when it started (inputs, weights, workspaces and activations of
    the loop itself)."""
    wl = W.LOOP_15S
    bf = torch.bfloat16
    timer = EventTimer(torch.cuda.current_stream())
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    t0 = time.time()
    blocks = []
    for b in range(wl.n_blocks):
        w = W.block_weights(wl, seed, "bf16", block=b)
        blocks.append({k: to_dev(getattr(w, k), bf) for k in ("w_qkv", "w_o", "w1", "w3", "w2", "g_q", "g_k")})
        del w
    tw = W.timestep_weights(wl, seed, "bf16")
    bi = W.block_inputs(wl, seed, "bf16")
    log(f"generated and uploaded loop inputs in {time.time() - t0:.1f}s")
    H, D, C = wl.n_heads, wl.head_dim, wl.dim
    hc = wl.head_count
    z0 = to_dev(bi.x, bf)
    z = z0.clone()
    x = z0.clone()
    t1, t2, tab = to_dev(tw.w_t1, bf), to_dev(tw.w_t2, bf), to_dev(tw.table, bf)
    mods = torch.empty((wl.n_blocks, 6, C), dtype=bf, device="cuda")
    pos, cu, vl = to_dev(bi.pos), to_dev(bi.cu_slots), to_dev(bi.valid_len)
    max_len = int(bi.valid_len.max())
    share = dict(qkv_attn=to_dev(bi.qkv_attn.reshape(wl.n_pad_total, -1), bf),
                 o_attn=torch.zeros((wl.n_pad_total, hc * D), dtype=bf, device="cuda"),
                 o_local=to_dev(bi.o_local.reshape(wl.n_loc, -1), bf), tok_begin=wl.tok_begin,
                 head_begin=wl.head_begin, head_count=hc)
    del bi
    tws = torch.empty(max(h3.timestep_workspace_size(C), 16), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()  # the upload's fp32 staging copies are not the loop's
    sig = W.STUDENT_SIGMAS
    fwd_ms = []

    def run(cfg, weights, ws, record=False):
        z.copy_(z0)
        x.copy_(z0)
        for k in range(len(sig) - 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            h3.h3_timestep_modulation(sig[k], t1, t2, tab, mods, ws=tws)
            for b in range(wl.n_blocks):
                h3.h3_dit_block_forward(cfg, weights[b], x, mods[b:b + 1], pos, cu, vl, max_len, ws=ws, **share)
            h3.h3_euler_update(z, x, x, sig[k], sig[k + 1])
            e1.record()
            if record:
                fwd_ms.append((e0, e1))

    cfg = h3.block_config(C, H, D, wl.ffn_dim, wl.sections, wl.theta, wl.eps_qk, wl.eps_mod, 0, bf)
    ws = torch.empty(h3.block_workspace_size(cfg, wl.n_loc, wl.n_pad_total, 1, hc), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        run(cfg, blocks, ws)
    torch.cuda.synchronize()
    loop_ms = timer.time(lambda: run(cfg, blocks, ws, record=True), steps)
    per_fwd = [a.elapsed_time(b) for a, b in fwd_ms[-(len(sig) - 1):]]
    peak_bf16 = torch.cuda.max_memory_allocated() - base
    # FP8: MX weights quantized once (untimed), the bf16 projection weights freed
    blocks8 = []
    for bw in blocks:
        blocks8.append({"mx": h3.block_weights_mx(bw), "g_q": bw["g_q"], "g_k": bw["g_k"]})
        for key in ("w_qkv", "w_o", "w1", "w3", "w2"):
            del bw[key]
    del blocks, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    cfg8 = h3.block_config(C, H, D, wl.ffn_dim, wl.sections, wl.theta, wl.eps_qk, wl.eps_mod, 0, bf,
                           attn_fp8=True, gemm_fp8=True)
    ws8 = torch.empty(h3.block_workspace_size(cfg8, wl.n_loc, wl.n_pad_total, 1, hc), dtype=torch.uint8,
                      device="cuda")
    for _ in range(warmup):
        run(cfg8, blocks8, ws8)
    torch.cuda.synchronize()
    loop8_ms = timer.time(lambda: run(cfg8, blocks8, ws8), steps)
    peak_fp8 = torch.cuda.max_memory_allocated() - base
    del blocks8, ws8, share, z, x, z0, mods, tws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    work = algorithmic_work(wl)
    blk_flop = work["attn_flop"] + work["qkv_flop"] + work["out_flop"] + work["w13_flop"] + work["w2_flop"]
    total_flop = blk_flop * wl.n_blocks * (len(sig) - 1)
    return {"loop_ms": loop_ms, "ms_per_forward": per_fwd,
            "ms_per_block": loop_ms / (wl.n_blocks * (len(sig) - 1)), "TFLOP/s": total_flop / loop_ms / 1e9,
            "fp8_loop_ms": loop8_ms, "fp8_ms_per_forward": loop8_ms / (len(sig) - 1),
            "fp8_speedup": loop_ms / loop8_ms,
            "peak_device_bytes_bf16": peak_bf16, "peak_device_bytes_fp8": peak_fp8,
            "peak_fp8_vs_bf16": peak_fp8 / peak_bf16,
            "workload": f"{wl.name}: {wl.n_blocks} DiT blocks x {len(sig) - 1} forwards, rank {wl.rank} of "
                        f"{wl.sp_degree} share (n_loc={wl.n_loc}; attention over N={wl.n_valid}, {hc} of {H} "
                        f"heads x {D})",
            "fp8_note": "FP8 attention and FP8 projections (MX e4m3 operands), only the MX weights resident; "
                        "parity at these shapes: tests/test_gpu_fp8_attn.py, tests/test_gpu_fp8_gemm.py"}


def run_loop_bench(args, h3, torch, W):
    """--config loop15s: the student loop alone, as the bench line."""
    wl = W.LOOP_15S
    steps = max(args.steps, 1)
    r = loop_measure(h3, torch, W, args.seed, steps, args.warmup)
    out = {
        "metric": "four-forward student loop, 15 s share: loop ms and ms per forward", "value": r["TFLOP/s"],
        "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": r["loop_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": r["workload"], "n_valid": wl.n_valid, "n_loc": wl.n_loc,
                   "blocks": wl.n_blocks, "forwards": len(W.STUDENT_SIGMAS) - 1,
                   "parallelism": "1 GPU (rank-share stand-in)"},
    }
    out.update({k: v for k, v in r.items() if k != "workload"})
    print(json.dumps(out))


def varlen8k_measure(h3, torch, W, timer, reps=20):
    """The 8k varlen attention case: 8 heads x 128, segments 4032/1500/17 with random
    suffix pads in an 8192-row buffer; bf16 and FP8 kernels."""
    c = W.varlen_case(seed=0, dtype="bf16")
    bf = torch.bfloat16
    H, D = c.n_heads, c.head_dim
    q, k, v = (to_dev(a.reshape(c.n_buf, H * D), bf) for a in (c.q, c.k, c.v))
    o = torch.empty_like(q)
    cu, vl = to_dev(c.cu_slots), to_dev(c.valid_len)
    ml = int(c.valid_len.max())
    flop = 4.0 * D * H * float(sum(int(n) ** 2 for n in c.valid_len))
    ws = torch.empty(max(h3.varlen_attn_workspace_size(c.n_buf, H, D, len(c.valid_len), bf), 16),
                     dtype=torch.uint8, device="cuda")
    ms = timer.time(lambda: h3.h3_varlen_attn(q, k, v, o, H, D, cu, vl, ml, ws=ws), reps, warm=2)
    ws8 = torch.empty(max(h3.varlen_attn_fp8_workspace_size(c.n_buf, H, D, len(c.valid_len)), 16),
                      dtype=torch.uint8, device="cuda")
    ms8 = timer.time(lambda: h3.h3_varlen_attn_fp8(q, k, v, o, H, D, cu, vl, ml, ws=ws8), reps, warm=2)
    return {"ms": ms, "TFLOP/s": flop / ms / 1e9, "frac_peak": flop / ms / 1e9 / BF16_PEAK_TFLOPS,
            "fp8_ms": ms8, "fp8_TFLOP/s": flop / ms8 / 1e9, "algorithmic_flop": flop,
            "workload": "8 heads x 128, segments 4032/1500/17 with random suffix pads in 8192 rows"}


def share_block_measure(h3, torch, W, timer, wl, seed, reps, warm=1):
    """One DiT block on a request share (rank 7 of 8), bf16: ms per block."""
    bf = torch.bfloat16
    w = W.block_weights(wl, seed, "bf16")
    bi = W.block_inputs(wl, seed, "bf16")
    wd = {k: to_dev(getattr(w, k), bf) for k in ("w_qkv", "w_o", "w1", "w3", "w2", "g_q", "g_k")}
    x = to_dev(bi.x, bf)
    mod = to_dev(bi.mod, bf)
    pos, cu, vl = to_dev(bi.pos), to_dev(bi.cu_slots), to_dev(bi.valid_len)
    hc, D = wl.head_count, wl.head_dim
    share = dict(qkv_attn=to_dev(bi.qkv_attn.reshape(wl.n_pad_total, -1), bf),
                 o_attn=torch.zeros((wl.n_pad_total, hc * D), dtype=bf, device="cuda"),
                 o_local=to_dev(bi.o_local.reshape(wl.n_loc, -1), bf),
                 tok_begin=wl.tok_begin, head_begin=wl.head_begin, head_count=hc)
    cfg = h3.block_config(wl.dim, wl.n_heads, D, wl.ffn_dim, wl.sections, wl.theta, wl.eps_qk,
                          wl.eps_mod, 0, bf)
    ws = torch.empty(h3.block_workspace_size(cfg, wl.n_loc, wl.n_pad_total, 1, hc), dtype=torch.uint8,
                     device="cuda")
    max_len = int(bi.valid_len.max())
    ms = timer.time(lambda: h3.h3_dit_block_forward(cfg, wd, x, mod, pos, cu, vl, max_len, ws=ws, **share),
                    reps, warm=2)
    work = algorithmic_work(wl)
    flop = work["attn_flop"] + work["qkv_flop"] + work["out_flop"] + work["w13_flop"] + work["w2_flop"]
    del wd, x, mod, share, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"ms": ms, "TFLOP/s": flop / ms / 1e9, "attn_TFLOP/s_share_of_block": work["attn_flop"] / flop,
            "workload": f"{wl.name}: one DiT block, rank {wl.rank} of {wl.sp_degree} share "
                        f"(n_loc={wl.n_loc}; attention over N={wl.n_valid})"}


# ------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU only; --gpus must be 1 (the "
                                   "sequence-parallel sharding across GPUs is a design, not built)"}))
        sys.exit(2)
    import numpy as np
    import torch
    import audio_video_diffusion_block_amd as h3
    import workloads as W

    wl = W.PRESETS[args.config]
    if wl.n_blocks > 1:
        run_loop_bench(args, h3, torch, W)
        return
    bf = torch.bfloat16
    stream = torch.cuda.current_stream()
    timer = EventTimer(stream)

    if args.only == "attn8k":
        # the 8k varlen attention case alone (for its kernel trace)
        r = varlen8k_measure(h3, torch, W, timer, reps=max(args.steps, 1))
        print(json.dumps({"kernel": "attn8k", **{k: r[k] for k in ("ms", "TFLOP/s", "fp8_ms")}}))
        return

    if args.only == "copy":
        # plain copy of known size: calibration of the HBM byte counters
        nbytes = 1 << 30
        a = torch.empty(nbytes // 2, dtype=bf, device="cuda").normal_()
        b = torch.empty_like(a)
        for _ in range(2):
            b.copy_(a)
        torch.cuda.synchronize()
        ms = timer.time(lambda: b.copy_(a), 3)
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms": ms,
                          "GB/s": 2 * nbytes / ms / 1e6}))
        return

    work = algorithmic_work(wl)
    w, bi = make_inputs(wl, args.seed)
    t0 = time.time()
    wd = {k: to_dev(getattr(w, k), bf) for k in ("w_qkv", "w_o", "w1", "w3", "w2", "g_q", "g_k")}
    x0 = to_dev(bi.x, bf)
    x = x0.clone()
    mod = to_dev(bi.mod, bf)
    pos = to_dev(bi.pos)
    cu = to_dev(bi.cu_slots)
    vl = to_dev(bi.valid_len)
    max_len = int(bi.valid_len.max())
    cfg = h3.block_config(wl.dim, wl.n_heads, wl.head_dim, wl.ffn_dim, wl.sections, wl.theta,
                          wl.eps_qk, wl.eps_mod, 0, bf)
    share = {}
    H, D, C = wl.n_heads, wl.head_dim, wl.dim
    hc = wl.head_count if wl.share_mode else H
    if wl.share_mode:
        share = dict(qkv_attn=to_dev(bi.qkv_attn.reshape(wl.n_pad_total, -1), bf),
                     o_attn=torch.zeros((wl.n_pad_total, hc * D), dtype=bf, device="cuda"),
                     o_local=to_dev(bi.o_local.reshape(wl.n_loc, -1), bf),
                     tok_begin=wl.tok_begin, head_begin=wl.head_begin, head_count=hc)
    n_buf = wl.n_pad_total if wl.share_mode else wl.n_loc
    ws = torch.empty(h3.block_workspace_size(cfg, wl.n_loc, n_buf, 1, hc if wl.share_mode else 0), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"uploaded in {time.time() - t0:.1f}s; workspace {ws.numel() / 2**30:.2f} GiB")

    def block():
        h3.h3_dit_block_forward(cfg, wd, x, mod, pos, cu, vl, max_len, ws=ws, **share)

    # attention alone, as the block launches it (head slice over the whole buffer)
    if wl.share_mode:
        qa = share["qkv_attn"]
        q_v, k_v, v_v = qa[:, :hc * D], qa[:, hc * D:2 * hc * D], qa[:, 2 * hc * D:]
        o_v = share["o_attn"]
    else:
        qkv_t = torch.randn((wl.n_loc, 3 * H * D), dtype=bf, device="cuda")
        q_v, k_v, v_v = qkv_t[:, :H * D], qkv_t[:, H * D:2 * H * D], qkv_t[:, 2 * H * D:]
        o_v = torch.empty((wl.n_loc, H * D), dtype=bf, device="cuda")
    attn_ws = torch.empty(max(h3.varlen_attn_workspace_size(n_buf, hc, D, 1, bf), 16), dtype=torch.uint8,
                          device="cuda")

    def attn():
        h3.h3_varlen_attn(q_v, k_v, v_v, o_v, hc, D, cu, vl, max_len, ws=attn_ws)

    if args.only in ("attn", "attn_fp8"):
        fn = attn
        if args.only == "attn_fp8":
            ws8 = torch.empty(max(h3.varlen_attn_fp8_workspace_size(n_buf, hc, D, 1), 16),
                              dtype=torch.uint8, device="cuda")
            fn = lambda: h3.h3_varlen_attn_fp8(q_v, k_v, v_v, o_v, hc, D, cu, vl, max_len, ws=ws8)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ms = timer.time(fn, max(args.steps, 1))
        print(json.dumps({"kernel": args.only, "attn_ms": ms, "attn_tflops": work["attn_flop"] / ms / 1e9}))
        return

    if args.only == "block":
        # the block's kernels alone (for per-kernel counters)
        for _ in range(args.warmup):
            block()
        torch.cuda.synchronize()
        ms = timer.time(block, max(args.steps, 1))
        print(json.dumps({"kernel": "block", "block_ms": ms}))
        return

    # ---- timed block steps
    log(f"warmup {args.warmup}, steps {args.steps}")
    for _ in range(args.warmup):
        block()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    step_ms = timer.time(block, args.steps)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    log(f"block {step_ms:.2f} ms/step (wall {wall_ms:.2f})")

    # ---- per-step breakdown: each C entry alone, HIP events on the launch stream
    reps = args.op_reps
    reps_short = max(reps, 20)  # sub-millisecond passes: more calls per event pair
    h1 = torch.empty((wl.n_loc, C), dtype=bf, device="cuda")
    qkv = torch.empty((wl.n_loc, 3 * H * D), dtype=bf, device="cuda")
    xs = x0.clone()
    ops = {}
    ops["modnorm"] = timer.time(lambda: h3.h3_modulate_residual(
        xs, shift=mod[:, 0], scale=mod[:, 1], h_out=h1), reps_short, warm=1)
    ops["qkv_gemm"] = timer.time(lambda: h3.h3_linear(h1, wd["w_qkv"], qkv), reps, warm=1)
    # the other GEMMs next, before the long attention launches leave the chip's
    # clock lowered for the short calls that follow them
    o_gemm = share["o_local"] if wl.share_mode else o_v
    ops["out_gemm_residual"] = timer.time(lambda: h3.h3_linear(o_gemm, wd["w_o"], xs, gate=mod[:, 2]),
                                          reps, warm=1)
    sw_ws = torch.empty(h3.swiglu_workspace_size(wl.n_loc, wl.ffn_dim, bf), dtype=torch.uint8, device="cuda")
    ops["swiglu_residual"] = timer.time(lambda: h3.h3_swiglu(
        h1, wd["w1"], wd["w3"], wd["w2"], xs, gate=mod[:, 5], ws=sw_ws), reps, warm=1)
    # FP8 projections on MX operands: weights quantized once, activations on the fly
    wmx = h3.block_weights_mx(wd)
    h1m = h3.h3_mx_quantize(h1)
    ops["act_quant"] = timer.time(lambda: h3.h3_mx_quantize(h1, h1m), reps_short, warm=1)
    ops["modnorm_mx"] = timer.time(lambda: h3.h3_modulate_mx(xs, mod[:, 0], mod[:, 1], out=h1m),
                                   reps_short, warm=1)
    ops["qkv_gemm_fp8"] = timer.time(lambda: h3.h3_linear_fp8(h1m, wmx[0], qkv), reps, warm=1)
    om = h3.h3_mx_quantize(o_gemm)
    ops["out_gemm_residual_fp8"] = timer.time(lambda: h3.h3_linear_fp8(om, wmx[1], xs, gate=mod[:, 2]), reps, warm=1)
    sw8_ws = torch.empty(h3.swiglu_fp8_workspace_size(wl.n_loc, wl.ffn_dim), dtype=torch.uint8, device="cuda")
    ops["swiglu_residual_fp8"] = timer.time(lambda: h3.h3_swiglu_fp8(
        h1m, wmx[2], wmx[3], wmx[4], xs, gate=mod[:, 5], ws=sw8_ws), reps, warm=1)
    del om, sw8_ws
    ops["qk_norm_rope"] = timer.time(lambda: h3.h3_qk_norm_rope(
        qkv[:, :H * D], qkv[:, H * D:2 * H * D], H, D, wd["g_q"], wd["g_k"], pos, wl.sections,
        wl.theta, wl.eps_qk), reps_short, warm=1)
    ops["attention"] = timer.time(attn, reps, warm=1)
    # the MX-scaled e4m3 attention on the same operands, with its own workspace
    ws8 = torch.empty(max(h3.varlen_attn_fp8_workspace_size(n_buf, hc, D, 1), 16),
                      dtype=torch.uint8, device="cuda")
    o8 = torch.empty_like(o_v)
    ops["attention_fp8"] = timer.time(lambda: h3.h3_varlen_attn_fp8(
        q_v, k_v, v_v, o8, hc, D, cu, vl, max_len, ws=ws8), reps, warm=1)
    # Skip-Softmax on the same operands (t = -20: random scores leave no key
    # block that far below the running max, so this is the rule's overhead)
    o_sk = torch.empty_like(o_v)
    ops["attention_skip_random"] = timer.time(lambda: h3.h3_varlen_attn_skip(
        q_v, k_v, v_v, o_sk, hc, D, cu, vl, max_len, -20.0, ws=attn_ws), reps, warm=1)
    ops["attention_fp8_skip_random"] = timer.time(lambda: h3.h3_varlen_attn_fp8_skip(
        q_v, k_v, v_v, o8, hc, D, cu, vl, max_len, -20.0, ws=ws8), reps, warm=1)
    # ... and on operands where attention is concentrated: every query is
    # 4 e0 + noise and 3 of 4 key blocks (after the first) score ~4.5 log2
    # units below the others, so with t = -3 they are skipped
    gsk = torch.Generator(device="cuda").manual_seed(11)
    qs = (torch.randn((n_buf, hc, D), generator=gsk, device="cuda") * 0.05)
    qs[:, :, 0] += 4.0
    ks = torch.randn((n_buf, hc, D), generator=gsk, device="cuda")
    far = torch.rand((n_buf + 63) // 64, generator=gsk, device="cuda") < 0.75
    far[0] = False
    far_rows = far.repeat_interleave(64)[:n_buf]
    c_far = 4.5 / (4.0 * 1.4426950408889634 / D ** 0.5)
    ks[far_rows] = torch.randn((int(far_rows.sum()), hc, D), generator=gsk, device="cuda") * 0.05
    ks[far_rows, :, 0] -= c_far
    qs, ks = qs.reshape(n_buf, hc * D).to(bf), ks.reshape(n_buf, hc * D).to(bf)
    ops["attention_concentrated_exact"] = timer.time(lambda: h3.h3_varlen_attn(
        qs, ks, v_v, o_sk, hc, D, cu, vl, max_len, ws=attn_ws), reps, warm=1)
    ops["attention_concentrated_skip"] = timer.time(lambda: h3.h3_varlen_attn_skip(
        qs, ks, v_v, o_sk, hc, D, cu, vl, max_len, -3.0, ws=attn_ws), reps, warm=1)
    ops["attention_fp8_concentrated"] = timer.time(lambda: h3.h3_varlen_attn_fp8(
        qs, ks, v_v, o8, hc, D, cu, vl, max_len, ws=ws8), reps, warm=1)
    ops["attention_fp8_concentrated_skip"] = timer.time(lambda: h3.h3_varlen_attn_fp8_skip(
        qs, ks, v_v, o8, hc, D, cu, vl, max_len, -3.0, ws=ws8), reps, warm=1)
    skip_frac = float(far.float().mean())
    del qs, ks, o_sk, far, far_rows, ws8, o8
    o_in = share["o_local"] if wl.share_mode else o_v
    if wl.share_mode:
        # the same block with the peer-major exchange buffers (QKV epilogue writes the
        # all-to-all send layout, the output projection reads the receive layout)
        P = wl.sp_degree
        peer = dict(qkv_attn=share["qkv_attn"], o_attn=share["o_attn"],
                    qkv_send=torch.empty((P, wl.n_loc, 3, hc, D), dtype=bf, device="cuda"),
                    o_recv=share["o_local"].reshape(wl.n_loc, P, hc * D).transpose(0, 1).contiguous(),
                    tok_begin=wl.tok_begin, head_begin=wl.head_begin, head_count=hc)
        xp = x0.clone()
        ops["block_peer_major"] = timer.time(lambda: h3.h3_dit_block_forward(
            cfg, wd, xp, mod, pos, cu, vl, max_len, ws=ws, **peer), reps, warm=1)
        del peer, xp
    # the whole block with FP8 steps (same launch sequence otherwise)
    wd8 = {"mx": wmx, "g_q": wd["g_q"], "g_k": wd["g_k"]}
    for key, a8, g8 in (("block_fp8_attention", True, False), ("block_fp8_projections", False, True),
                        ("block_fp8", True, True)):
        cfg8 = h3.block_config(wl.dim, wl.n_heads, wl.head_dim, wl.ffn_dim, wl.sections, wl.theta,
                               wl.eps_qk, wl.eps_mod, 0, bf, attn_fp8=a8, gemm_fp8=g8)
        ws_b8 = torch.empty(h3.block_workspace_size(cfg8, wl.n_loc, n_buf, 1, hc if wl.share_mode else 0), dtype=torch.uint8,
                            device="cuda")
        x8 = x0.clone()
        ops[key] = timer.time(lambda: h3.h3_dit_block_forward(
            cfg8, wd8 if g8 else wd, x8, mod, pos, cu, vl, max_len, ws=ws_b8, **share), reps, warm=1)
        del ws_b8, x8
    del wmx, h1m, wd8
    # post-DiT tail: the 10 s request's decoded frames (1344x768, 243 frames) to uint8 BTHWC
    fr = W.FRAMES_10S
    frames = torch.rand((fr["B"], 3, fr["T"], fr["H"], fr["W"]), device="cuda") * 2.1 - 1.05
    fout = torch.empty((fr["B"], fr["T"], fr["H"], fr["W"], 3), dtype=torch.uint8, device="cuda")
    ops["frames_u8"] = timer.time(lambda: h3.h3_frames_to_u8(frames, fout, 0), reps_short, warm=1)
    frames_bytes = frames.numel() * 5  # 4 bytes read + 1 byte written per value
    del frames, fout
    torch.cuda.synchronize()
    attn_ms = ops["attention"]
    attn_tflops = work["attn_flop"] / attn_ms / 1e9
    total_flop = work["attn_flop"] + work["qkv_flop"] + work["out_flop"] + work["w13_flop"] + work["w2_flop"]
    breakdown = {
        "attention": {"ms": attn_ms, "TFLOP/s": attn_tflops, "frac_peak": attn_tflops / BF16_PEAK_TFLOPS},
        "attention_fp8": {"ms": ops["attention_fp8"],
                          "TFLOP/s": work["attn_flop"] / ops["attention_fp8"] / 1e9,
                          "frac_peak": work["attn_flop"] / ops["attention_fp8"] / 1e9 / FP8_PEAK_TFLOPS,
                          "peak": "fp8 dense MFMA", "speedup_vs_bf16": attn_ms / ops["attention_fp8"],
                          "operands": "MX e4m3 Q/K/V (E8M0 scale per 32), P as e4m3"},
        "attention_skip": {"random_ms": ops["attention_skip_random"],
                           "random_vs_exact": ops["attention_skip_random"] / attn_ms,
                           "concentrated_exact_ms": ops["attention_concentrated_exact"],
                           "concentrated_skip_ms": ops["attention_concentrated_skip"],
                           "concentrated_speedup": ops["attention_concentrated_exact"] / ops["attention_concentrated_skip"],
                           "concentrated_far_block_frac": skip_frac,
                           "fp8_random_ms": ops["attention_fp8_skip_random"],
                           "fp8_random_vs_fp8": ops["attention_fp8_skip_random"] / ops["attention_fp8"],
                           "fp8_concentrated_ms": ops["attention_fp8_concentrated"],
                           "fp8_concentrated_skip_ms": ops["attention_fp8_concentrated_skip"],
                           "fp8_concentrated_speedup": ops["attention_fp8_concentrated"] / ops["attention_fp8_concentrated_skip"],
                           "fp8_skip_vs_bf16_exact": ops["attention_concentrated_exact"] / ops["attention_fp8_concentrated_skip"],
                           "note": "Skip-Softmax on the bf16 and FP8 paths; random operands t=-20 (no block "
                                   "skipped), concentrated operands t=-3 (the far key blocks skipped)"},
        "block_fp8_attention": {"ms": ops["block_fp8_attention"],
                                "TFLOP/s": total_flop / ops["block_fp8_attention"] / 1e9,
                                "note": "the same block with attention on the FP8 path"},
        "block_fp8_projections": {"ms": ops["block_fp8_projections"],
                                  "TFLOP/s": total_flop / ops["block_fp8_projections"] / 1e9,
                                  "note": "the same block with the four projections on MX-e4m3 operands"},
        "block_fp8": {"ms": ops["block_fp8"], "TFLOP/s": total_flop / ops["block_fp8"] / 1e9,
                      "speedup_vs_bf16": step_ms / ops["block_fp8"],
                      "note": "FP8 attention and FP8 projections together"},
        "qkv_gemm_fp8": {"ms": ops["qkv_gemm_fp8"], "TFLOP/s": work["qkv_flop"] / ops["qkv_gemm_fp8"] / 1e9,
                         "frac_peak": work["qkv_flop"] / ops["qkv_gemm_fp8"] / 1e9 / FP8_PEAK_TFLOPS},
        "out_gemm_residual_fp8": {"ms": ops["out_gemm_residual_fp8"],
                                  "TFLOP/s": work["out_flop"] / ops["out_gemm_residual_fp8"] / 1e9},
        "swiglu_residual_fp8": {"ms": ops["swiglu_residual_fp8"],
                                "TFLOP/s": (work["w13_flop"] + work["w2_flop"]) / ops["swiglu_residual_fp8"] / 1e9,
                                "note": "includes quantizing g"},
        "modnorm_mx": {"ms": ops["modnorm_mx"],
                       "GB/s": wl.n_loc * C * (3 * 2 + 1 + 1 / 32) / ops["modnorm_mx"] / 1e6,
                       "frac_hbm": wl.n_loc * C * (3 * 2 + 1 + 1 / 32) / ops["modnorm_mx"] / 1e6 / HBM_PEAK_GBS,
                       "note": "modulated norm written as the MX e4m3 operand of the FP8 projections "
                               "(x, shift, scale read; e4m3 bytes and scales written)"},
        "act_quant": {"ms": ops["act_quant"], "GB/s": wl.n_loc * C * (2 + 1 + 1 / 32) / ops["act_quant"] / 1e6,
                      "note": "h1 bf16 -> MX e4m3 (one per projection input)"},
        "qkv_gemm": {"ms": ops["qkv_gemm"], "TFLOP/s": work["qkv_flop"] / ops["qkv_gemm"] / 1e9},
        "out_gemm_residual": {"ms": ops["out_gemm_residual"],
                              "TFLOP/s": work["out_flop"] / ops["out_gemm_residual"] / 1e9},
        "swiglu_residual": {"ms": ops["swiglu_residual"],
                            "TFLOP/s": (work["w13_flop"] + work["w2_flop"]) / ops["swiglu_residual"] / 1e9},
        "modnorm": {"ms": ops["modnorm"], "GB/s": work["modnorm_bytes"] / ops["modnorm"] / 1e6,
                    "frac_hbm": work["modnorm_bytes"] / ops["modnorm"] / 1e6 / HBM_PEAK_GBS},
        "qk_norm_rope": {"ms": ops["qk_norm_rope"], "GB/s": work["qknorm_bytes"] / ops["qk_norm_rope"] / 1e6,
                         "frac_hbm": work["qknorm_bytes"] / ops["qk_norm_rope"] / 1e6 / HBM_PEAK_GBS},
        "block_peer_major": ({"ms": ops["block_peer_major"],
                              "layout": "qkv_send [P,n,3,hc,D] from the QKV epilogue, o_recv [P,n,hc*D] "
                                        "read in place by the output projection"}
                             if "block_peer_major" in ops else None),
        "frames_u8": {"ms": ops["frames_u8"], "GB/s": frames_bytes / ops["frames_u8"] / 1e6,
                      "frac_hbm": frames_bytes / ops["frames_u8"] / 1e6 / HBM_PEAK_GBS,
                      "workload": "10 s decoded video, 243 x 3 x 768 x 1344 fp32 -> uint8 BTHWC"},
    }
    value = total_flop / step_ms / 1e9  # TFLOP/s of the whole block

    traffic = traffic_record()
    roofline = {"bound": "mfma", "achieved": attn_tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": attn_tflops / BF16_PEAK_TFLOPS, "traffic": traffic,
                "kernel": "attn_fwd_bf16_pipe_kernel<128,8> (+ V transpose pass)",
                "algorithmic_flop_per_launch": work["attn_flop"]}
    copy_gbps = copy_rate(timer)
    hbm_ceiling_rec = {
        "copy_gbps": copy_gbps,
        "modnorm_frac_of_copy": breakdown["modnorm"]["GB/s"] / copy_gbps,
        "qk_norm_rope_frac_of_copy": breakdown["qk_norm_rope"]["GB/s"] / copy_gbps,
        "frames_u8_frac_of_copy": breakdown["frames_u8"]["GB/s"] / copy_gbps,
        "note": "torch's device copy of 1 GiB; bytes = read + written"}

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: one DiT block, rank {wl.rank} of {wl.sp_degree} share "
                               f"(n_loc={wl.n_loc} tokens x C={C}; attention over N={wl.n_valid} "
                               f"valid tokens, heads {wl.head_begin}-{wl.head_begin + hc - 1} of {H} x {D})",
                   "n_valid": wl.n_valid, "n_loc": wl.n_loc, "dim": C, "heads": H, "head_dim": D,
                   "ffn_dim": wl.ffn_dim, "head_slice": hc, "parallelism": "1 GPU (rank-share stand-in)"},
        "block_ms": step_ms, "attn_tflops": attn_tflops,
        "fused_op_gbps": {k: breakdown[k]["GB/s"] for k in ("modnorm", "qk_norm_rope", "frames_u8")},
        "breakdown": breakdown, "roofline": roofline, "hbm_ceiling": hbm_ceiling_rec,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, w, bi, work)
    if not args.no_extra and wl.name == "share10s":
        # the other configurations of the request sweep, each after the 10 s
        # share's buffers are freed
        del w, bi, wd, x, x0, mod, pos, cu, vl, share, ws, attn_ws, h1, qkv, xs, sw_ws
        del q_v, k_v, v_v, o_v, o_in
        if wl.share_mode:
            del qa
        else:
            del qkv_t
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        log("extra configs: 8k varlen attention")
        out["varlen8k_attention"] = varlen8k_measure(h3, torch, W, timer)
        log("extra configs: 5 s share block")
        out["share5s_block"] = share_block_measure(h3, torch, W, timer, W.SHARE_5S, args.seed, 10)
        log("extra configs: 15 s four-forward loop (bf16, then FP8 with MX weights only)")
        out["loop15s"] = loop_measure(h3, torch, W, args.seed, 1, 1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
