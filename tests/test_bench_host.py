"""Host-side checks of bench.py (CPU): the one-GPU guard, and the algorithmic work
that every reported rate divides by, against the sizes the workload definition
gives (10 s request share: 61 latent frames of 48 x 84 patches plus 254 audio
tokens, rank 7 of 8, 5 of 40 heads of 128, hidden 5120, SwiGLU 13,824)."""
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stdout


def test_algorithmic_work_of_the_10s_share():
    wl = W.PRESETS["share10s"]
    n_valid = 61 * 48 * 84 + 254
    assert wl.n_valid == n_valid == 246206
    n_loc = (n_valid + 7) // 8 * 8 // 8
    assert wl.n_loc == n_loc == 30776
    w = bench.algorithmic_work(wl)
    # attention: QK^T and PV, 2 flops per multiply-add, over valid rows of the 5-head slice
    assert w["attn_flop"] == 2 * 2 * 128 * 5 * n_valid ** 2
    assert round(w["attn_flop"] / 1e12, 2) == 155.18
    assert round(w["qkv_flop"] / 1e12, 3) == 4.841
    assert round(w["out_flop"] / 1e12, 3) == 1.614
    assert round(w["w13_flop"] / 1e12, 3) == 8.713
    assert round(w["w2_flop"] / 1e12, 3) == 4.357
    # bytes: each input read once, each output written once, bf16
    assert w["modnorm_bytes"] == 2 * 4 * n_loc * 5120          # x, shift, scale in; h out
    assert w["qknorm_bytes"] == 2 * 4 * n_loc * 40 * 128 + 16 * n_loc
    assert round(w["modnorm_bytes"] / 1e9, 3) == 1.261
