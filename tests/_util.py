"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
import numpy as np
import torch

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}

# bf16 outputs: the stated bound (max-abs 2e-2, mean-abs 2e-3) plus a relative
# L2 bound; fp32 outputs: max-abs 1e-4, mean-abs 1e-5.
TOL = {"bf16": dict(max_abs=2e-2, mean_abs=2e-3, rel_l2=1e-2),
       "f32": dict(max_abs=1e-4, mean_abs=1e-5, rel_l2=1e-5)}


def dev(a, dtype: str, device="cuda"):
    """float32 numpy values (already representable in `dtype`) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=device, dtype=TORCH_DT[dtype])


def dev_i32(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


# e4m3 byte -> value (OCP: bias 7, 3 mantissa bits, 0x7F/0xFF NaN), from the format's definition
E4M3_DECODE = np.array([(-1.0 if c & 0x80 else 1.0) *
                        (((c & 7) * 2.0 ** -9) if ((c >> 3) & 15) == 0
                         else (1 + (c & 7) / 8) * 2.0 ** (((c >> 3) & 15) - 7))
                        for c in range(256)])
E4M3_DECODE[0x7F] = E4M3_DECODE[0xFF] = np.nan


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    return dict(max_abs=float(d.max()) if d.size else 0.0, mean_abs=float(d.mean()) if d.size else 0.0,
                rel_l2=float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)))


def assert_close(got, ref, dtype: str, what: str = "", **override):
    tol = dict(TOL[dtype])
    tol.update(override)
    e = errors(got, ref)
    assert np.isfinite(np.asarray(got)).all(), f"{what}: non-finite output"
    bad = {k: (e[k], tol[k]) for k in tol if e[k] > tol[k]}
    print(f"[{what}] {dtype} " + " ".join(f"{k}={v:.3e}" for k, v in e.items()), flush=True)
    assert not bad, f"{what}: {bad}"
    return e


def share_buffers(wl, bi, dtype, peer=False):
    """The rank-share exchange buffers with the other ranks' rows/heads in place:
    the qkv_attn/o_local stand-in, or the peer-major qkv_send/o_recv layout."""
    P, hc, D, n = wl.sp_degree, wl.head_count, wl.head_dim, wl.n_loc
    extra = dict(qkv_attn=dev(bi.qkv_attn.reshape(wl.n_pad_total, -1), dtype),
                 o_attn=torch.zeros((wl.n_pad_total, hc * D), dtype=TORCH_DT[dtype], device="cuda"),
                 tok_begin=wl.tok_begin, head_begin=wl.head_begin, head_count=hc)
    if peer:
        # o_recv[p, t] = heads [p*hc, (p+1)*hc) of local row t (block `rank` is overwritten)
        o_recv = np.ascontiguousarray(bi.o_local.reshape(n, P, hc, D).transpose(1, 0, 2, 3))
        extra.update(qkv_send=torch.full((P, n, 3, hc, D), float("nan"), dtype=TORCH_DT[dtype],
                                         device="cuda"),
                     o_recv=dev(o_recv, dtype))
    else:
        extra.update(o_local=dev(bi.o_local.reshape(n, -1), dtype))
    return extra
