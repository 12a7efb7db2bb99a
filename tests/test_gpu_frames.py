"""Output-frame conversion on the GPU against the oracle, bit-exact (GPU)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


def _run(lib, x, layout):
    B, _, T, H, Wd = x.shape
    xt = torch.from_numpy(x).cuda()
    shape = (B, T, H, Wd, 3) if layout == 0 else (B, T, 3, H, Wd)
    out = torch.full(shape, 77, dtype=torch.uint8, device="cuda")
    lib.h3_frames_to_u8(xt, out, layout)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("shape", [(2, 3, 5, 48), (2, 3, 5, 40), (1, 1, 1, 16), (1, 2, 3, 7)],
                         ids=["vec", "ragged_w", "one_chunk", "tiny_ragged"])
def test_frames_parity_small(lib, layout, shape):
    B, T, H, Wd = shape
    x = W.frames(11, B, T, H, Wd)
    # every boundary case at least once
    flat = x.reshape(-1)
    flat[:8] = np.array([-1.0, 1.0, 0.0, np.nan, np.inf, -np.inf, 1.5, -1.5], np.float32)[:flat.size]
    np.testing.assert_array_equal(_run(lib, x, layout), O.frames_to_u8(x, layout))


def test_frames_empty_and_errors(lib):
    x = torch.zeros((1, 3, 0, 4, 16), dtype=torch.float32, device="cuda")
    out = torch.zeros((1, 0, 4, 16, 3), dtype=torch.uint8, device="cuda")
    lib.h3_frames_to_u8(x, out, 0)  # nothing to do
    x = torch.zeros((1, 3, 2, 4, 16), dtype=torch.float32, device="cuda")
    out = torch.zeros((1, 2, 4, 16, 3), dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.H3Error):
        lib._check(lib._c_frames(x.data_ptr(), 1, 2, 4, 16, out.data_ptr(), 2, None))
    with pytest.raises(lib.H3Error):  # misaligned output
        lib._check(lib._c_frames(x.data_ptr(), 1, 2, 4, 16, out.data_ptr() + 1, 0, None))


@pytest.mark.parametrize("layout", [0, 1])
def test_frames_10s_sampled(lib, layout):
    """1344x768, 243 frames (the 10 s request): three whole frames compared."""
    d = W.FRAMES_10S
    print(f"frames 10s layout {layout}: {d}", flush=True)
    x = W.frames(0, d["B"], d["T"], d["H"], d["W"])
    got = _run(lib, x, layout)
    for t in (0, d["T"] // 2, d["T"] - 1):
        xs = np.ascontiguousarray(x[:, :, t:t + 1])
        ref = O.frames_to_u8(xs, layout)
        np.testing.assert_array_equal(got[:, t:t + 1], ref)
