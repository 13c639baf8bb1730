"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
import sys

import numpy as np


def say(*a):
    """Name the case before a GPU step, flushed, so a failing run says where it was."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def ulp16(y):
    a = np.abs(np.asarray(y, dtype=np.float16))
    return np.spacing(a).astype(np.float64)


def assert_y_close(Y_gpu, Y_orc, what=""):
    """|Y_gpu - Y_orc| <= 2e-3 * max|Y_orc| + ulp16(Y_orc) per element."""
    Y_gpu = np.asarray(Y_gpu)
    Y_orc = np.asarray(Y_orc)
    assert Y_gpu.shape == Y_orc.shape, (Y_gpu.shape, Y_orc.shape)
    assert np.all(np.isfinite(Y_gpu.astype(np.float64))), what + ": non-finite output"
    yo = Y_orc.astype(np.float64)
    err = np.abs(Y_gpu.astype(np.float64) - yo)
    tol = 2e-3 * (np.abs(yo).max() if yo.size else 0.0) + ulp16(Y_orc)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; first {tuple(i)}: "
                             f"gpu {Y_gpu[tuple(i)]} oracle {Y_orc[tuple(i)]} tol {tol[tuple(i)]}")
    return float(err.max()) if err.size else 0.0
