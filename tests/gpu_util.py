"""Helpers for the GPU tests: device upload, the parity bar, case logging."""
from __future__ import annotations

import sys

import numpy as np

# The parity bar, per output: |y_gpu - y_ref| <= 1e-5 * sum_j |w_j x_j| + 1e-6.
REL = 1e-5
ABS = 1e-6


def log(msg: str) -> None:
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible")
    return torch


def up(a: np.ndarray):
    torch = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def w_dev(w: np.ndarray, n: int, p: int):
    return up(w.reshape(p, (n // 32) * 34))


def down(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def parity(y_gpu: np.ndarray, y64: np.ndarray, mag: np.ndarray, label: str) -> float:
    """Assert the bar element by element; returns the worst error / bound."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64).reshape(-1)
    y64 = np.asarray(y64, dtype=np.float64).reshape(-1)
    mag = np.asarray(mag, dtype=np.float64).reshape(-1)
    assert y_gpu.shape == y64.shape
    assert np.all(np.isfinite(y_gpu)), "%s: non-finite output" % label
    err = np.abs(y_gpu - y64)
    bound = REL * mag + ABS
    worst = float(np.max(err / bound)) if err.size else 0.0
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, "%s: %d outputs over the bar, first row %d: gpu %r ref %r bound %r" % (
        label, bad.size, bad[0], y_gpu[bad[0]], y64[bad[0]], bound[bad[0]])
    return worst
