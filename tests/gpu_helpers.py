"""Shared pieces of the GPU parity tests: device fixture, transfers and the
parity assertion (the oracle's bar: |y - y_ref| <= 1e-4 sum|s q x| + 1e-6)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import q8_block_quantized_amd as q8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="session")
def cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    q8.q8_init()  # a load or architecture failure raises: never a silent skip
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def gpu_matvec(w: np.ndarray, x: np.ndarray, device) -> np.ndarray:
    import torch
    n = x.size
    p = w.shape[0]
    wd = to_dev(w.reshape(-1), device)
    xd = to_dev(x.astype(np.float32).reshape(-1), device)
    yd = torch.full((p,), float("nan"), dtype=torch.float32, device=device)
    q8.q8_matvec(wd, xd, yd)
    torch.cuda.synchronize()
    assert n == xd.numel()
    return yd.cpu().numpy()


def gpu_batched(w: np.ndarray, x: np.ndarray, device) -> np.ndarray:
    import torch
    m = x.shape[0]
    p = w.shape[0]
    wd = to_dev(w.reshape(-1), device)
    xd = to_dev(x.astype(np.float32), device)
    yd = torch.full((m, p), float("nan"), dtype=torch.float32, device=device)
    q8.q8_matvec_batched(wd, xd, yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def oracle_rows(w: np.ndarray, x: np.ndarray, threads: int = 16):
    """The oracle's y and tol ([m, p]) for every row of x [m, n], rows of W
    split over `threads` host threads (bit-identical to one thread)."""
    x = np.atleast_2d(x)
    p = w.shape[0]
    ref = np.empty((x.shape[0], p))
    tol = np.empty((x.shape[0], p))
    for r in range(x.shape[0]):
        ref[r], tol[r] = oracle.get().matvec_mt(w, x[r], threads)[:2]
    return ref, tol


def assert_parity(y_gpu, y_ref, tol, label: str) -> float:
    err = oracle.matvec_errors(y_gpu, y_ref, tol)
    worst = int(np.argmax(err)) if err.size else 0
    mx = float(err.max()) if err.size else 0.0
    assert mx <= 1.0, (f"{label}: output {worst} gpu={y_gpu.ravel()[worst]!r} "
                       f"ref={np.ravel(y_ref)[worst]!r} err/tol={mx:.3g}")
    return mx
