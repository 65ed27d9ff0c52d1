"""Shared plumbing for GPU parity tests: device upload, stored-format views and
the row-relative error metric.  No arithmetic of the method lives here."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda"


def up(x, dtype=None):
    """numpy -> device tensor (contiguous)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def up_bf16(x):
    """fp32 numpy -> bf16 device tensor; returns (tensor, stored values as fp64 numpy)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.to(DEV), t.double().numpy()


def down(t) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.double().cpu().numpy()
    return t.cpu().numpy()


def row_rel_err(x, y) -> float:
    """max over output rows (last axis is the row) of ||x_r - y_r||_inf / ||y_r||_inf."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, np.shape(x)[-1])
    y = np.asarray(y, dtype=np.float64).reshape(-1, np.shape(y)[-1])
    num = np.max(np.abs(x - y), axis=1)
    den = np.maximum(np.max(np.abs(y), axis=1), 1e-30)
    return float(np.max(num / den)) if num.size else 0.0


def workspace(nbytes: int):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=DEV)


def stream():
    return torch.cuda.current_stream().cuda_stream


def sorted_unique_choice(rng: np.random.Generator, n_visible: int, k: int) -> np.ndarray:
    """k random distinct indices of [0, n_visible) in ascending order, -1 padded to k."""
    take = min(k, n_visible)
    sel = np.sort(rng.choice(n_visible, size=take, replace=False)) if take else np.zeros(0, np.int64)
    out = np.full(k, -1, dtype=np.int64)
    out[:take] = sel
    return out
