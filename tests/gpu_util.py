"""Helpers for the GPU parity tests: device transfer, the oracle on the same
inputs, and the error measures with their tolerances.

Tolerances (per output tensor, normwise):  max_i |gpu_i - ref_i| / max_i |ref_i|
  fp32 storage, fp32 accumulation:                 <= 1e-5
  bf16 storage (inputs/outputs), fp32 accumulation: <= 1e-2
The reference is the float64 oracle on exactly the values the GPU consumed
(bf16 inputs are exact in float64).  Index tables are compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"f32": 1e-5, "bf16": 1e-2}


def tdtype(dt: str):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def host(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def normwise(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(gpu - ref)))
    if scale == 0.0:
        return err
    return err / scale


def p999(gpu, ref) -> float:
    """99.9th percentile of the elementwise error, relative to max |ref|
    (reported beside the normwise error; the bound is on the normwise one)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref))) or 1.0
    return float(np.percentile(np.abs(gpu - ref), 99.9)) / scale


def assert_close(gpu, ref, dt: str, what: str):
    e = normwise(gpu, ref)
    assert np.all(np.isfinite(np.asarray(gpu, dtype=np.float64))), f"{what}: non-finite output"
    print(f"  {what}: normwise {e:.2e}, elementwise p99.9 {p999(gpu, ref):.2e}")
    assert e <= TOL[dt], f"{what}: normwise error {e:.3e} > {TOL[dt]:.0e}"
    return e


def sample_rows(n: int, count: int, seed: int = 0, tile: int = 128) -> np.ndarray:
    """First/last rows, rows around tile boundaries, plus random rows."""
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng(seed)
    fixed = [0, 1, n - 1, n - 2]
    for b in range(tile, n, max(tile, n // 8 // tile * tile)):
        fixed += [b - 1, b]
    extra = rng.choice(n, size=min(n, count), replace=False)
    rows = np.unique(np.clip(np.array(fixed + list(extra)), 0, n - 1))
    return rows.astype(np.int64)
