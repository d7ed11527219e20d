"""Shared helpers of the GPU tests: device transfer and the error metric.

Error metric (row-wise, the reading of "max relative error" used throughout):
    max over rows i of  max_m |x_im - y_im| / max_m |y_im|
with y the fp64 oracle.  Elementwise relative error is meaningless for outputs
near zero (they are convex combinations of zero-mean values), while the
row-wise form measures error against the scale of each output vector.
"""
import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_dev(a: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    raise ValueError(dtype)


def rowwise_rel(x, y) -> float:
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    num = np.abs(x - y).max(axis=-1)
    den = np.abs(y).max(axis=-1)
    return float((num / den).max())


def whole_rel(x, y) -> float:
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        return float("inf")
    return float(np.abs(x - y).max() / np.abs(y).max())
