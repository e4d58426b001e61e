"""Helpers for the GPU parity tests: move seeded inputs to the device and
compare the HIP path's output with the float64 oracle."""
from __future__ import annotations

import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-4}   # max-abs error bars of the method's contract


def to_dev(x: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def from_dev(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def i32_dev(a):
    import torch
    return None if a is None else torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()


def max_err(got: np.ndarray, want: np.ndarray) -> float:
    assert got.shape == want.shape, (got.shape, want.shape)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - want)))


def nan_filled(like, shape=None, dtype=None):
    """A device tensor shaped and typed like `like` (or as given), filled with NaN: a
    sentinel that shows any output element a kernel leaves unwritten."""
    import torch
    if shape is None:
        return torch.full_like(like, float("nan"))
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def assert_all_written(t, what="output"):
    """Every element of t is finite: no NaN sentinel survived (checked on the device; one
    boolean comes back)."""
    import torch
    assert bool(torch.isfinite(t).all().item()), f"{what}: some elements were never written"
