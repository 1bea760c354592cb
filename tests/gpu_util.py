"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances on the max-abs relative error ||a - b||_inf / ||b||_inf against
# the float64 oracle: float32 outputs 1e-4, bf16 outputs 2e-2, gradients
# produced through bf16 intermediates 5e-2.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
TOL_GRAD = 5e-2


def dev(a: np.ndarray, dtype=torch.float32) -> torch.Tensor:
    """Upload a float32 array (values already representable in `dtype`)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype != torch.float32:
        t = t.to(dtype)
    return t.cuda()


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy()


def max_rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    scale = np.max(np.abs(b))
    diff = np.max(np.abs(a - b))
    if scale == 0:
        return float(diff)
    return float(diff / scale)


def assert_close(a, b, tol, what=""):
    e = max_rel(a, b)
    assert e <= tol, f"{what}: max-abs relative error {e:.3e} > {tol:.1e}"
    return e


def poison(t: torch.Tensor) -> torch.Tensor:
    """Fill an output buffer with NaN (or -7 for ints) so unwritten entries show."""
    if t.dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.fill_(-7)
    return t
