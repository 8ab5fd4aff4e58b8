"""Helpers shared by the GPU tests (host-side data movement and the error metric only)."""
from __future__ import annotations

import numpy as np
import torch

from oracle.kata_oracle import row_rel_err  # noqa: F401  (re-exported for the tests)

TOL = {"f32": 1e-4, "bf16": 2e-2}

# row-wise gradient bars (grad_row_err): a row's gradient is a sum over many products; the
# fp32 routes round each product at 2^-24 and the bf16 MFMA routes round both factors to bf16
# (2^-9 each), so one row can show several times the tensor's normwise error where it cancels
ROW_BAR_F32 = 1e-3
ROW_BAR_MFMA = 3e-2


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy (bf16-exact when dtype == 'bf16') -> contiguous device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to("cuda:0").contiguous()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def grad_row_err(got: np.ndarray, ref: np.ndarray, rel_floor: float = 1e-2) -> float:
    """Row-wise gradient error: max over rows t (vectors along the last axis) of
    ||got_t - ref_t||_inf / max(||ref_t||_inf, f), f = rel_floor * max_t ||ref_t||_inf.
    A row whose exact gradient is below 1% of the largest row is judged against that 1%,
    so rows with (near) zero gradient do not divide rounding noise by zero."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    if ref.size == 0:
        return 0.0
    rn = np.abs(ref).max(axis=1)
    f = rel_floor * float(rn.max())
    if f == 0.0:
        return float(np.abs(got - ref).max())
    return float((np.abs(got - ref).max(axis=1) / np.maximum(rn, f)).max())
