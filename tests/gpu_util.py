"""Helpers shared by the GPU tests (host-side data movement and the error metric only)."""
from __future__ import annotations

import numpy as np
import torch

from oracle.kata_oracle import row_rel_err  # noqa: F401  (re-exported for the tests)

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy (bf16-exact when dtype == 'bf16') -> contiguous device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to("cuda:0").contiguous()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
