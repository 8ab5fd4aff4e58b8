"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

Holds no arithmetic of the method: it only draws N(0,1) numbers from a seed and rounds
them to bfloat16 where a workload is bfloat16. Both the float64 oracle and the HIP path
consume exactly these values.

Recipe: ``np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)``, drawn
in the order q, k, v with C-order shapes q,k: [B,H,T,p], v: [B,H,T,dv]; bfloat16 inputs
are the float32 draws rounded to nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["round_bf16", "Workload", "WORKLOADS", "draw_qkv", "draw_decode_history",
           "draw_decode_steps", "VARLEN", "draw_varlen"]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32
    arrays whose values are exactly representable in bfloat16. NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                      # no overflow for finite values and infinities
    r &= np.uint32(0xFFFF0000)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC00000
    return r.view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    p: int
    dv: int
    dtype: str            # "f32" or "bf16"
    seed: int
    chunks: tuple = ()    # chunk sizes used by the chunked form


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 256, 16, 16, "f32", 0, (32,)),
    "mid": Workload("mid", 8, 16, 2048, 32, 64, "bf16", 1, (64,)),
    "long": Workload("long", 1, 16, 131072, 32, 64, "bf16", 2, (64, 128)),
    "quadratic": Workload("quadratic", 2, 16, 8192, 64, 64, "bf16", 3, ()),
}

# Recurrent decode workload: 128 sequences x 16 heads, p=32, dv=64, a 4096-token
# float32 history (seed 4) that fills the state, then 256 single-token bf16 steps (seed 5).
DECODE = dict(N=128, H=16, p=32, dv=64, hist=4096, steps=256, hist_seed=4, step_seed=5)
# packed variable-length batch: B sequences with lengths uniform in [lo, hi] (about the long
# workload's 131072 tokens in all), token-major q, k [total, H, p], v [total, H, dv]
VARLEN = dict(B=16, H=16, p=32, dv=64, lo=2048, hi=14336, seed=6)


def draw_qkv(seed: int, B: int, H: int, T: int, p: int, dv: int, dtype: str = "bf16"):
    """q, k: [B,H,T,p]; v: [B,H,T,dv] float32 arrays (bf16-exact when dtype == 'bf16')."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, p), dtype=np.float32)
    k = rng.standard_normal((B, H, T, p), dtype=np.float32)
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    return q, k, v


def draw_decode_history(seed: int, N: int, H: int, T: int, p: int, dv: int):
    """History keys and values, float32: k [N,H,T,p], v [N,H,T,dv]."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((N, H, T, p), dtype=np.float32)
    v = rng.standard_normal((N, H, T, dv), dtype=np.float32)
    return k, v


def draw_decode_steps(seed: int, steps: int, N: int, H: int, p: int, dv: int,
                      dtype: str = "bf16"):
    """Per-step tokens: q, k [steps,N,H,p], v [steps,N,H,dv]."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((steps, N, H, p), dtype=np.float32)
    k = rng.standard_normal((steps, N, H, p), dtype=np.float32)
    v = rng.standard_normal((steps, N, H, dv), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


def draw_varlen(spec=None):
    """(lens [B] int, q, k [total, H, p], v [total, H, dv]) float32, bf16-exact."""
    spec = spec or VARLEN
    rng = np.random.default_rng(spec["seed"])
    lens = rng.integers(spec["lo"], spec["hi"] + 1, size=spec["B"])
    total = int(lens.sum())
    q = round_bf16(rng.standard_normal((total, spec["H"], spec["p"]), dtype=np.float32))
    k = round_bf16(rng.standard_normal((total, spec["H"], spec["p"]), dtype=np.float32))
    v = round_bf16(rng.standard_normal((total, spec["H"], spec["dv"]), dtype=np.float32))
    return [int(x) for x in lens], q, k, v
