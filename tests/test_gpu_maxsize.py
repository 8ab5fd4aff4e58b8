"""Parity at the longest sequence the library accepts.

A sequence is addressed with 32-bit byte offsets, so the calls accept T * max(p, dv) * 4 < 2^31
(the host check is pinned in test_abi_cpu.py). At p = 32, dv = 64 that is T = 8,388,607 tokens:
one head of that length runs through the chunked forward (both scans, C = 128, fp32 output, so
the last output row ends 256 bytes below 2^31) and the flash-style quadratic form (bf16 output),
and sampled rows are checked against the float64 definition: the first and last rows, chunk and
segment edges near the end, and rows spread over the sequence.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kernelized_linear_attention_normalize_amd as kata
from kata_inputs import draw_qkv
from oracle import kata_oracle as ko
from tests.gpu_util import TOL, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

P, DV = 32, 64
T_MAX = (2**31 - 1) // (max(P, DV) * 4)  # largest T with T * max(p, dv) * 4 < 2^31


def test_t_max_is_the_accepted_limit():
    assert T_MAX * DV * 4 < 2**31 - 1 <= (T_MAX + 1) * DV * 4
    assert T_MAX == 8388607


@pytest.fixture(scope="module")
def max_case():
    print(f"[case] max length B=1 H=1 T={T_MAX} p={P} dv={DV} bf16 seed 31", flush=True)
    q, k, v = draw_qkv(31, 1, 1, T_MAX, P, DV, "bf16")
    rng = np.random.default_rng(32)
    rows = sorted(set([0, 1, 127, 128, 8191, 8192, 1 << 22, T_MAX - 8193, T_MAX - 8192, T_MAX - 129,
                       T_MAX - 128, T_MAX - 2, T_MAX - 1] + list(rng.integers(0, T_MAX, 12))))
    ref = ko.naive_rows(q[0, 0], k[0, 0], v[0, 0], rows)
    dev = (to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"))
    return rows, ref, dev


@pytest.mark.parametrize("scan", ["associative", "sequential"])
def test_chunked_at_max_length(max_case, scan):
    rows, ref, (qd, kd, vd) = max_case
    print(f"[case] chunked_fwd T={T_MAX} C=128 scan={scan} fp32 out", flush=True)
    got = kata.chunked_fwd(qd, kd, vd, C=128, scan=scan, out_dtype=torch.float32)
    torch.cuda.synchronize()
    err = row_rel_err(to_np(got[0, 0, rows]), ref)
    print(f"  chunked T={T_MAX} {scan}: max row err over {len(rows)} sampled rows {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_quadratic_at_max_length(max_case):
    rows, ref, (qd, kd, vd) = max_case
    # same q, k at p = 32 as the chunked test (the quadratic kernel takes p in {16, 32, 64})
    print(f"[case] quadratic_fwd T={T_MAX} bf16 out", flush=True)
    got = kata.quadratic_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    err = row_rel_err(to_np(got[0, 0, rows]), ref)
    print(f"  quadratic T={T_MAX}: max row err over {len(rows)} sampled rows {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
