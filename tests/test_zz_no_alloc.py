"""kata_chunked_fwd_noalloc on the GPU: the entry point that keeps its workspace in the
library's fixed device scratch array gives the same output as kata_chunked_fwd with a
caller-allocated workspace, call after call (the second call smaller than the first, so it
reuses scratch the first one filled)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kernelized_linear_attention_normalize_amd as kata
from kata_inputs import draw_qkv
from oracle import kata_oracle as ko
from tests.gpu_util import TOL, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


def _run_pair(seed, B, H, T, p, dv, C, scan, dt):
    print(f"[case] noalloc seed={seed} B={B} H={H} T={T} p={p} dv={dv} C={C} scan={scan} {dt}", flush=True)
    q, k, v = draw_qkv(seed, B, H, T, p, dv, dt)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    assert kata.chunked_workspace_bytes(B, H, T, p, dv, C, kata._scan_code(scan), qd.dtype) > 0  # uses the scratch
    ref = kata.chunked_fwd(qd, kd, vd, C=C, scan=scan)
    out = torch.full_like(ref, float("nan"))
    got = kata.chunked_fwd_noalloc(qd, kd, vd, out, C=C, scan=scan)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got, ref)
    # and within the oracle's tolerance on a few whole heads
    rows = min(T, 4096)
    for h in (0, H - 1):
        r = ko.naive(q[0, h, :rows], k[0, h, :rows], v[0, h, :rows])
        err = row_rel_err(to_np(got[0, h, :rows]), r)
        print(f"  head {h}: rel err {err:.3e}", flush=True)
        assert err <= TOL[dt]


def test_noalloc_matches_chunked_fwd_two_calls():
    _run_pair(41, 1, 16, 32768, 32, 64, 128, "associative", "bf16")   # 16 heads x 16 segments
    _run_pair(42, 2, 3, 5000, 32, 64, 64, "associative", "bf16")      # smaller, ragged tail


def test_noalloc_other_shapes():
    _run_pair(43, 1, 2, 3000, 16, 32, 32, "associative", "bf16")
    _run_pair(44, 1, 1, 1000, 16, 16, 32, "associative", "f32")
