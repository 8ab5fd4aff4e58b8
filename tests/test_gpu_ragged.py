"""Sequences of different lengths in one call (kata_chunked_fwd_ragged), against the float64
oracles run on each sequence alone: outputs of the used rows, untouched rows past each
length, and the state after each sequence's last token (zero for an empty sequence)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kernelized_linear_attention_normalize_amd as kata
from kata_inputs import draw_qkv
from oracle import kata_families as kf
from tests.gpu_util import TOL, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


def _normwise(got, ref):
    axes = tuple(range(1, ref.ndim))
    den = np.sqrt((ref ** 2).sum(axes))
    return float(np.max(np.sqrt(((got - ref) ** 2).sum(axes)) / den))


@pytest.mark.parametrize("dt,family,p,g,dv,C,scan", [
    ("bf16", "full", 32, 1, 64, 128, "associative"), ("bf16", "full", 32, 1, 64, 64, "sequential"),
    ("bf16", "full", 16, 1, 32, 32, "associative"), ("f32", "full", 16, 1, 32, 64, "associative"),
    ("bf16", "sigma", 64, 2, 64, 128, "associative"), ("bf16", "sigma", 32, 2, 32, 64, "associative"),
    ("bf16", "block", 32, 2, 64, 128, "sequential")])
def test_ragged_lengths(dt, family, p, g, dv, C, scan):
    B, H, T = 4, 2, 2100
    lens = [2100, 1001, 0, 37]
    print(f"[case] ragged {dt} {family}{g} p={p} dv={dv} C={C} scan={scan} lens={lens}", flush=True)
    q, k, v = draw_qkv(48, B, H, T, p, dv, dt)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    out = torch.full((B, H, T, dv), 7.0, dtype=torch.float32, device="cuda:0")
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    o, S, Z = kata.chunked_fwd(qd, kd, vd, C=C, scan=scan, out=out, return_state=True, family=family, g=g,
                               lengths=ln)
    o, S, Z = to_np(o), to_np(S), to_np(Z)
    bar = 1e-2 if dt == "bf16" else 1e-5
    for b, L in enumerate(lens):
        assert np.all(o[b, :, L:] == 7.0), f"rows past the length of sequence {b} were written"
        if L == 0:
            assert np.all(S[b] == 0.0) and np.all(Z[b] == 0.0)
            continue
        ref = kf.naive_family(q[b, :, :L], k[b, :, :L], v[b, :, :L], family, g)
        err = row_rel_err(o[b, :, :L], ref)
        S_ref, Z_ref = kf.prefill_state_family(k[b, :, :L], v[b, :, :L], family, g)
        es, ez = _normwise(S[b], S_ref), _normwise(Z[b], Z_ref)
        print(f"  seq {b} L={L} rel_err={err:.3e} state S={es:.2e} Z={ez:.2e}", flush=True)
        assert err <= TOL[dt]
        assert es <= bar and ez <= bar
