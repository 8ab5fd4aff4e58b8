"""Seeded randomized sweep of the forward forms against the float64 oracle (GPU).

Each case draws its configuration from a fixed seed: batch, heads, a length that is rarely a
multiple of the chunk (ragged tails, lengths below one chunk, lengths that leave the last
segment short), p and dv from the supported sets, the chunk, the scan, the input and output
dtypes and, for the packed layout, the per-sequence lengths (empty ones included). The bar
is the forward's: row-relative error <= 1e-4 for fp32 inputs, <= 2e-2 for bf16 inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kernelized_linear_attention_normalize_amd as kata
from kata_inputs import draw_qkv
from oracle import kata_oracle as ko
from tests.gpu_util import ROW_BAR_MFMA, TOL, grad_row_err, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

N_CASES = 12


def _config(i: int):
    rng = np.random.default_rng(1000 + i)
    dt = ("bf16", "f32")[int(rng.integers(0, 2))]
    p = int(rng.choice([16, 32]))
    dv = int(rng.choice([16, 32, 64]))
    C = int(rng.choice([32, 64, 128]))
    if dt == "f32" and p == 32 and dv == 64:
        C = 32  # the fp32 kernel's LDS holds the 528 x 64 state with chunks of 32
    T = int(rng.integers(1, 2600))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    scan = ("sequential", "associative")[int(rng.integers(0, 2))]
    o_dt = (torch.float32, torch.bfloat16)[int(rng.integers(0, 2))]
    return dict(dt=dt, p=p, dv=dv, C=C, T=T, B=B, H=H, scan=scan, o_dt=o_dt, seed=2000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_chunked_and_quadratic(i):
    c = _config(i)
    print(f"[case] sweep {i}: {c}", flush=True)
    q, k, v = draw_qkv(c["seed"], c["B"], c["H"], c["T"], c["p"], c["dv"], c["dt"])
    ref = ko.naive(q, k, v)
    qd, kd, vd = (to_dev(x, c["dt"]) for x in (q, k, v))
    o = to_np(kata.chunked_fwd(qd, kd, vd, C=c["C"], scan=c["scan"], out_dtype=c["o_dt"]))
    # bf16 output rounds each element once more (relative 2^-9)
    bar = TOL[c["dt"]] + (4e-3 if c["o_dt"] == torch.bfloat16 else 0.0)
    e = row_rel_err(o, ref)
    print(f"  chunked rel_err={e:.2e}", flush=True)
    assert e <= bar
    oq = to_np(kata.quadratic_fwd(qd, kd, vd, out_dtype=c["o_dt"]))
    eq = row_rel_err(oq, ref)
    print(f"  quadratic rel_err={eq:.2e}", flush=True)
    assert eq <= bar


@pytest.mark.parametrize("i", range(6))
def test_sweep_packed(i):
    c = _config(100 + i)
    rng = np.random.default_rng(3000 + i)
    B = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(0, 1500, size=B)]
    if i % 3 == 0:
        lens[0] = 0
    max_len = max(max(lens), 1)
    print(f"[case] packed sweep {i}: {c} lens={lens}", flush=True)
    q, k, v = draw_qkv(c["seed"], B, c["H"], max_len, c["p"], c["dv"], c["dt"])
    pack = lambda x: np.concatenate([np.transpose(x[b, :, :L], (1, 0, 2)) for b, L in enumerate(lens)], axis=0)
    pq, pk_, pv = pack(q), pack(k), pack(v)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda:0")
    if pq.shape[0] == 0:
        return  # nothing to compare (the call itself is covered by the ABI tests)
    o = to_np(kata.chunked_fwd_varlen(to_dev(pq, c["dt"]), to_dev(pk_, c["dt"]), to_dev(pv, c["dt"]), cu, max_len,
                                      C=c["C"], scan=c["scan"], out_dtype=torch.float32))
    start = 0
    for b, L in enumerate(lens):
        if L:
            got = np.transpose(o[start:start + L], (1, 0, 2))
            e = row_rel_err(got, ko.naive(q[b, :, :L], k[b, :, :L], v[b, :, :L]))
            print(f"  seq {b} L={L} rel_err={e:.2e}", flush=True)
            assert e <= TOL[c["dt"]]
        start += L


@pytest.mark.parametrize("i", range(8))
def test_sweep_chunked_backward(i):
    """The O(T) backward on bf16 MFMA (kata_chunked_bwd, and kata_chunked_bwd_varlen on odd
    cases) at seeded shapes: p, dv from its set, lengths rarely a multiple of the 32-token
    chunk, both scans. Bar: the bf16 MFMA backward's, normwise 1e-2 per gradient tensor
    against the float64 oracle."""
    from oracle import kata_backward as kb
    rng = np.random.default_rng(4000 + i)
    p, dv = int(rng.choice([16, 32])), int(rng.choice([32, 64]))
    T = int(rng.integers(2, 1800))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    scan = ("sequential", "associative")[int(rng.integers(0, 2))]
    print(f"[case] backward sweep {i}: p={p} dv={dv} T={T} B={B} H={H} {scan}", flush=True)
    q, k, v = draw_qkv(5000 + i, B, H, T, p, dv, "bf16")
    go = draw_qkv(6000 + i, B, H, T, dv, dv, "bf16")[0]
    ref = kb.backward(q, k, v, go)
    if i % 2 == 0:
        got = [to_np(x) for x in kata.chunked_bwd(*(to_dev(x, "bf16") for x in (q, k, v, go)), C=32, scan=scan)]
    else:  # the same batch packed token-major, every sequence of length T
        pack = lambda x: np.concatenate([np.transpose(x[b], (1, 0, 2)) for b in range(B)], axis=0)
        cu = torch.tensor([b * T for b in range(B + 1)], dtype=torch.int32, device="cuda:0")
        out = kata.chunked_bwd_varlen(*(to_dev(pack(x), "bf16") for x in (q, k, v, go)), cu, T, scan=scan)
        got = [np.stack([np.transpose(to_np(x)[b * T:(b + 1) * T], (1, 0, 2)) for b in range(B)]) for x in out]
    floor = 1e-2 * float(np.linalg.norm(go))
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        e = float(np.linalg.norm(a - r) / max(np.linalg.norm(r), floor))
        er = grad_row_err(a, r)
        print(f"  {name} rel={e:.2e} row-wise={er:.2e}", flush=True)
        assert e <= 1e-2, name
        assert er <= ROW_BAR_MFMA, f"{name} row-wise"
