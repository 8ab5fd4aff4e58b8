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


# ------------------------------------------------------------------ packed (varlen) layout
def _pack(x, lens):
    """padded [B, H, T, d] -> packed token-major [sum(lens), H, d]"""
    return np.concatenate([np.transpose(x[b, :, :L], (1, 0, 2)) for b, L in enumerate(lens)], axis=0)


@pytest.mark.parametrize("dt,family,p,g,dv,C,scan", [
    ("bf16", "full", 32, 1, 64, 128, "associative"), ("bf16", "full", 32, 1, 64, 64, "sequential"),
    ("bf16", "full", 16, 1, 32, 32, "associative"), ("f32", "full", 16, 1, 32, 64, "associative"),
    ("bf16", "sigma", 32, 2, 32, 64, "associative"), ("f32", "block", 16, 2, 16, 32, "sequential"),
    ("bf16", "sigma", 64, 2, 64, 128, "associative")])
def test_varlen_packed(dt, family, p, g, dv, C, scan):
    """Token-major packed sequences (kata_chunked_fwd_varlen): each sequence against the oracle
    run on it alone, the state after its last token, rows outside every sequence untouched, and
    bitwise agreement with the padded ragged call on the same data (same kernels and plan)."""
    B, H, max_len = 4, 3, 1600
    lens = [1500, 0, 37, 777]
    print(f"[case] varlen {dt} {family}{g} p={p} dv={dv} C={C} scan={scan} lens={lens}", flush=True)
    q, k, v = draw_qkv(49, B, H, max_len, p, dv, dt)
    extra = 5  # rows after the last sequence, outside every sequence
    pk = [np.concatenate([_pack(x, lens), x[0, :, :extra].transpose(1, 0, 2)], axis=0) for x in (q, k, v)]
    total = pk[0].shape[0]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda:0")
    out = torch.full((total, H, dv), 7.0, dtype=torch.float32, device="cuda:0")
    o, S, Z = kata.chunked_fwd_varlen(*(to_dev(x, dt) for x in pk), cu, max_len, C=C, scan=scan, out=out,
                                      return_state=True, family=family, g=g)
    o, S, Z = to_np(o), to_np(S), to_np(Z)
    assert np.all(o[sum(lens):] == 7.0), "rows outside every sequence were written"
    bar = 1e-2 if dt == "bf16" else 1e-5
    starts = np.concatenate([[0], np.cumsum(lens)])
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(S[b] == 0.0) and np.all(Z[b] == 0.0)
            continue
        got = np.transpose(o[starts[b]:starts[b] + L], (1, 0, 2))  # [H, L, dv]
        ref = kf.naive_family(q[b, :, :L], k[b, :, :L], v[b, :, :L], family, g)
        err = row_rel_err(got, ref)
        S_ref, Z_ref = kf.prefill_state_family(k[b, :, :L], v[b, :, :L], family, g)
        es, ez = _normwise(S[b], S_ref), _normwise(Z[b], Z_ref)
        print(f"  seq {b} L={L} rel_err={err:.3e} state S={es:.2e} Z={ez:.2e}", flush=True)
        assert err <= TOL[dt]
        assert es <= bar and ez <= bar
    # the padded ragged call on the same rows gives the same bits
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    op, Sp, Zp = kata.chunked_fwd(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), C=C, scan=scan,
                                  out_dtype=torch.float32, return_state=True, family=family, g=g, lengths=ln)
    op = to_np(op)
    for b, L in enumerate(lens):
        assert np.array_equal(np.transpose(o[starts[b]:starts[b] + L], (1, 0, 2)), op[b, :, :L])
    assert np.array_equal(S, to_np(Sp)) and np.array_equal(Z, to_np(Zp))


@pytest.mark.parametrize("family,g,p,dv,odt,cut", [
    ("full", 1, 32, 64, torch.float32, False), ("full", 1, 64, 64, torch.bfloat16, False),
    ("full", 1, 16, 16, torch.float32, False), ("full", 1, 64, 32, torch.float32, True),
    ("sigma", 2, 64, 64, torch.float32, False), ("block", 2, 64, 32, torch.bfloat16, True)])
def test_quadratic_varlen_packed(family, g, p, dv, odt, cut):
    """Token-major packed sequences on the quadratic form (kata_quadratic_fwd_varlen, bf16):
    each sequence against the oracle on it alone, lengths across several 512-query blocks and
    ragged 64-key blocks (0, 1, 37, 513, ...), rows outside every sequence untouched, and
    bitwise agreement with kata_quadratic_fwd on each sequence alone. cut: max_len below the
    longest length, whose rows past max_len are then not written."""
    B, H = 6, 3
    lens = [1100, 0, 1, 37, 600, 513]
    max_len = 1024 if cut else 1200
    print(f"[case] quadratic varlen {family}{g} p={p} dv={dv} out={odt} lens={lens} max_len={max_len}", flush=True)
    q, k, v = draw_qkv(53, B, H, max(lens), p, dv, "bf16")
    extra = 5
    pk = [np.concatenate([_pack(x, lens), x[0, :, :extra].transpose(1, 0, 2)], axis=0) for x in (q, k, v)]
    total = pk[0].shape[0]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda:0")
    out = torch.full((total, H, dv), 7.0, dtype=odt, device="cuda:0")
    qd, kd, vd = (to_dev(x, "bf16") for x in pk)
    o = to_np(kata.quadratic_fwd_varlen(qd, kd, vd, cu, max_len, out=out, family=family, g=g))
    starts = np.concatenate([[0], np.cumsum(lens)])
    assert np.all(o[starts[-1]:] == 7.0), "rows outside every sequence were written"
    for b, L in enumerate(lens):
        Lc = min(L, max_len)
        if L > Lc:
            assert np.all(o[starts[b] + Lc:starts[b] + L] == 7.0), "rows past max_len were written"
        if Lc == 0:
            continue
        got = np.transpose(o[starts[b]:starts[b] + Lc], (1, 0, 2))
        ref = kf.naive_family(q[b, :, :Lc], k[b, :, :Lc], v[b, :, :Lc], family, g)
        err = row_rel_err(got, ref)
        print(f"  seq {b} L={Lc} rel_err={err:.3e}", flush=True)
        assert err <= TOL["bf16"]
        alone = kata.quadratic_fwd(*(to_dev(np.ascontiguousarray(x[b:b + 1, :, :Lc]), "bf16") for x in (q, k, v)),
                                   out_dtype=odt, family=family, g=g)
        assert np.array_equal(got, to_np(alone)[0]), f"seq {b} differs from the padded call"


@pytest.mark.parametrize("dt,family,g,p,dv,odt,cut", [
    ("f32", "full", 1, 32, 64, torch.float32, False), ("f32", "full", 1, 16, 16, torch.bfloat16, True),
    ("bf16", "sigma", 2, 32, 32, torch.float32, False), ("f32", "block", 2, 64, 48, torch.float32, True),
    ("bf16", "sigma", 4, 64, 16, torch.bfloat16, False)])
def test_quadratic_varlen_valu(dt, family, g, p, dv, odt, cut):
    """Packed sequences on the VALU quadratic kernels (kata_quadratic_fwd_varlen with fp32
    inputs, or a family shape without MFMA kernels): each sequence against the oracle on it
    alone, bit for bit equal to kata_quadratic_fwd on it alone, rows outside every sequence
    untouched; cut: max_len below the longest length (its rows past max_len not written)."""
    B, H = 6, 2
    lens = [300, 0, 1, 37, 170, 65]
    max_len = 256 if cut else 320
    print(f"[case] quadratic varlen valu {dt} {family}{g} p={p} dv={dv} out={odt} max_len={max_len}", flush=True)
    q, k, v = draw_qkv(57, B, H, max(lens), p, dv, dt)
    extra = 5
    pk = [np.concatenate([_pack(x, lens), x[0, :, :extra].transpose(1, 0, 2)], axis=0) for x in (q, k, v)]
    total = pk[0].shape[0]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda:0")
    out = torch.full((total, H, dv), 7.0, dtype=odt, device="cuda:0")
    o = to_np(kata.quadratic_fwd_varlen(*(to_dev(x, dt) for x in pk), cu, max_len, out=out, family=family, g=g))
    starts = np.concatenate([[0], np.cumsum(lens)])
    assert np.all(o[starts[-1]:] == 7.0), "rows outside every sequence were written"
    bar = 1e-4 if odt == torch.float32 else TOL["bf16"]
    for b, L in enumerate(lens):
        Lc = min(L, max_len)
        if L > Lc:
            assert np.all(o[starts[b] + Lc:starts[b] + L] == 7.0), "rows past max_len were written"
        if Lc == 0:
            continue
        got = np.transpose(o[starts[b]:starts[b] + Lc], (1, 0, 2))
        ref = kf.naive_family(q[b, :, :Lc], k[b, :, :Lc], v[b, :, :Lc], family, g)
        err = row_rel_err(got, ref)
        print(f"  seq {b} L={Lc} rel_err={err:.3e}", flush=True)
        assert err <= bar
        alone = kata.quadratic_fwd(*(to_dev(np.ascontiguousarray(x[b:b + 1, :, :Lc]), dt) for x in (q, k, v)),
                                   out_dtype=odt, family=family, g=g)
        assert np.array_equal(got, to_np(alone)[0]), f"seq {b} differs from the padded call"
