"""Gradients of the causal forward on the GPU (kata_quadratic_bwd, through the C ABI and the
autograd wrapper) against the float64 backward oracle (oracle/kata_backward.py).

Bar: normwise ||g_gpu - g_ref|| / ||g_ref|| <= 2e-4 per gradient tensor (fp32 arithmetic on
fp32 or exact bf16 inputs; the oracle gets the same input values), <= 1e-2 on the bf16 MFMA
routes. Next to it a row-wise bar (grad_row_err: max over rows of the row's inf-norm error
relative to the row, floored at 1% of the largest row): ROW_BAR_F32 on the fp32 routes,
ROW_BAR_MFMA on the bf16 MFMA routes."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kernelized_linear_attention_normalize_amd as kata
from kata_inputs import draw_qkv
from oracle import kata_backward as kb
from tests.gpu_util import ROW_BAR_F32, ROW_BAR_MFMA, grad_row_err, to_dev, to_np

pytestmark = pytest.mark.gpu


def _rows(name, got, ref, bar):
    e = grad_row_err(got, ref)
    print(f"  {name} row-wise={e:.2e} (bar {bar:.0e})", flush=True)
    assert e <= bar, f"{name} row-wise"


def _rel(got, ref, floor):
    """Normwise error relative to the reference, or to `floor` where the exact gradient is
    (near) zero (e.g. dq at T = 1: o_1 = v_1 for every q)."""
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), floor))


@pytest.mark.parametrize("dt,family,g,p,dv,T", [
    ("f32", "full", 1, 16, 16, 33), ("f32", "full", 1, 32, 64, 257), ("bf16", "full", 1, 64, 48, 200),
    ("f32", "sigma", 2, 32, 32, 100), ("bf16", "block", 2, 64, 64, 130),
    ("f32", "sigma", 4, 64, 16, 70)])
def test_quadratic_bwd_matches_oracle(dt, family, g, p, dv, T):
    print(f"[case] bwd {dt} {family}{g} p={p} dv={dv} T={T}", flush=True)
    q, k, v = draw_qkv(49, 2, 2, T, p, dv, dt)
    go = draw_qkv(50, 2, 2, T, dv, dv, dt)[0]
    q[0, 1, 0] = 0.0
    k[1, 0, T // 2] = 0.0
    ref = kb.backward(q, k, v, go, family, g)
    got = kata.quadratic_bwd(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(go, dt), family=family, g=g)
    floor = 1e-2 * float(np.linalg.norm(go))
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        e = _rel(to_np(a), r, floor)
        print(f"  {name} rel={e:.2e}", flush=True)
        assert e <= 2e-4, name
        _rows(name, to_np(a), r, ROW_BAR_F32)
    assert np.all(to_np(got[0])[0, 1, 0] == 0.0)


def test_single_token():
    """T = 1: o_1 = v_1 whatever q and k, so dv = grad_o and the exact dq, dk vanish (their
    fp32 values are rounding noise amplified by 1 / (q_hat . k_hat), so only finiteness is
    checked for them)."""
    q, k, v = draw_qkv(53, 2, 3, 1, 32, 64, "bf16")
    go = draw_qkv(54, 2, 3, 1, 64, 64, "bf16")[0]
    dq, dk, dvv = kata.quadratic_bwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(go, "bf16"))
    np.testing.assert_allclose(to_np(dvv), go, rtol=1e-6, atol=1e-6)
    assert np.all(np.isfinite(to_np(dq))) and np.all(np.isfinite(to_np(dk)))


def test_autograd_wrapper():
    """kata_attention: chunked forward, gradients from kata_quadratic_bwd through autograd."""
    q, k, v = draw_qkv(51, 1, 2, 300, 32, 64, "f32")
    go = draw_qkv(52, 1, 2, 300, 64, 64, "f32")[0]
    qd, kd, vd = (to_dev(x, "f32").requires_grad_(True) for x in (q, k, v))
    o = kata.kata_attention(qd, kd, vd, C=64)
    (o * to_dev(go, "f32")).sum().backward()
    ref = kb.backward(q, k, v, go)
    for name, t, r in zip(("dq", "dk", "dv"), (qd.grad, kd.grad, vd.grad), ref):
        assert _rel(to_np(t), r, 1e-2 * float(np.linalg.norm(go))) <= 2e-4, name


def test_autograd_wrapper_long_bf16():
    """kata_attention on a long bf16 sequence: the gradients come from the O(T) state form
    (T >= STATE_BWD_MIN_T), at the bf16 MFMA backward's bar against the oracle."""
    T = kata.STATE_BWD_MIN_T + 29
    q, k, v = draw_qkv(53, 1, 2, T, 32, 64, "bf16")
    go = draw_qkv(54, 1, 2, T, 64, 64, "bf16")[0]
    qd, kd, vd = (to_dev(x, "bf16").requires_grad_(True) for x in (q, k, v))
    o = kata.kata_attention(qd, kd, vd, C=64)
    (o.float() * to_dev(go, "f32")).sum().backward()
    ref = kb.backward(q, k, v, go)
    for name, t, r in zip(("dq", "dk", "dv"), (qd.grad, kd.grad, vd.grad), ref):
        e = _rel(to_np(t.float()), r, 1e-2 * float(np.linalg.norm(go)))
        print(f"  {name} rel={e:.2e}", flush=True)
        assert e <= 1.2e-2, name  # the bf16 MFMA bar plus the gradients' rounding to bf16


# ------------------------------------------------------------------ MFMA path
@pytest.mark.parametrize("p,dv,T", [(64, 64, 700), (32, 64, 1030), (64, 32, 257), (32, 32, 64), (64, 64, 600)])
def test_quadratic_bwd_mfma(p, dv, T):
    """bf16 inputs of the full map with p, dv in {32, 64} run the bf16 MFMA backward. Its
    per-pair operands (the weight over D_t and dW_ts S_ts) are rounded to bf16 (relative
    2^-9) before the fp32 accumulation, as the forward rounds its weights; bar: normwise
    1e-2 per gradient tensor. Zero query and key rows get zero gradients."""
    print(f"[case] bwd mfma p={p} dv={dv} T={T}", flush=True)
    q, k, v = draw_qkv(61, 2, 3, T, p, dv, "bf16")
    go = draw_qkv(62, 2, 3, T, dv, dv, "bf16")[0]
    q[1, 2, 5] = 0.0
    k[0, 1, T // 3] = 0.0
    ref = kb.backward(q, k, v, go)
    got = kata.quadratic_bwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(go, "bf16"))
    floor = 1e-2 * float(np.linalg.norm(go))
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        e = _rel(to_np(a), r, floor)
        print(f"  {name} rel={e:.2e}", flush=True)
        assert e <= 1e-2, name
        _rows(name, to_np(a), r, ROW_BAR_MFMA)
    assert np.all(to_np(got[0])[1, 2, 5] == 0.0) and np.all(to_np(got[1])[0, 1, T // 3] == 0.0)


def test_quadratic_bwd_mfma_matches_valu_path():
    """The MFMA path (bf16 inputs) and the fp32 VALU path (the same values as fp32 inputs)
    agree to the MFMA path's bar."""
    q, k, v = draw_qkv(63, 1, 2, 333, 64, 64, "bf16")
    go = draw_qkv(64, 1, 2, 333, 64, 64, "bf16")[0]
    a = kata.quadratic_bwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(go, "bf16"))
    b = kata.quadratic_bwd(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), to_dev(go, "f32"))
    for name, x, y in zip(("dq", "dk", "dv"), a, b):
        e = _rel(to_np(x), to_np(y), 1e-2 * float(np.linalg.norm(go)))
        print(f"  {name} rel={e:.2e}", flush=True)
        assert e <= 1e-2, name


# ------------------------------------------------------------------ O(T) chunked path
def _mfma_route(dt, p, dv):
    """bf16 inputs of these shapes run the bf16 MFMA state-form kernels."""
    return dt == "bf16" and p in (16, 32) and dv in (32, 64)


# bar of the bf16 MFMA state form: its products (states, a_t, weights, e_ts) are rounded to
# bf16 (relative 2^-9) before fp32 accumulation, as in the forward
MFMA_BWD_BAR = 1e-2


@pytest.mark.parametrize("dt,p,dv,C,T,scan", [
    ("f32", 16, 16, 16, 1, "sequential"), ("f32", 16, 32, 32, 300, "associative"),
    ("bf16", 32, 64, 16, 517, "associative"), ("bf16", 32, 32, 32, 1000, "sequential"),
    ("f32", 16, 64, 64, 777, "associative"), ("bf16", 32, 16, 64, 130, "associative"),
    ("bf16", 16, 32, 32, 1, "associative"), ("bf16", 16, 64, 16, 95, "sequential"),
    ("bf16", 32, 64, 32, 2049, "associative"), ("bf16", 16, 32, 64, 1500, "associative")])
def test_chunked_bwd_matches_oracle(dt, p, dv, C, T, scan):
    """kata_chunked_bwd against the float64 backward oracle, normwise per gradient tensor
    (T = 1: dq, dk are exactly zero, so only dv): <= 2e-4 on the fp32 VALU kernels, <= 1e-2
    on the bf16 MFMA kernels. Zero query and key rows get exactly zero gradients."""
    bar = MFMA_BWD_BAR if _mfma_route(dt, p, dv) else 2e-4
    print(f"[case] chunked bwd {dt} p={p} dv={dv} C={C} T={T} {scan} bar={bar}", flush=True)
    q, k, v = draw_qkv(81, 2, 3, T, p, dv, dt)
    go = draw_qkv(82, 2, 3, T, dv, dv, dt)[0]
    if T > 4:
        q[0, 2, 3] = 0.0
        k[1, 1, T // 2] = 0.0
    ref = kb.backward(q, k, v, go)
    got = kata.chunked_bwd(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(go, dt), C=C, scan=scan)
    floor = 1e-2 * float(np.linalg.norm(go))
    names = ("dq", "dk", "dv") if T > 1 else ("dv",)
    for name in names:
        i = ("dq", "dk", "dv").index(name)
        e = _rel(to_np(got[i]), ref[i], floor)
        print(f"  {name} rel={e:.2e}", flush=True)
        assert e <= bar, name
        _rows(name, to_np(got[i]), ref[i], ROW_BAR_MFMA if _mfma_route(dt, p, dv) else ROW_BAR_F32)
    if T > 4:
        assert np.all(to_np(got[0])[0, 2, 3] == 0.0) and np.all(to_np(got[1])[1, 1, T // 2] == 0.0)


@pytest.mark.parametrize("p,dv,T,scan", [(32, 64, 3000, "associative"), (16, 32, 2333, "associative"),
                                         (32, 32, 1200, "sequential")])
def test_chunked_bwd_mfma_many_segments(p, dv, T, scan):
    """One sequence-head pair per workgroup set: B H = 2 gives up to 64 segments per head
    (one 128-token forward chunk each at these lengths), so the forward prefixes, the
    reverse summaries and their scans all take part; bf16 MFMA bar against the oracle."""
    print(f"[case] chunked bwd mfma segments p={p} dv={dv} T={T} {scan}", flush=True)
    q, k, v = draw_qkv(85, 1, 2, T, p, dv, "bf16")
    go = draw_qkv(86, 1, 2, T, dv, dv, "bf16")[0]
    q[0, 1, T - 1] = 0.0
    k[0, 0, 128] = 0.0
    ref = kb.backward(q, k, v, go)
    got = kata.chunked_bwd(*(to_dev(x, "bf16") for x in (q, k, v, go)), C=32, scan=scan)
    floor = 1e-2 * float(np.linalg.norm(go))
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        e = _rel(to_np(a), r, floor)
        print(f"  {name} rel={e:.2e}", flush=True)
        assert e <= MFMA_BWD_BAR, name
        _rows(name, to_np(a), r, ROW_BAR_MFMA)
        _rows(name, to_np(a), r, ROW_BAR_MFMA)
    assert np.all(to_np(got[0])[0, 1, T - 1] == 0.0) and np.all(to_np(got[1])[0, 0, 128] == 0.0)


def test_chunked_bwd_mfma_matches_other_paths():
    """The bf16 MFMA state form against the fp32 VALU state form (the same values as fp32
    inputs) and the flash-style bf16 MFMA backward, at the MFMA bar."""
    q, k, v = draw_qkv(87, 1, 2, 1777, 32, 64, "bf16")
    go = draw_qkv(88, 1, 2, 1777, 64, 64, "bf16")[0]
    a = kata.chunked_bwd(*(to_dev(x, "bf16") for x in (q, k, v, go)), C=16)
    b = kata.chunked_bwd(*(to_dev(x, "f32") for x in (q, k, v, go)), C=16)
    c = kata.quadratic_bwd(*(to_dev(x, "bf16") for x in (q, k, v, go)))
    floor = 1e-2 * float(np.linalg.norm(go))
    for name, x, y, z in zip(("dq", "dk", "dv"), a, b, c):
        e1 = _rel(to_np(x), to_np(y), floor)
        e2 = _rel(to_np(x), to_np(z), floor)
        print(f"  {name} vs fp32 state form {e1:.2e}, vs flash form {e2:.2e}", flush=True)
        assert e1 <= MFMA_BWD_BAR and e2 <= MFMA_BWD_BAR, name


def test_chunked_bwd_long_matches_quadratic_path():
    """A longer sequence with many segments: the O(T) path and the flash-style VALU path
    (fp32 inputs) agree."""
    q, k, v = draw_qkv(83, 1, 2, 3000, 32, 32, "f32")
    go = draw_qkv(84, 1, 2, 3000, 32, 32, "f32")[0]
    a = kata.chunked_bwd(*(to_dev(x, "f32") for x in (q, k, v, go)), C=32)
    b = kata.quadratic_bwd(*(to_dev(x, "f32") for x in (q, k, v, go)))
    for name, x, y in zip(("dq", "dk", "dv"), a, b):
        e = _rel(to_np(x), to_np(y), 1e-2 * float(np.linalg.norm(go)))
        print(f"  {name} rel={e:.2e}", flush=True)
        assert e <= 2e-4, name


@pytest.mark.parametrize("p,dv,scan", [(32, 64, "associative"), (16, 32, "sequential"), (32, 32, "associative")])
def test_chunked_bwd_varlen(p, dv, scan):
    """Packed sequences (token-major, cu_seqlens; kata_chunked_bwd_varlen): each sequence's
    gradients against the oracle run on it alone, at the bf16 MFMA bar. An empty sequence, a
    short one (its later segments are empty) and rows after the last sequence (left at zero)."""
    B, H, max_len = 4, 2, 1400
    lens = [1300, 0, 45, 700]
    extra = 3
    print(f"[case] chunked bwd varlen p={p} dv={dv} {scan} lens={lens}", flush=True)
    q, k, v = draw_qkv(91, B, H, max_len, p, dv, "bf16")
    go = draw_qkv(92, B, H, max_len, dv, dv, "bf16")[0]

    def pack(x):
        rows = [np.transpose(x[b, :, :L], (1, 0, 2)) for b, L in enumerate(lens)]
        return np.concatenate(rows + [np.transpose(x[0, :, :extra], (1, 0, 2))], axis=0)

    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda:0")
    got = kata.chunked_bwd_varlen(*(to_dev(pack(x), "bf16") for x in (q, k, v, go)), cu, max_len, scan=scan)
    got = [to_np(x) for x in got]
    n = sum(lens)
    assert all(np.all(x[n:] == 0.0) for x in got), "rows outside every sequence were written"
    start = 0
    for b, L in enumerate(lens):
        if L:
            ref = kb.backward(q[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L], go[b:b + 1, :, :L])
            for name, x, r in zip(("dq", "dk", "dv"), got, ref):
                e = _rel(np.transpose(x[start:start + L], (1, 0, 2))[None], r,
                         1e-2 * float(np.linalg.norm(go[b, :, :L])))
                print(f"  seq {b} L={L} {name} rel={e:.2e}", flush=True)
                assert e <= MFMA_BWD_BAR, (b, name)
                _rows(f"seq {b} {name}", np.transpose(x[start:start + L], (1, 0, 2))[None], r, ROW_BAR_MFMA)
        start += L


@pytest.mark.parametrize("p,dv,lens,max_len", [(32, 64, [1300, 0, 45, 700], 1400), (64, 32, [700, 129, 0, 513], 700),
                                              (64, 64, [1300, 64, 1], 1200), (32, 32, [200, 1], 200)])
def test_quadratic_bwd_varlen(p, dv, lens, max_len):
    """Packed sequences on the flash-style MFMA backward (kata_quadratic_bwd_varlen): each
    sequence's gradients bit for bit equal to kata_quadratic_bwd on that sequence alone, and
    against the oracle at the bf16 MFMA bars. An empty sequence, one-token and short ones, a
    sequence longer than max_len (cut: its rows past max_len are not written) and rows after
    the last sequence (left at zero)."""
    B, H, extra = len(lens), 2, 3
    Tmax = max(lens)
    print(f"[case] quadratic bwd varlen p={p} dv={dv} lens={lens} max_len={max_len}", flush=True)
    q, k, v = draw_qkv(93, B, H, Tmax, p, dv, "bf16")
    go = draw_qkv(94, B, H, Tmax, dv, dv, "bf16")[0]

    def pack(x):
        rows = [np.transpose(x[b, :, :L], (1, 0, 2)) for b, L in enumerate(lens)]
        return np.concatenate(rows + [np.transpose(x[0, :, :extra], (1, 0, 2))], axis=0)

    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda:0")
    got = kata.quadratic_bwd_varlen(*(to_dev(pack(x), "bf16") for x in (q, k, v, go)), cu, max_len)
    got = [to_np(x) for x in got]
    n = sum(lens)
    assert all(np.all(x[n:] == 0.0) for x in got), "rows outside every sequence were written"
    start = 0
    for b, L in enumerate(lens):
        Lc = min(L, max_len)
        if Lc:
            seq = lambda x: np.transpose(x[start:start + Lc], (1, 0, 2))[None]
            alone = kata.quadratic_bwd(*(to_dev(x[b:b + 1, :, :Lc], "bf16") for x in (q, k, v, go)))
            for name, x, a in zip(("dq", "dk", "dv"), got, alone):
                assert np.array_equal(seq(x), to_np(a)), (b, name, "differs from the padded call")
            ref = kb.backward(q[b:b + 1, :, :Lc], k[b:b + 1, :, :Lc], v[b:b + 1, :, :Lc], go[b:b + 1, :, :Lc])
            for name, x, r in zip(("dq", "dk", "dv"), got, ref):
                e = _rel(seq(x), r, 1e-2 * float(np.linalg.norm(go[b, :, :Lc])))
                print(f"  seq {b} L={Lc} {name} rel={e:.2e}", flush=True)
                assert e <= MFMA_BWD_BAR, (b, name)
                _rows(f"seq {b} {name}", seq(x), r, ROW_BAR_MFMA)
        if L > Lc:
            assert all(np.all(x[start + Lc:start + L] == 0.0) for x in got), "rows past max_len were written"
        start += L


def test_autograd_varlen():
    """kata_attention_varlen: the packed forward and a packed backward through autograd (at
    this max_len the flash-style one), each sequence against the oracle at the bf16 MFMA bar
    (gradients rounded to bf16 add 2^-9)."""
    B, H, max_len, p, dv = 3, 2, 900, 32, 64
    lens = [900, 0, 333]
    q, k, v = draw_qkv(95, B, H, max_len, p, dv, "bf16")
    go = draw_qkv(96, B, H, max_len, dv, dv, "bf16")[0]
    pack = lambda x: np.concatenate([np.transpose(x[b, :, :L], (1, 0, 2)) for b, L in enumerate(lens)], axis=0)
    qd, kd, vd = (to_dev(pack(x), "bf16").requires_grad_(True) for x in (q, k, v))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda:0")
    o = kata.kata_attention_varlen(qd, kd, vd, cu, max_len)
    (o.float() * to_dev(pack(go), "f32")).sum().backward()
    start = 0
    for b, L in enumerate(lens):
        if L:
            ref = kb.backward(q[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L], go[b:b + 1, :, :L])
            for name, t, r in zip(("dq", "dk", "dv"), (qd.grad, kd.grad, vd.grad), ref):
                got = np.transpose(to_np(t.float())[start:start + L], (1, 0, 2))[None]
                e = _rel(got, r, 1e-2 * float(np.linalg.norm(go[b, :, :L])))
                print(f"  seq {b} {name} rel={e:.2e}", flush=True)
                assert e <= 1.2e-2, (b, name)
        start += L


def _pack_rows(x, lens, extra):
    """[B, H, T, w] -> token-major packed [sum(lens) + extra, H, w]: the sequences' rows, then
    `extra` rows of sequence 0 that belong to no sequence"""
    rows = [np.transpose(x[b, :, :L], (1, 0, 2)) for b, L in enumerate(lens)]
    return np.concatenate(rows + [np.transpose(x[0, :, :extra], (1, 0, 2))], axis=0)


@pytest.mark.parametrize("dt,p,dv,lens,max_len", [
    ("f32", 32, 64, [300, 0, 45, 170], 320), ("bf16", 16, 16, [200, 1, 0, 97], 200),
    ("f32", 64, 32, [260, 33], 240), ("bf16", 32, 48, [129, 64], 130)])
def test_quadratic_bwd_varlen_valu(dt, p, dv, lens, max_len):
    """Packed sequences on the VALU flash-style backward (kata_quadratic_bwd_varlen with fp32
    inputs or a shape without MFMA kernels): each sequence's gradients bit for bit equal to
    kata_quadratic_bwd on that sequence alone, and within the fp32 bars of the oracle. An
    empty and a one-token sequence, a sequence longer than max_len (its rows past max_len are
    not written) and rows after the last sequence (left at zero)."""
    B, H, extra = len(lens), 2, 3
    print(f"[case] quadratic bwd varlen valu {dt} p={p} dv={dv} lens={lens} max_len={max_len}", flush=True)
    q, k, v = draw_qkv(97, B, H, max(lens), p, dv, dt)
    go = draw_qkv(98, B, H, max(lens), dv, dv, dt)[0]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda:0")
    got = kata.quadratic_bwd_varlen(*(to_dev(_pack_rows(x, lens, extra), dt) for x in (q, k, v, go)), cu, max_len)
    got = [to_np(x) for x in got]
    n = sum(lens)
    assert all(np.all(x[n:] == 0.0) for x in got), "rows outside every sequence were written"
    start = 0
    for b, L in enumerate(lens):
        Lc = min(L, max_len)
        if Lc:
            seq = lambda x: np.transpose(x[start:start + Lc], (1, 0, 2))[None]
            alone = kata.quadratic_bwd(*(to_dev(np.ascontiguousarray(x[b:b + 1, :, :Lc]), dt) for x in (q, k, v, go)))
            for name, x, a in zip(("dq", "dk", "dv"), got, alone):
                assert np.array_equal(seq(x), to_np(a)), (b, name, "differs from the padded call")
            ref = kb.backward(q[b:b + 1, :, :Lc], k[b:b + 1, :, :Lc], v[b:b + 1, :, :Lc], go[b:b + 1, :, :Lc])
            # one token: the exact dq, dk vanish (o = v whatever q and k are) and fp32 returns
            # rounding noise scaled by 1 / (q_hat . k_hat), so only dv = g is checked
            for name, x, r in list(zip(("dq", "dk", "dv"), got, ref))[0 if Lc > 1 else 2:]:
                e = _rel(seq(x), r, 1e-2 * float(np.linalg.norm(go[b, :, :Lc])))
                print(f"  seq {b} L={Lc} {name} rel={e:.2e}", flush=True)
                assert e <= 2e-4, (b, name)
                _rows(f"seq {b} {name}", seq(x), r, ROW_BAR_F32)
        if L > Lc:
            assert all(np.all(x[start + Lc:start + L] == 0.0) for x in got), "rows past max_len were written"
        start += L


@pytest.mark.parametrize("dt,p,dv,scan", [("f32", 32, 64, "associative"), ("bf16", 32, 16, "sequential"),
                                           ("f32", 16, 32, "associative")])
def test_chunked_bwd_varlen_valu(dt, p, dv, scan):
    """Packed sequences on the fp32 VALU state form (kata_chunked_bwd_varlen with fp32 inputs or
    a shape without MFMA kernels; the chunk is the largest of 64, 32, 16 that fits LDS): each
    sequence's gradients against the oracle on it alone at the fp32 bars. Several segments per
    sequence-head, an empty sequence, a short one (its later segments are empty) and rows
    after the last sequence (left at zero)."""
    B, H, max_len, extra = 4, 2, 700, 3
    lens = [650, 0, 45, 300]
    print(f"[case] chunked bwd varlen valu {dt} p={p} dv={dv} {scan} lens={lens}", flush=True)
    q, k, v = draw_qkv(99, B, H, max_len, p, dv, dt)
    go = draw_qkv(100, B, H, max_len, dv, dv, dt)[0]
    q[3, 1, 7] = 0.0  # a zero query row: zero dq
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda:0")
    got = kata.chunked_bwd_varlen(*(to_dev(_pack_rows(x, lens, extra), dt) for x in (q, k, v, go)), cu, max_len,
                                  scan=scan)
    got = [to_np(x) for x in got]
    n = sum(lens)
    assert all(np.all(x[n:] == 0.0) for x in got), "rows outside every sequence were written"
    assert np.all(got[0][lens[0] + lens[1] + lens[2] + 7, 1] == 0.0), "zero query row"
    start = 0
    for b, L in enumerate(lens):
        if L:
            seq = lambda x: np.transpose(x[start:start + L], (1, 0, 2))[None]
            ref = kb.backward(q[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L], go[b:b + 1, :, :L])
            for name, x, r in zip(("dq", "dk", "dv"), got, ref):
                e = _rel(seq(x), r, 1e-2 * float(np.linalg.norm(go[b, :, :L])))
                print(f"  seq {b} L={L} {name} rel={e:.2e}", flush=True)
                assert e <= 2e-4, (b, name)
                _rows(f"seq {b} {name}", seq(x), r, ROW_BAR_F32)
        start += L


@pytest.mark.parametrize("dt,p,dv,bar", [("f32", 32, 64, 2e-4), ("bf16", 64, 32, 1.2e-2)])
def test_autograd_varlen_other_inputs(dt, p, dv, bar):
    """kata_attention_varlen beyond the bf16 state-form shapes: fp32 inputs (the packed fp32
    chunked forward and the VALU flash-style backward) and p = 64 (no chunked kernels: the
    packed quadratic forward, and the MFMA flash-style backward), each sequence against the
    oracle (fp32 bar, or the bf16 MFMA bar with gradients rounded to bf16)."""
    B, H, max_len = 3, 2, 400
    lens = [400, 0, 133]
    print(f"[case] autograd varlen {dt} p={p} dv={dv}", flush=True)
    q, k, v = draw_qkv(101, B, H, max_len, p, dv, dt)
    go = draw_qkv(102, B, H, max_len, dv, dv, dt)[0]
    pack = lambda x: np.concatenate([np.transpose(x[b, :, :L], (1, 0, 2)) for b, L in enumerate(lens)], axis=0)
    qd, kd, vd = (to_dev(pack(x), dt).requires_grad_(True) for x in (q, k, v))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda:0")
    o = kata.kata_attention_varlen(qd, kd, vd, cu, max_len)
    (o.float() * to_dev(pack(go), "f32")).sum().backward()
    start = 0
    for b, L in enumerate(lens):
        if L:
            ref = kb.backward(q[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L], go[b:b + 1, :, :L])
            for name, t, r in zip(("dq", "dk", "dv"), (qd.grad, kd.grad, vd.grad), ref):
                got = np.transpose(to_np(t.float())[start:start + L], (1, 0, 2))[None]
                e = _rel(got, r, 1e-2 * float(np.linalg.norm(go[b, :, :L])))
                print(f"  seq {b} {name} rel={e:.2e}", flush=True)
                assert e <= bar, (b, name)
        start += L


@pytest.mark.parametrize("B,H,T,p,dv,scan", [(4, 16, 128, 32, 64, "associative"), (3, 8, 33, 16, 32, "associative"),
                                             (2, 16, 256, 32, 32, "sequential")])
def test_chunked_bwd_mfma_many_heads(B, H, T, p, dv, scan):
    """The O(T) backward with many sequence-heads (up to 64) and lengths at or just past a
    chunk or segment boundary (T = 128, 33, 256), at the bf16 MFMA bar against the oracle."""
    print(f"[case] chunked bwd mfma heads B={B} H={H} T={T} p={p} dv={dv} {scan}", flush=True)
    q, k, v = draw_qkv(97, B, H, T, p, dv, "bf16")
    go = draw_qkv(98, B, H, T, dv, dv, "bf16")[0]
    ref = kb.backward(q, k, v, go)
    got = kata.chunked_bwd(*(to_dev(x, "bf16") for x in (q, k, v, go)), C=32, scan=scan)
    floor = 1e-2 * float(np.linalg.norm(go))
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        e = _rel(to_np(a), r, floor)
        print(f"  {name} rel={e:.2e}", flush=True)
        assert e <= MFMA_BWD_BAR, name
        _rows(name, to_np(a), r, ROW_BAR_MFMA)
