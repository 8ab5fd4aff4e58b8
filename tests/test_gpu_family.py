"""Parity of the reduced PSD families (KATA-Sigma g, KATA-M g) on the GPU, through the C ABI,
with the float64 family oracle (oracle/kata_families.py).

Bar: max over output rows of ||o_gpu - o_ref||_inf / ||o_ref||_inf <= 1e-4 for fp32 inputs
and <= 2e-2 for bf16 inputs (the family kernels compute in fp32; bf16 inputs are exact
bf16 numbers and the output is rounded once); lifts within fp32 rounding.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kernelized_linear_attention_normalize_amd as kata
from kata_inputs import draw_qkv
from oracle import kata_families as kf
from tests.gpu_util import TOL, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


def _case(tag, seed, B, H, T, p, dv, dt):
    print(f"[case] {tag} seed={seed} B={B} H={H} T={T} p={p} dv={dv} dtype={dt}", flush=True)
    return draw_qkv(seed, B, H, T, p, dv, dt)


@pytest.mark.parametrize("family,p,g", [("sigma", 32, 2), ("block", 32, 2), ("sigma", 64, 4),
                                        ("block", 64, 2), ("sigma", 12, 3), ("block", 128, 8)])
def test_family_lift(family, p, g):
    rng = np.random.default_rng(40)
    u = rng.standard_normal((37, p)).astype(np.float32)
    u[3] = 0.0
    got = to_np(kata.lift(to_dev(u, "f32"), family=family, g=g))
    ref = kf.lift_family(u, family, g)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6)
    assert np.all(got[3] == 0.0)


@pytest.mark.parametrize("family,p,g,dv,C,T,dt", [
    ("sigma", 32, 2, 64, 64, 700, "bf16"), ("block", 32, 2, 64, 128, 1000, "bf16"),
    ("sigma", 64, 2, 32, 32, 300, "bf16"), ("block", 16, 4, 16, 32, 257, "f32"),
    ("sigma", 16, 2, 32, 64, 130, "f32")])
def test_family_chunked(family, p, g, dv, C, T, dt):
    q, k, v = _case(f"family-chunked-{family}{g}", 41, 2, 2, T, p, dv, dt)
    q[0, 1, 5] = 0.0
    k[1, 0, :3] = 0.0
    ref = kf.naive_family(q, k, v, family, g)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    for scan in ("sequential", "associative"):
        got = to_np(kata.chunked_fwd(qd, kd, vd, C=C, scan=scan, out_dtype=torch.float32, family=family, g=g))
        err = row_rel_err(got, ref)
        print(f"  scan={scan} rel_err={err:.3e}", flush=True)
        assert err <= TOL[dt]


def test_family_chunked_many_segments_and_state():
    """Many segments through the scan, the final state in the decode layout, and decoding on."""
    family, p, g, dv, C, T0, steps = "sigma", 32, 2, 32, 32, 3000, 5
    q, k, v = _case("family-segments", 42, 1, 3, T0 + steps, p, dv, "bf16")
    ref = kf.naive_family(q, k, v, family, g)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    pre = lambda x: x[:, :, :T0].contiguous()
    o, S, Z = kata.chunked_fwd(pre(qd), pre(kd), pre(vd), C=C, scan="associative", out_dtype=torch.float32,
                               return_state=True, family=family, g=g)
    assert row_rel_err(to_np(o), ref[:, :, :T0]) <= TOL["bf16"]
    S_ref, Z_ref = kf.prefill_state_family(k[:, :, :T0], v[:, :, :T0], family, g)
    np.testing.assert_allclose(to_np(S), S_ref, rtol=1e-4, atol=1e-3)
    np.testing.assert_allclose(to_np(Z), Z_ref, rtol=1e-4, atol=1e-3)
    for t in range(T0, T0 + steps):
        st = lambda x: x[:, :, t].contiguous()
        got = kata.decode_step(st(qd), st(kd), st(vd), S, Z, out_dtype=torch.float32, family=family, g=g)
        assert row_rel_err(to_np(got), ref[:, :, t]) <= TOL["bf16"]


@pytest.mark.parametrize("dv,C,T", [(64, 128, 700), (32, 64, 1000), (64, 64, 333), (32, 128, 129)])
def test_sigma2_p64_mfma_chunked(dv, C, T):
    """KATA-Sigma 2 at p = 64 with bf16 inputs on the MFMA kernels: dv = 64 on the fp16
    kernels with the two-block lift, dv = 32 over 2T virtual rows (two 32-component blocks
    per token, the key norm over both, token-level causality); both scans, ragged T."""
    q, k, v = _case("sigma2-mfma", 46, 2, 3, T, 64, dv, "bf16")
    q[0, 2, 4] = 0.0
    k[1, 1, :2] = 0.0
    k[0, 0, 7, 32:] = 0.0  # one block of a key zero: the other block still counts
    ref = kf.naive_family(q, k, v, "sigma", 2)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    for scan in ("sequential", "associative"):
        for odt in (torch.float32, torch.bfloat16):
            got = to_np(kata.chunked_fwd(qd, kd, vd, C=C, scan=scan, out_dtype=odt, family="sigma", g=2))
            err = row_rel_err(got, ref)
            print(f"  scan={scan} out={odt} rel_err={err:.3e}", flush=True)
            assert err <= TOL["bf16"]


def test_sigma2_p64_mfma_many_segments_and_state():
    """Many segments, the final Sigma 2 state from the MFMA kernels, decoding on from it."""
    T0, steps = 5000, 4
    q, k, v = _case("sigma2-mfma-state", 47, 1, 2, T0 + steps, 64, 64, "bf16")
    ref = kf.naive_family(q, k, v, "sigma", 2)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    pre = lambda x: x[:, :, :T0].contiguous()
    o, S, Z = kata.chunked_fwd(pre(qd), pre(kd), pre(vd), C=128, scan="associative", out_dtype=torch.float32,
                               return_state=True, family="sigma", g=2)
    assert row_rel_err(to_np(o), ref[:, :, :T0]) <= TOL["bf16"]
    S_ref, Z_ref = kf.prefill_state_family(k[:, :, :T0], v[:, :, :T0], "sigma", 2)
    nw = lambda g_, r_: float(np.max(np.sqrt(((g_ - r_) ** 2).sum(axis=tuple(range(2, r_.ndim))))
                                     / np.sqrt((r_ ** 2).sum(axis=tuple(range(2, r_.ndim))))))
    es, ez = nw(to_np(S), S_ref), nw(to_np(Z), Z_ref)
    print(f"  state rel err S={es:.2e} Z={ez:.2e}", flush=True)
    assert es <= 1e-2 and ez <= 1e-2
    for t in range(T0, T0 + steps):
        st = lambda x: x[:, :, t].contiguous()
        got = kata.decode_step(st(qd), st(kd), st(vd), S, Z, out_dtype=torch.float32, family="sigma", g=2)
        assert row_rel_err(to_np(got), ref[:, :, t]) <= TOL["bf16"]


@pytest.mark.parametrize("family,p,g,dv,T,dt", [
    ("sigma", 64, 2, 64, 700, "bf16"), ("block", 64, 2, 64, 513, "bf16"), ("sigma", 32, 4, 16, 200, "f32"),
    ("block", 16, 2, 32, 65, "f32"), ("sigma", 64, 2, 16, 1100, "bf16"), ("block", 64, 2, 32, 1537, "bf16"),
    ("sigma", 64, 4, 64, 300, "bf16")])
def test_family_quadratic(family, p, g, dv, T, dt):
    """bf16 with p = 64, g = 2 runs the MFMA kernel (32-component blocks, several 512-query
    blocks, ragged key blocks); the other cases the VALU kernel."""
    q, k, v = _case(f"family-quadratic-{family}{g}", 43, 2, 2, T, p, dv, dt)
    q[1, 1, 2] = 0.0
    ref = kf.naive_family(q, k, v, family, g)
    got = to_np(kata.quadratic_fwd(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), out_dtype=torch.float32,
                                   family=family, g=g))
    err = row_rel_err(got, ref)
    print(f"  rel_err={err:.3e}", flush=True)
    assert err <= TOL[dt]


@pytest.mark.parametrize("family,p,g,dv", [("sigma", 32, 2, 64), ("block", 64, 4, 48), ("sigma", 64, 8, 16)])
def test_family_decode_from_oracle_state(family, p, g, dv):
    """Decode steps from a float64-built prefill state (rounded to fp32) against the oracle."""
    rng = np.random.default_rng(44)
    N, H, hist, steps = 3, 2, 200, 4
    kh = rng.standard_normal((N, H, hist, p))
    vh = rng.standard_normal((N, H, hist, dv))
    S0, Z0 = kf.prefill_state_family(kh, vh, family, g)
    S0, Z0 = np.ascontiguousarray(S0, dtype=np.float32), np.ascontiguousarray(Z0, dtype=np.float32)
    q, k, v = (rng.standard_normal((steps, N, H, x)).astype(np.float32) for x in (p, p, dv))
    ref, S_ref, Z_ref = kf.decode_steps_family(S0, Z0, q, k, v, family, g)
    S = torch.from_numpy(S0).to("cuda:0")
    Z = torch.from_numpy(Z0).to("cuda:0")
    for t in range(steps):
        got = kata.decode_step(to_dev(q[t], "f32"), to_dev(k[t], "f32"), to_dev(v[t], "f32"), S, Z,
                               family=family, g=g)
        assert row_rel_err(to_np(got), ref[t]) <= TOL["f32"]
    np.testing.assert_allclose(to_np(S), S_ref, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(to_np(Z), Z_ref, rtol=1e-5, atol=1e-4)


def test_family_full_is_the_full_path():
    """family='full' routes to the full-map kernels: bit-identical outputs."""
    q, k, v = _case("family-full", 45, 1, 2, 500, 32, 64, "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    assert torch.equal(kata.chunked_fwd(qd, kd, vd, C=64), kata.chunked_fwd(qd, kd, vd, C=64, family="full"))
    assert torch.equal(kata.quadratic_fwd(qd, kd, vd), kata.quadratic_fwd(qd, kd, vd, family="full", g=1))


# ------------------------------------------------------------------ higher even orders
@pytest.mark.parametrize("p,r", [(4, 2), (16, 2), (5, 3), (3, 4), (8, 1)])
def test_order_lift(p, r):
    rng = np.random.default_rng(55)
    u = rng.standard_normal((21, p)).astype(np.float32)
    u[2] = 0.0
    got = to_np(kata.lift(to_dev(u, "f32"), order=r))
    ref = kf.lift_order(u, r)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=0, atol=5e-6)


@pytest.mark.parametrize("p,dv,T,r,dt", [(64, 64, 700, 2, "bf16"), (32, 16, 333, 2, "bf16"), (16, 32, 200, 3, "f32"),
                                         (64, 64, 130, 4, "bf16"), (32, 32, 65, 2, "f32")])
def test_order_quadratic(p, dv, T, r, dt):
    """Weights (q_hat . k_hat)^(2r): bf16 with r = 2 runs the MFMA kernel, the rest VALU."""
    q, k, v = _case(f"order-quadratic-r{r}", 56, 2, 2, T, p, dv, dt)
    ref = kf.naive_order(q, k, v, r)
    got = to_np(kata.quadratic_fwd(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), out_dtype=torch.float32, order=r))
    err = row_rel_err(got, ref)
    print(f"  rel_err={err:.3e}", flush=True)
    assert err <= TOL[dt]
