"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Bar: max over output rows of ||o_gpu - o_ref||_inf / ||o_ref||_inf <= 1e-4 for fp32 inputs
and <= 2e-2 for bf16 inputs; the packed index map of kata_lift must match exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kernelized_linear_attention_normalize_amd as kata
from kata_inputs import DECODE, WORKLOADS, draw_decode_history, draw_decode_steps, draw_qkv, round_bf16
from oracle import kata_oracle as ko
from tests.gpu_util import TOL, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


def _case(tag, seed, B, H, T, p, dv, dt):
    print(f"[case] {tag} seed={seed} B={B} H={H} T={T} p={p} dv={dv} dtype={dt}", flush=True)
    return draw_qkv(seed, B, H, T, p, dv, dt)


# ------------------------------------------------------------------ lift
@pytest.mark.parametrize("p", [1, 3, 16, 32, 64, 128])
def test_lift_index_map_exact(p):
    ii, jj = ko.packed_pairs(p)
    n = ko.packed_dim(p)
    rows = []
    for i in range(p):
        e = np.zeros(p, np.float32); e[i] = 2.0
        rows.append(e)
    for (i, j) in [(0, p - 1), (p // 2, p - 1), (0, p // 3)]:
        if i != j:
            e = np.zeros(p, np.float32); e[i] = e[j] = 1.0
            rows.append(e)
    u = np.stack(rows)
    psi = to_np(kata.lift(to_dev(u, "f32")))
    assert psi.shape == (len(rows), n)
    for r in range(p):  # e_i -> a single 1 at the position of (i, i)
        nz = np.flatnonzero(psi[r])
        assert len(nz) == 1 and (ii[nz[0]], jj[nz[0]]) == (r, r) and psi[r, nz[0]] == 1.0
    for r in range(p, len(rows)):
        i, j = np.flatnonzero(u[r])[[0, -1]]
        nz = set((int(ii[x]), int(jj[x])) for x in np.flatnonzero(psi[r]))
        assert nz == {(i, i), (j, j), (i, j)}


@pytest.mark.parametrize("in_dt,out_dt", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
def test_lift_values(in_dt, out_dt):
    rng = np.random.default_rng(7)
    u = rng.standard_normal((1000, 32)).astype(np.float32)
    u[5] = 0.0
    if in_dt == "bf16":
        u = round_bf16(u)
    out = kata.lift(to_dev(u, in_dt), out_dtype=torch.bfloat16 if out_dt == "bf16" else torch.float32)
    got = to_np(out)
    ref = ko.lift(u)
    tol = 1e-6 if out_dt == "f32" else 2 ** -8
    assert np.all(got[5] == 0.0)
    assert np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-3)) < tol * 4
    assert np.allclose(np.linalg.norm(got[np.arange(1000) != 5], axis=-1), 1.0, atol=tol * 8)


# ------------------------------------------------------------------ tiny (fp32)
@pytest.mark.parametrize("scan", ["sequential", "associative"])
def test_tiny_chunked(scan):
    w = WORKLOADS["tiny"]
    q, k, v = _case("tiny-chunked", w.seed, w.B, w.H, w.T, w.p, w.dv, w.dtype)
    ref = ko.naive(q, k, v)
    got = to_np(kata.chunked_fwd(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), C=32, scan=scan))
    assert row_rel_err(got, ref) <= TOL["f32"]


def test_tiny_quadratic():
    w = WORKLOADS["tiny"]
    q, k, v = _case("tiny-quadratic", w.seed, w.B, w.H, w.T, w.p, w.dv, w.dtype)
    ref = ko.naive(q, k, v)
    got = to_np(kata.quadratic_fwd(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")))
    assert row_rel_err(got, ref) <= TOL["f32"]


def test_tiny_recurrent_decode():
    w = WORKLOADS["tiny"]
    q, k, v = _case("tiny-recurrent", w.seed, w.B, w.H, w.T, w.p, w.dv, w.dtype)
    ref = ko.naive(q, k, v)
    n = ko.packed_dim(w.p)
    S = torch.zeros((w.B, w.H, n, w.dv), dtype=torch.float32, device="cuda:0")
    Z = torch.zeros((w.B, w.H, n), dtype=torch.float32, device="cuda:0")
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    outs = []
    for t in range(w.T):
        outs.append(kata.decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                     vd[:, :, t].contiguous(), S, Z))
    got = to_np(torch.stack(outs, dim=2))
    assert row_rel_err(got, ref) <= TOL["f32"]
    S_ref, Z_ref = ko.prefill_state(k, v)
    assert np.allclose(to_np(S), S_ref, rtol=1e-4, atol=1e-4)
    assert np.allclose(to_np(Z), Z_ref, rtol=1e-4, atol=1e-4)


# ------------------------------------------------------------------ bf16 chunked: shapes, tails, modes
@pytest.mark.parametrize("p,dv,C,T", [(32, 64, 64, 700), (32, 64, 128, 1000), (32, 64, 32, 300),
                                      (16, 16, 32, 257), (16, 64, 64, 640), (32, 32, 128, 129),
                                      (32, 16, 64, 65), (16, 32, 128, 390)])
def test_chunked_bf16_shapes(p, dv, C, T):
    q, k, v = _case("chunked-bf16", 11, 2, 3, T, p, dv, "bf16")
    q[0, 1, 7] = 0.0          # a zero query row
    k[1, 0, :3] = 0.0         # zero keys at the start of a sequence
    ref = ko.naive(q, k, v)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    for scan in ("sequential", "associative"):
        got = to_np(kata.chunked_fwd(qd, kd, vd, C=C, scan=scan))
        err = row_rel_err(got, ref)
        print(f"  scan={scan} rel_err={err:.3e}", flush=True)
        assert err <= TOL["bf16"]
    got32 = to_np(kata.chunked_fwd(qd, kd, vd, C=C, scan="associative", out_dtype=torch.float32))
    assert row_rel_err(got32, ref) <= TOL["bf16"]


@pytest.mark.parametrize("H,dt,p,dv", [(1, "bf16", 32, 64), (10, "bf16", 32, 64), (1, "f32", 16, 32),
                                       (10, "f32", 16, 32)])
def test_chunked_many_segments(H, dt, p, dv):
    """Few heads over many chunks: 63 (H=1) and 25 (H=10) segment summaries per head go
    through the inter-segment scan (its 64- and 32-lane segment layouts)."""
    q, k, v = _case("chunked-segments", 14, 1, H, 4096, p, dv, dt)
    ref = ko.naive(q, k, v)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    got = to_np(kata.chunked_fwd(qd, kd, vd, C=32, scan="associative", out_dtype=torch.float32))
    err = row_rel_err(got, ref)
    print(f"  rel_err={err:.3e}", flush=True)
    assert err <= TOL[dt]


@pytest.mark.parametrize("case", ["v*1e4", "v*1e-4", "v jumps 1e4 at T/2", "q*1e-3 k*1e3", "v*1e30"])
@pytest.mark.parametrize("C,scan", [(128, "associative"), (64, "sequential")])
def test_chunked_value_and_row_scales(case, C, scan):
    """The fp16-operand kernels carry values as sigma v with a power-of-two sigma chosen from
    a running bound, and queries as lambda q_hat: the output must not depend on the scale of
    v beyond its rounding, nor on the norms of q and k. Uniformly scaled values, a jump of the
    value scale inside the sequence (sigma falls mid-sequence and the state is rescaled),
    values near the top of the fp32 range, and scaled query and key rows, at the bf16 bar."""
    B, H, T, p, dv = 1, 4, 2048, 32, 64
    q, k, v = draw_qkv(61, B, H, T, p, dv, "f32")
    if case == "v*1e4":
        v = v * 1e4
    elif case == "v*1e-4":
        v = v * 1e-4
    elif case == "v jumps 1e4 at T/2":
        v[:, :, T // 2:] *= 1e4
    elif case == "q*1e-3 k*1e3":
        q, k = q * 1e-3, k * 1e3
    else:
        v = v * 1e30
    q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    print(f"[case] chunked scales {case} C={C} {scan}", flush=True)
    ref = ko.naive(q, k, v)
    got = to_np(kata.chunked_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), C=C, scan=scan,
                                 out_dtype=torch.float32))
    assert np.all(np.isfinite(got))
    e = row_rel_err(got, ref)
    print(f"  row-rel err {e:.2e}", flush=True)
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("T", [1, 5, 31, 64])
def test_chunked_short_sequences(T):
    q, k, v = _case("chunked-short", 12, 1, 2, T, 32, 64, "bf16")
    ref = ko.naive(q, k, v)
    got = to_np(kata.chunked_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), C=64))
    assert row_rel_err(got, ref) <= TOL["bf16"]


def test_chunked_empty_is_noop():
    q = torch.zeros((1, 2, 0, 32), dtype=torch.bfloat16, device="cuda:0")
    v = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    assert kata.chunked_fwd(q, q, v, C=64).shape == (1, 2, 0, 64)
    assert kata.quadratic_fwd(q, q, v).shape == (1, 2, 0, 64)


@pytest.mark.parametrize("dt,scan", [("bf16", "associative"), ("bf16", "sequential"), ("f32", "associative")])
def test_chunked_passes_match_one_call(dt, scan):
    """The three passes issued as separate calls reproduce one kata_chunked_fwd call bit for bit."""
    p, dv = (32, 64) if dt == "bf16" else (16, 32)
    q, k, v = _case("chunked-passes", 15, 1, 3, 2500, p, dv, dt)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    one = kata.chunked_fwd(qd, kd, vd, C=64, scan=scan)
    need = kata.chunked_workspace_bytes(1, 3, 2500, p, dv, 64, kata._scan_code(scan),
                                        torch.bfloat16 if dt == "bf16" else torch.float32)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(one)
    for mask in (kata.PASS_SUMMARIES, kata.PASS_SCAN, kata.PASS_SEGMENTS):
        kata.chunked_fwd(qd, kd, vd, C=64, scan=scan, out=out, workspace=ws, passes=mask)
    assert torch.equal(out, one)


def test_chunked_deterministic():
    q, k, v = _case("determinism", 13, 1, 4, 3000, 32, 64, "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    a = kata.chunked_fwd(qd, kd, vd, C=64)
    b = kata.chunked_fwd(qd, kd, vd, C=64)
    assert torch.equal(a, b)


# ------------------------------------------------------------------ prefill -> decode handoff
def _normwise(got, ref):
    """max over (b, h) of ||got - ref||_F / ||ref||_F (last one or two axes are the state)."""
    axes = tuple(range(2, ref.ndim))
    return float(np.max(np.sqrt(((got - ref) ** 2).sum(axes)) / np.sqrt((ref ** 2).sum(axes))))


@pytest.mark.parametrize("dt,p,dv,C,scan,T0", [
    ("bf16", 32, 64, 128, "associative", 4100), ("bf16", 32, 64, 64, "sequential", 700),
    ("bf16", 16, 32, 32, "associative", 2000), ("bf16", 32, 16, 64, "associative", 129),
    ("bf16", 16, 64, 128, "sequential", 300),
    ("f32", 16, 32, 32, "associative", 1000), ("f32", 16, 16, 64, "sequential", 77)])
def test_prefill_state_then_decode(dt, p, dv, C, scan, T0):
    """kata_chunked_fwd_state's final state continues each sequence through kata_decode_step:
    the prefill outputs, the state after the prefill and every decode output match the
    oracle over the whole sequence."""
    steps, B, H = 6, 2, 3
    q, k, v = _case("handoff", 16, B, H, T0 + steps, p, dv, dt)
    k[1, 2, :5] = 0.0  # zero keys add nothing to the state
    ref = ko.naive(q, k, v)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    pre = lambda x: x[:, :, :T0].contiguous()
    o, S, Z = kata.chunked_fwd(pre(qd), pre(kd), pre(vd), C=C, scan=scan,
                               out_dtype=torch.float32, return_state=True)
    assert row_rel_err(to_np(o), ref[:, :, :T0]) <= TOL[dt]
    S_ref, Z_ref = ko.prefill_state(k[:, :, :T0], v[:, :, :T0])
    es, ez = _normwise(to_np(S), S_ref), _normwise(to_np(Z), Z_ref)
    print(f"  state rel err S={es:.2e} Z={ez:.2e}", flush=True)
    bar = 1e-2 if dt == "bf16" else 1e-5
    assert es <= bar and ez <= bar
    for t in range(T0, T0 + steps):
        step = lambda x: x[:, :, t].contiguous()
        got = kata.decode_step(step(qd), step(kd), step(vd), S, Z, out_dtype=torch.float32)
        assert row_rel_err(to_np(got), ref[:, :, t]) <= TOL[dt]


def test_prefill_state_empty_sequences():
    """T = 0: the state is zero (written, whatever the buffers held)."""
    q = torch.zeros((2, 3, 0, 32), dtype=torch.bfloat16, device="cuda:0")
    v = torch.zeros((2, 3, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    o, S, Z = kata.chunked_fwd(q, q, v, C=64, return_state=True)
    assert o.shape == (2, 3, 0, 64) and S.shape == (2, 3, 528, 64) and Z.shape == (2, 3, 528)
    assert int(torch.count_nonzero(S)) == 0 and int(torch.count_nonzero(Z)) == 0


def test_prefill_state_matches_plain_forward():
    """Asking for the state does not change o (same kernels, bit for bit)."""
    q, k, v = _case("handoff-o", 17, 1, 4, 3000, 32, 64, "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    a = kata.chunked_fwd(qd, kd, vd, C=128)
    b, _, _ = kata.chunked_fwd(qd, kd, vd, C=128, return_state=True)
    assert torch.equal(a, b)


# ------------------------------------------------------------------ fp32 at p = 32, dv = 64
@pytest.mark.parametrize("C,scan,T", [(64, "associative", 1000), (128, "associative", 1500), (128, "sequential", 700),
                                      (32, "associative", 333)])
def test_chunked_f32_p32_dv64(C, scan, T):
    """fp32 inputs at p = 32, dv = 64 (for C = 64, 128 the fp32 kernel runs twice, once per
    half of the value columns) against the definition at the fp32 bar, with the final state
    against the oracle's prefill state."""
    q, k, v = _case("f32-p32-dv64", 21, 2, 3, T, 32, 64, "f32")
    q[1, 2, 5] = 0.0
    ref = ko.naive(q, k, v)
    o, S, Z = kata.chunked_fwd(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), C=C, scan=scan,
                               out_dtype=torch.float32, return_state=True)
    err = row_rel_err(to_np(o), ref)
    print(f"  fp32 p=32 dv=64 C={C} {scan} T={T}: rel_err={err:.2e}", flush=True)
    assert err <= TOL["f32"]
    S_ref, Z_ref = ko.prefill_state(k, v)
    assert np.allclose(to_np(S), S_ref, rtol=1e-4, atol=1e-3)
    assert np.allclose(to_np(Z), Z_ref, rtol=1e-4, atol=1e-3)


# ------------------------------------------------------------------ mid config (every head)
def test_mid_all_heads():
    """The mid configuration, all 128 (b, h) and every row, against the O(T^2) definition,
    for the chunked form in both scans and the quadratic form."""
    w = WORKLOADS["mid"]
    q, k, v = _case("mid", w.seed, w.B, w.H, w.T, w.p, w.dv, w.dtype)
    ref = ko.naive(q, k, v)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    forms = {
        "chunked C=64 associative": lambda: kata.chunked_fwd(qd, kd, vd, C=64, scan="associative"),
        "chunked C=64 sequential": lambda: kata.chunked_fwd(qd, kd, vd, C=64, scan="sequential"),
        "chunked C=128 associative": lambda: kata.chunked_fwd(qd, kd, vd, C=128, scan="associative"),
        "quadratic": lambda: kata.quadratic_fwd(qd, kd, vd),
    }
    for name, run in forms.items():
        got = to_np(run())
        errs = [row_rel_err(got[b, h], ref[b, h]) for b in range(w.B) for h in range(w.H)]
        print(f"  mid {name}: max row err over all {len(errs)} heads {max(errs):.3e}", flush=True)
        assert max(errs) <= TOL["bf16"]


# ------------------------------------------------------------------ long config (full heads)
LONG_FULL_HEADS = (0, 15)


@pytest.fixture(scope="module")
def long_case():
    """The long configuration with a float64 reference for every row of heads 0 and 15:
    the oracle's chunked-state form at C = 512, itself compared with the O(T^2) definition
    on rows spread over the sequence (chunk edges included)."""
    w = WORKLOADS["long"]
    q, k, v = _case("long", w.seed, w.B, w.H, w.T, w.p, w.dv, w.dtype)
    tie_rows = [0, 1, 63, 64, 127, 128, 511, 512, 513, 65535, 65536, 100000, w.T - 1]
    refs = {}
    for h in LONG_FULL_HEADS:
        ref = ko.chunked(q[0, h], k[0, h], v[0, h], C=512, scan="sequential")
        tie = row_rel_err(ref[tie_rows], ko.naive_rows(q[0, h], k[0, h], v[0, h], tie_rows))
        print(f"  long head {h}: oracle chunked(C=512) vs naive on {len(tie_rows)} rows {tie:.2e}", flush=True)
        assert tie <= 1e-10
        refs[h] = ref
    dev = (to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"))
    return w, q, k, v, refs, dev


@pytest.mark.parametrize("scan", ["associative", "sequential"])
@pytest.mark.parametrize("C", [64, 128])
def test_long_full_heads(long_case, C, scan):
    """Every row of two whole heads of the 131072-token configuration, in the launch
    configuration the benchmark times (C = 128, associative) and the other three; sampled
    rows of two more heads against the O(T^2) definition."""
    w, q, k, v, refs, (qd, kd, vd) = long_case
    got = kata.chunked_fwd(qd, kd, vd, C=C, scan=scan)
    for h in LONG_FULL_HEADS:
        err = row_rel_err(to_np(got[0, h]), refs[h])
        print(f"  long C={C} {scan} head={h}: max row err over {w.T} rows {err:.3e}", flush=True)
        assert err <= TOL["bf16"]
    rng = np.random.default_rng(99)
    rows = sorted(set([0, 1, 2, 7, C - 1, C, 8191, 8192, w.T - 1] + list(rng.integers(0, w.T, 24))))
    for h in (5, 9):
        err = row_rel_err(to_np(got[0, h, rows]), ko.naive_rows(q[0, h], k[0, h], v[0, h], rows))
        print(f"  long C={C} {scan} head={h}: sampled rows {err:.3e}", flush=True)
        assert err <= TOL["bf16"]


# ------------------------------------------------------------------ quadratic config
def test_quadratic_config():
    """Two whole heads of the quadratic configuration against the definition, sampled rows
    of a third."""
    w = WORKLOADS["quadratic"]
    q, k, v = _case("quadratic", w.seed, w.B, w.H, w.T, w.p, w.dv, w.dtype)
    got = to_np(kata.quadratic_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")))
    for (b, h) in ((0, 0), (1, 15)):
        err = row_rel_err(got[b, h], ko.naive(q[b, h], k[b, h], v[b, h]))
        print(f"  quadratic head=({b},{h}): max row err over {w.T} rows {err:.3e}", flush=True)
        assert err <= TOL["bf16"]
    rng = np.random.default_rng(98)
    rows = sorted(set([0, 1, 5, 127, 128, 4095, w.T - 1] + list(rng.integers(0, w.T, 30))))
    err = row_rel_err(got[1, 8, rows], ko.naive_rows(q[1, 8], k[1, 8], v[1, 8], rows))
    print(f"  quadratic head=(1,8): sampled rows {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("p,dv,T", [(16, 16, 200), (32, 32, 333), (64, 16, 130), (16, 64, 1),
                                    (64, 64, 1100), (32, 16, 1537), (16, 32, 700)])
def test_quadratic_shapes(p, dv, T):
    """Single and several 512-query blocks (the longest-first block order over all (b,h)),
    ragged key blocks, a zero query row."""
    q, k, v = _case("quadratic-shapes", 14, 2, 2, T, p, dv, "bf16")
    q[1, 1, 3 % T] = 0.0
    ref = ko.naive(q, k, v)
    got = to_np(kata.quadratic_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")))
    assert row_rel_err(got, ref) <= TOL["bf16"]


# ------------------------------------------------------------------ decode (small)
def test_decode_small_from_prefill():
    rng = np.random.default_rng(15)
    N, H, p, dv, Th, steps = 3, 2, 32, 64, 200, 20
    kh = rng.standard_normal((N, H, Th, p)).astype(np.float32)
    vh = rng.standard_normal((N, H, Th, dv)).astype(np.float32)
    S0, Z0 = ko.prefill_state(kh, vh)
    S0, Z0 = np.ascontiguousarray(S0, np.float32), np.ascontiguousarray(Z0, np.float32)
    qs = round_bf16(rng.standard_normal((steps, N, H, p)).astype(np.float32))
    ks = round_bf16(rng.standard_normal((steps, N, H, p)).astype(np.float32))
    vs = round_bf16(rng.standard_normal((steps, N, H, dv)).astype(np.float32))
    ref, S_ref, Z_ref = ko.decode_steps(S0, Z0, qs, ks, vs)
    S = torch.from_numpy(S0).cuda(); Z = torch.from_numpy(Z0).cuda()
    qd, kd, vd = to_dev(qs, "bf16"), to_dev(ks, "bf16"), to_dev(vs, "bf16")
    outs = [kata.decode_step(qd[s], kd[s], vd[s], S, Z) for s in range(steps)]
    got = to_np(torch.stack(outs))
    assert row_rel_err(got, ref) <= TOL["bf16"]
    assert np.allclose(to_np(S), S_ref, rtol=1e-4, atol=1e-3)
    assert np.allclose(to_np(Z), Z_ref, rtol=1e-4, atol=1e-3)


def _threaded(fn, parts, workers=16):
    """Run fn over independent parts on host threads (numpy releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, parts))


def test_decode_config_all_heads():
    """The decode configuration in its benchmarked launch shape: 128 sequences x 16 heads,
    every head prefilled from its seeded 4096-token history, 256 steps; every output of every
    step and the final states against the oracle."""
    N, H, p, dv, steps = DECODE["N"], DECODE["H"], DECODE["p"], DECODE["dv"], DECODE["steps"]
    print(f"[case] decode config N={N} H={H} p={p} dv={dv} steps={steps}", flush=True)
    kh, vh = draw_decode_history(DECODE["hist_seed"], N, H, DECODE["hist"], p, dv)
    n = p * (p + 1) // 2
    S0 = np.empty((N, H, n, dv), np.float32)
    Z0 = np.empty((N, H, n), np.float32)

    def prefill(a):
        s_, z_ = ko.prefill_state(kh[a], vh[a])
        S0[a], Z0[a] = s_, z_

    _threaded(prefill, range(N), workers=8)
    del kh, vh
    qs, ks, vs = draw_decode_steps(DECODE["step_seed"], steps, N, H, p, dv)
    S = torch.from_numpy(S0).cuda()
    Z = torch.from_numpy(Z0).cuda()
    qd, kd, vd = to_dev(qs, "bf16"), to_dev(ks, "bf16"), to_dev(vs, "bf16")
    out = torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda:0")
    got = np.empty((steps, N, H, dv), np.float32)
    for st in range(steps):
        kata.decode_step(qd[st], kd[st], vd[st], S, Z, out=out)
        got[st] = out.float().cpu().numpy()
    S_end, Z_end = to_np(S), to_np(Z)
    groups = [slice(a, a + 8) for a in range(0, N, 8)]

    def check(sl):
        ref, S_ref, Z_ref = ko.decode_steps(S0[sl], Z0[sl], qs[:, sl], ks[:, sl], vs[:, sl])
        errs = [row_rel_err(got[:, sl][:, a, b], ref[:, a, b]) for a in range(ref.shape[1]) for b in range(H)]
        s_ok = np.allclose(S_end[sl], S_ref, rtol=1e-4, atol=1e-2)
        z_ok = np.allclose(Z_end[sl], Z_ref, rtol=1e-4, atol=1e-2)
        return max(errs), s_ok and z_ok

    res = _threaded(check, groups, workers=8)
    err = max(r[0] for r in res)
    print(f"  decode: max row err over {N * H} heads x {steps} steps {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    assert all(r[1] for r in res)
