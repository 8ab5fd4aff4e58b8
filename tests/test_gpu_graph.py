"""The entry points under HIP graph capture (torch.cuda.CUDAGraph on ROCm records the
kernels the library enqueues on the capturing stream). Each captured graph is replayed
several times with new inputs copied into its static tensors and eager work between the
replays; every replay is compared with the eager call on the same inputs, bit for bit.

The library only enqueues kernels (zero fills are a fill kernel, never a memset node), so
capture needs nothing special from it."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kernelized_linear_attention_normalize_amd as kata
from kata_inputs import draw_qkv
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("scan", ["associative", "sequential"])
def test_graph_chunked_forward(scan):
    B, H, T, p, dv, C = 1, 4, 5000, 32, 64, 128
    print(f"[case] graph chunked {scan}", flush=True)
    q, k, v = (to_dev(x, "bf16") for x in draw_qkv(70, B, H, T, p, dv, "bf16"))
    out = torch.empty((B, H, T, dv), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(max(kata.chunked_workspace_bytes(B, H, T, p, dv, C, kata._scan_code(scan)), 1),
                     dtype=torch.uint8, device="cuda:0")
    g = _capture(lambda: kata.chunked_fwd(q, k, v, C=C, scan=scan, out=out, workspace=ws))
    for rep in range(3):
        nq, nk, nv = (to_dev(x, "bf16") for x in draw_qkv(71 + rep, B, H, T, p, dv, "bf16"))
        q.copy_(nq), k.copy_(nk), v.copy_(nv)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = kata.chunked_fwd(nq, nk, nv, C=C, scan=scan, out_dtype=torch.float32)  # eager, between replays
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {rep} differs from the eager call"


def test_graph_quadratic_and_decode():
    """The quadratic forward and a decode step in one graph: every replay advances the state
    by one token, exactly as the eager steps do."""
    N, H, p, dv = 8, 4, 32, 64
    n = p * (p + 1) // 2
    rng = np.random.default_rng(75)
    S0 = torch.from_numpy(rng.standard_normal((N, H, n, dv), dtype=np.float32)).abs().cuda()
    Z0 = torch.from_numpy(rng.standard_normal((N, H, n), dtype=np.float32)).abs().cuda()
    S, Z = S0.clone(), Z0.clone()
    Se, Ze = S0.clone(), Z0.clone()
    qs, ks, vs = (torch.empty((N, H, w), dtype=torch.bfloat16, device="cuda:0") for w in (p, p, dv))
    o = torch.empty((N, H, dv), dtype=torch.float32, device="cuda:0")
    Bq, Tq = 2, 700
    qq, kq, vq = (to_dev(x, "bf16") for x in draw_qkv(76, Bq, H, Tq, p, dv, "bf16"))
    oq = torch.empty((Bq, H, Tq, dv), dtype=torch.float32, device="cuda:0")

    def step():
        kata.decode_step(qs, ks, vs, S, Z, out=o)
        kata.quadratic_fwd(qq, kq, vq, out=oq)

    # the warm-up inside _capture runs one step on (S, Z): start the eager copy from there
    qs.copy_(torch.zeros_like(qs)), ks.copy_(torch.zeros_like(ks)), vs.copy_(torch.zeros_like(vs))
    g = _capture(step)
    Se.copy_(S), Ze.copy_(Z)
    for rep in range(4):
        tq, tk, tv = (torch.from_numpy(rng.standard_normal((N, H, w), dtype=np.float32)).to(torch.bfloat16).cuda()
                      for w in (p, p, dv))
        qs.copy_(tq), ks.copy_(tk), vs.copy_(tv)
        g.replay()
        torch.cuda.synchronize()
        oe = kata.decode_step(tq, tk, tv, Se, Ze, out_dtype=torch.float32)  # eager step between replays
        torch.cuda.synchronize()
        assert torch.equal(o, oe) and torch.equal(S, Se) and torch.equal(Z, Ze), f"decode replay {rep}"
        assert torch.equal(oq, kata.quadratic_fwd(qq, kq, vq, out_dtype=torch.float32)), f"quadratic replay {rep}"


def test_graph_chunked_backward():
    """The O(T) backward (bf16 MFMA state form: forward summaries, scans, three kernels) under
    capture with a caller-provided workspace: every replay equals the eager call."""
    B, H, T, p, dv = 1, 2, 1500, 32, 64
    print("[case] graph chunked backward", flush=True)
    q, k, v = (to_dev(x, "bf16") for x in draw_qkv(77, B, H, T, p, dv, "bf16"))
    go = to_dev(draw_qkv(78, B, H, T, dv, dv, "bf16")[0], "bf16")
    lib = kata.load()
    ws = torch.empty(int(lib.kata_chunked_bwd_workspace_bytes(B, H, T, p, dv, 32, kata.SCAN_ASSOCIATIVE)),
                     dtype=torch.uint8, device="cuda:0")
    outs = []

    def step():
        outs[:] = kata.chunked_bwd(q, k, v, go, C=32, workspace=ws)

    g = _capture(step)
    for rep in range(3):
        nq, nk, nv = (to_dev(x, "bf16") for x in draw_qkv(79 + rep, B, H, T, p, dv, "bf16"))
        q.copy_(nq), k.copy_(nk), v.copy_(nv)
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in outs]
        ref = kata.chunked_bwd(nq, nk, nv, go, C=32)  # eager, between replays
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"


def test_graph_packed_sequences_new_lengths():
    """The packed forms (chunked and quadratic) in one graph. cu_seqlens is device memory read
    by the kernels, so every replay takes new sequence lengths as well as new tokens without a
    new capture (the grid is sized by max_len); each replay equals the eager calls bit for bit."""
    H, p, dv, C, max_len = 2, 32, 64, 64, 700
    total = 1500
    print("[case] graph packed sequences", flush=True)
    rng = np.random.default_rng(83)

    def draw(lens):
        x = [torch.from_numpy(rng.standard_normal((total, H, w), dtype=np.float32)).to(torch.bfloat16).cuda()
             for w in (p, p, dv)]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda:0")
        return x, cu

    (q, k, v), cu = draw([700, 0, 300, 500])
    oc = torch.empty((total, H, dv), dtype=torch.float32, device="cuda:0")
    oq = torch.empty((total, H, dv), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(max(kata.chunked_workspace_bytes(4, H, max_len, p, dv, C, kata.SCAN_ASSOCIATIVE), 1),
                     dtype=torch.uint8, device="cuda:0")

    def step():
        kata.chunked_fwd_varlen(q, k, v, cu, max_len, C=C, out=oc, workspace=ws)
        kata.quadratic_fwd_varlen(q, k, v, cu, max_len, out=oq)

    g = _capture(step)
    for rep, lens in enumerate([[1, 699, 0, 700], [350, 350, 77, 123], [700, 700, 0, 0]]):
        (nq, nk, nv), ncu = draw(lens)
        q.copy_(nq), k.copy_(nk), v.copy_(nv), cu.copy_(ncu)
        oc.fill_(7.0), oq.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        gc, gq = oc.clone(), oq.clone()
        rc = torch.full_like(oc, 7.0)
        rq = torch.full_like(oq, 7.0)
        kata.chunked_fwd_varlen(nq, nk, nv, ncu, max_len, C=C, out=rc)  # eager, between replays
        kata.quadratic_fwd_varlen(nq, nk, nv, ncu, max_len, out=rq)
        torch.cuda.synchronize()
        n = sum(lens)
        assert torch.equal(gc, rc) and torch.equal(gq, rq), f"replay {rep} differs from the eager calls"
        assert bool((gc[n:] == 7.0).all()) and bool((gq[n:] == 7.0).all()), f"replay {rep}: rows past the sequences"
