"""The Python binding's guards: inputs whose dtypes disagree, or a caller's output tensor of the
wrong shape, are rejected before any library call (the C calls take one input dtype and write
through the output pointer, so either would send a kernel past a buffer)."""
from __future__ import annotations

import pytest
import torch

import kernelized_linear_attention_normalize_amd as kata

pytestmark = pytest.mark.gpu


def _qkv(B=1, H=2, T=64, p=32, dv=64, dt=torch.bfloat16):
    g = torch.Generator(device="cpu").manual_seed(5)
    mk = lambda *s: torch.randn(*s, generator=g).to(dt).cuda()
    return mk(B, H, T, p), mk(B, H, T, p), mk(B, H, T, dv)


def test_mixed_input_dtypes_are_rejected():
    q, k, v = _qkv()
    for args in ((q.float(), k, v), (q, k.float(), v), (q, k, v.float())):
        with pytest.raises(TypeError):
            kata.chunked_fwd(*args, C=64)
        with pytest.raises(TypeError):
            kata.quadratic_fwd(*args)
    n = kata.packed_dim(32)
    S = torch.zeros(1, 2, n, 64, device="cuda")
    Z = torch.zeros(1, 2, n, device="cuda")
    with pytest.raises(TypeError):
        kata.decode_step(q[:, :, 0].contiguous(), k[:, :, 0].float().contiguous(), v[:, :, 0].contiguous(), S, Z)


def test_wrong_output_shapes_are_rejected():
    q, k, v = _qkv()
    short = torch.empty(1, 2, 63, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        kata.chunked_fwd(q, k, v, C=64, out=short)
    with pytest.raises(ValueError):
        kata.quadratic_fwd(q, k, v, out=short)
    with pytest.raises(TypeError):
        kata.chunked_fwd(q, k, v, C=64, out=torch.empty(1, 2, 64, 64, dtype=torch.float16, device="cuda"))
    cu = torch.tensor([0, 30, 64], dtype=torch.int32, device="cuda")
    qp, kp, vp = (x[0].transpose(0, 1).contiguous() for x in (q, k, v))  # [total, H, *]
    with pytest.raises(ValueError):
        kata.chunked_fwd_varlen(qp, kp, vp, cu, 34, out=torch.empty(60, 2, 64, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        kata.quadratic_fwd_varlen(qp, kp, vp, cu, 34, out=torch.empty(64, 2, 32, dtype=torch.bfloat16, device="cuda"))
    # the right shapes still run
    o = kata.chunked_fwd(q, k, v, C=64, out=torch.empty(1, 2, 64, 64, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
