"""Python binding of libkata.so, the MI355X (gfx950) KATA causal linear-attention library.

Thin ctypes layer: it checks tensor placement, dtype and contiguity, allocates outputs
and workspaces with torch on the tensors' device, and passes raw device pointers and the
current HIP stream to the C ABI declared in include/kata.h. Every step of the computation
runs in the library's HIP kernels; there is no CPU path. If the library is missing the
calls raise.

The method: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric
Cones" (arXiv 2607.17419): o_t = psi(q_t)^T S_t / psi(q_t)^T Z_t with the rank-one lift
psi(u) = u_hat u_hat^T packed into n = p(p+1)/2 coordinates.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["KataError", "library_path", "load", "packed_dim", "feature_dim", "lift",
           "chunked_workspace_bytes", "chunked_workspace_bytes_family", "chunked_fwd", "quadratic_fwd", "decode_step",
           "SCAN_SEQUENTIAL", "SCAN_ASSOCIATIVE", "PASS_SUMMARIES", "PASS_SCAN", "PASS_SEGMENTS",
           "PASS_ALL", "FEATURES", "quadratic_bwd", "kata_attention", "order_dim", "chunked_fwd_varlen",
           "quadratic_fwd_varlen", "chunked_bwd", "chunked_bwd_varlen", "quadratic_bwd_varlen", "kata_attention_varlen",
           "STATE_BWD_MIN_T",
           "chunked_fwd_noalloc", "NOALLOC_SCRATCH_BYTES"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkata.so")
_lib = None

DTYPE_F32, DTYPE_BF16 = 0, 1
SCAN_SEQUENTIAL, SCAN_ASSOCIATIVE = 0, 1
PASS_SUMMARIES, PASS_SCAN, PASS_SEGMENTS, PASS_ALL = 1, 2, 4, 7
# PSD feature families: full map, KATA-Sigma g, KATA-M g (kata_feature_t)
FEATURES = {"full": 0, "sigma": 1, "block": 2}
_STATUS = {0: "KATA_OK", 1: "KATA_ERR_NULL", 2: "KATA_ERR_SHAPE", 3: "KATA_ERR_DTYPE",
           4: "KATA_ERR_UNSUPPORTED", 5: "KATA_ERR_ALIGN", 6: "KATA_ERR_ALIAS",
           7: "KATA_ERR_WORKSPACE", 8: "KATA_ERR_HIP", 9: "KATA_ERR_SCAN", 10: "KATA_ERR_PASS",
           11: "KATA_ERR_FEATURE", 12: "KATA_ERR_SCRATCH"}


class KataError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)}")


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libkata.so (raises if it has not been built) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.kata_packed_dim.argtypes, lib.kata_packed_dim.restype = [I], I64
    lib.kata_status_string.argtypes, lib.kata_status_string.restype = [I], ctypes.c_char_p
    lib.kata_lift.argtypes, lib.kata_lift.restype = [P, I, I64, I, P, I, P], I
    lib.kata_chunked_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.kata_chunked_workspace_bytes.restype = SZ
    lib.kata_chunked_fwd.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, I, P, SZ, P]
    lib.kata_chunked_fwd.restype = I
    lib.kata_chunked_fwd_noalloc.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, I, P]
    lib.kata_chunked_fwd_noalloc.restype = I
    lib.kata_chunked_fwd_passes.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, I, P, SZ, I, P]
    lib.kata_chunked_fwd_passes.restype = I
    lib.kata_chunked_fwd_state.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, I, P, SZ, P, P, P]
    lib.kata_chunked_fwd_state.restype = I
    lib.kata_quadratic_fwd.argtypes = [P, P, P, I, P, I, I, I, I, I, I, P]
    lib.kata_quadratic_fwd.restype = I
    lib.kata_decode_step.argtypes = [P, P, P, I, P, P, P, I, I, I, I, I, P]
    lib.kata_decode_step.restype = I
    lib.kata_feature_dim.argtypes, lib.kata_feature_dim.restype = [I, I, I], I64
    lib.kata_lift_family.argtypes, lib.kata_lift_family.restype = [P, I, I64, I, I, I, P, I, P], I
    lib.kata_chunked_workspace_bytes_family.argtypes = [I, I, I, I, I, I, I, I, I, I]
    lib.kata_chunked_workspace_bytes_family.restype = SZ
    lib.kata_chunked_fwd_family.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, I, I, I, P, SZ, P, P, P]
    lib.kata_chunked_fwd_family.restype = I
    lib.kata_chunked_fwd_ragged.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, I, I, I, P, P, SZ, P, P, P]
    lib.kata_chunked_fwd_ragged.restype = I
    lib.kata_chunked_fwd_varlen.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, I, I, I, I, P, P, SZ, P, P, P]
    lib.kata_chunked_fwd_varlen.restype = I
    lib.kata_quadratic_fwd_varlen.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, I, I, P, P]
    lib.kata_quadratic_fwd_varlen.restype = I
    lib.kata_order_dim.argtypes, lib.kata_order_dim.restype = [I, I], I64
    lib.kata_lift_order.argtypes, lib.kata_lift_order.restype = [P, I, I64, I, I, P, I, P], I
    lib.kata_quadratic_fwd_order.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, P]
    lib.kata_quadratic_fwd_order.restype = I
    lib.kata_chunked_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.kata_chunked_bwd_workspace_bytes.restype = SZ
    lib.kata_chunked_bwd.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, P, P, P, P, SZ, P]
    lib.kata_chunked_bwd.restype = I
    lib.kata_chunked_bwd_varlen_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.kata_chunked_bwd_varlen_workspace_bytes.restype = SZ
    lib.kata_chunked_bwd_varlen.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, P, P, P, P, P, SZ, P]
    lib.kata_chunked_bwd_varlen.restype = I
    lib.kata_quadratic_bwd_workspace_bytes.argtypes = [I, I, I]
    lib.kata_quadratic_bwd_workspace_bytes.restype = SZ
    lib.kata_quadratic_bwd.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, P, P, P, P, SZ, P]
    lib.kata_quadratic_bwd.restype = I
    lib.kata_quadratic_bwd_varlen_workspace_bytes.argtypes = [I, I, I]
    lib.kata_quadratic_bwd_varlen_workspace_bytes.restype = SZ
    lib.kata_quadratic_bwd_varlen.argtypes = [P, P, P, P, I, I, I, I, I, I, I, P, P, P, P, P, SZ, P]
    lib.kata_quadratic_bwd_varlen.restype = I
    lib.kata_quadratic_fwd_family.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, I, P]
    lib.kata_quadratic_fwd_family.restype = I
    lib.kata_decode_step_family.argtypes = [P, P, P, I, I, I, P, P, P, I, I, I, I, I, P]
    lib.kata_decode_step_family.restype = I
    _lib = lib
    return lib


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _dev(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda:
            raise ValueError("KATA tensors must be on a GPU device (no CPU path)")
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("KATA tensors must be contiguous")
    return dev


def _same_dtype(*ts: torch.Tensor) -> None:
    """The C calls take one input dtype for q, k and v (and grad_o): a mismatch would make a
    kernel read a tensor with the wrong element size."""
    for t in ts:
        if t.dtype != ts[0].dtype:
            raise TypeError("q, k and v must share one dtype (float32 or bfloat16)")
    _dt(ts[0])


def _out(out, shape, dtype, dev: torch.device) -> torch.Tensor:
    """A new output tensor, or the caller's after checking its shape and dtype (the C calls
    write shape's elements through the pointer)."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(shape)}")
    _dt(out)
    _dev(out)
    if out.device != dev:
        raise ValueError("out must be on the inputs' device")
    return out


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise KataError(status, where)


def packed_dim(p: int) -> int:
    return int(load().kata_packed_dim(p))


def _fam(family: str, g: int) -> int:
    if family not in FEATURES:
        raise ValueError(f"family must be one of {tuple(FEATURES)}")
    return FEATURES[family]


def feature_dim(p: int, family: str = "full", g: int = 1) -> int:
    """Packed feature width of a family: p(p+1)/2, m(m+1)/2 (Sigma g) or g m(m+1)/2 (M g)."""
    n = int(load().kata_feature_dim(p, _fam(family, g), g))
    if n < 0:
        raise ValueError(f"invalid feature family ({family}, g={g}) for p={p}")
    return n


def order_dim(p: int, r: int) -> int:
    """binom(p + 2r - 1, 2r): packed width of the even-order lift psi_2r."""
    n = int(load().kata_order_dim(p, r))
    if n < 0:
        raise ValueError(f"invalid order r={r} for p={p}")
    return n


def lift(u: torch.Tensor, out_dtype: torch.dtype | None = None, family: str = "full",
         g: int = 1, order: int = 1) -> torch.Tensor:
    """[..., p] -> [..., n]: packed psi(u_hat) (rank-one lift, after Eq. (8)), the family's map
    (reduced PSD families paragraph), or with order = r > 1 the even-order lift psi_2r."""
    lib = load()
    dev = _dev(u)
    p = u.shape[-1]
    rows = u.numel() // p if p else 0
    if order != 1:
        if family != "full":
            raise ValueError("higher orders apply to the full map")
        out = torch.empty(u.shape[:-1] + (order_dim(p, order),), dtype=out_dtype or u.dtype, device=dev)
        with torch.cuda.device(dev):
            _check(lib.kata_lift_order(u.data_ptr(), _dt(u), rows, p, order, out.data_ptr(), _dt(out),
                                       _stream(dev)), "kata_lift_order")
        return out
    out = torch.empty(u.shape[:-1] + (feature_dim(p, family, g),), dtype=out_dtype or u.dtype, device=dev)
    with torch.cuda.device(dev):
        if family == "full":
            _check(lib.kata_lift(u.data_ptr(), _dt(u), rows, p, out.data_ptr(), _dt(out),
                                 _stream(dev)), "kata_lift")
        else:
            _check(lib.kata_lift_family(u.data_ptr(), _dt(u), rows, p, _fam(family, g), g, out.data_ptr(),
                                        _dt(out), _stream(dev)), "kata_lift_family")
    return out


def chunked_workspace_bytes(B, H, T, p, dv, C, scan=SCAN_ASSOCIATIVE, in_dtype=torch.bfloat16):
    return int(load().kata_chunked_workspace_bytes(B, H, T, p, dv, C, int(scan),
                                                   DTYPE_BF16 if in_dtype == torch.bfloat16 else DTYPE_F32))


def chunked_fwd_varlen(q, k, v, cu_seqlens, max_len: int, C: int = 64, scan="associative", out_dtype=None,
                       out=None, workspace=None, return_state: bool = False, family: str = "full", g: int = 1):
    """Chunked forward over B sequences packed without padding (token-major, as in varlen
    attention): q, k [total, H, p]; v [total, H, dv] -> o [total, H, dv]. cu_seqlens: int32
    device tensor [B + 1] of sequence offsets (0 first, non-decreasing); max_len >= every
    length. return_state: also return the state after each sequence's last token,
    (o, S [B,H,n,dv], Z [B,H,n]) in float32. Rows outside every sequence are not written."""
    lib = load()
    dev = _dev(q, k, v)
    total, H, p = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:2] != q.shape[:2]:
        raise ValueError("shape mismatch between q, k and v")
    _same_dtype(q, k, v)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d int32 tensor [B + 1]")
    _dev(cu_seqlens, q)
    B = cu_seqlens.numel() - 1
    sc = _scan_code(scan)
    out = _out(out, (total, H, dv), out_dtype or v.dtype, dev)
    fam = _fam(family, g)
    need = int(lib.kata_chunked_workspace_bytes_family(B, H, max_len, p, dv, C, sc, _dt(q), fam, g))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    S = Z = None
    if return_state:
        n = feature_dim(p, family, g)
        S = torch.empty((B, H, n, dv), dtype=torch.float32, device=dev)
        Z = torch.empty((B, H, n), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check(lib.kata_chunked_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q), out.data_ptr(),
                                           _dt(out), B, H, total, max_len, p, dv, C, sc, fam, g,
                                           cu_seqlens.data_ptr(), ws_ptr, ws_bytes,
                                           S.data_ptr() if S is not None else None,
                                           Z.data_ptr() if Z is not None else None, _stream(dev)),
               "kata_chunked_fwd_varlen")
    return (out, S, Z) if return_state else out


def quadratic_fwd_varlen(q, k, v, cu_seqlens, max_len: int, out_dtype=None, out=None, family: str = "full",
                         g: int = 1):
    """Flash-style quadratic forward over B sequences packed without padding: q, k
    [total, H, p]; v [total, H, dv] -> o [total, H, dv], each sequence causal over its own
    tokens. cu_seqlens: int32 device tensor [B + 1] of sequence offsets (0 first,
    non-decreasing); max_len >= every length. The shapes of quadratic_fwd (bf16 or fp32;
    family, g as there): bf16 MFMA kernels where they exist, else the VALU kernels. Rows
    outside every sequence are not written."""
    lib = load()
    dev = _dev(q, k, v)
    total, H, p = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:2] != q.shape[:2]:
        raise ValueError("shape mismatch between q, k and v")
    _same_dtype(q, k, v)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d int32 tensor [B + 1]")
    _dev(cu_seqlens, q)
    B = cu_seqlens.numel() - 1
    out = _out(out, (total, H, dv), out_dtype or v.dtype, dev)
    with torch.cuda.device(dev):
        _check(lib.kata_quadratic_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q), out.data_ptr(),
                                             _dt(out), B, H, total, max_len, p, dv, _fam(family, g), g,
                                             cu_seqlens.data_ptr(),
                                             _stream(dev)), "kata_quadratic_fwd_varlen")
    return out


def chunked_workspace_bytes_family(B, H, T, p, dv, C, scan=SCAN_ASSOCIATIVE, in_dtype=torch.bfloat16,
                                   fam: str = "full", g: int = 1):
    return int(load().kata_chunked_workspace_bytes_family(
        B, H, T, p, dv, C, int(scan), DTYPE_BF16 if in_dtype == torch.bfloat16 else DTYPE_F32, _fam(fam, g), g))


def _scan_code(scan) -> int:
    if isinstance(scan, str):
        return {"sequential": SCAN_SEQUENTIAL, "associative": SCAN_ASSOCIATIVE}[scan]
    return int(scan)


NOALLOC_SCRATCH_BYTES = 64 << 20  # KATA_NOALLOC_SCRATCH_BYTES


def chunked_fwd_noalloc(q, k, v, out, C: int = 64, scan="associative"):
    """kata_chunked_fwd_noalloc: the chunked forward with the library's fixed device scratch as
    its workspace (nothing is allocated by the call). The caller passes the output tensor
    out [B,H,T,dv] (float32 or bfloat16). Calls overlapping on one GPU race on the scratch."""
    lib = load()
    dev = _dev(q, k, v, out)
    B, H, T, p = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or tuple(out.shape) != (B, H, T, dv):
        raise ValueError("shape mismatch between q, k, v and out")
    _same_dtype(q, k, v)
    _dt(out)
    with torch.cuda.device(dev):
        _check(lib.kata_chunked_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q),
                                            out.data_ptr(), _dt(out), B, H, T, p, dv, C, _scan_code(scan),
                                            _stream(dev)), "kata_chunked_fwd_noalloc")
    return out


def chunked_fwd(q, k, v, C: int = 64, scan="associative", out_dtype=None, out=None,
                workspace=None, passes: int = PASS_ALL, return_state: bool = False,
                family: str = "full", g: int = 1, lengths=None):
    """Exact O(T) chunked-state forward. q, k: [B,H,T,p]; v: [B,H,T,dv] -> o [B,H,T,dv].
    passes: subset of the passes to enqueue (PASS_SUMMARIES | PASS_SCAN | PASS_SEGMENTS);
    running them in separate calls needs the same out and workspace each time.
    return_state: also return the state after the last token, (o, S [B,H,n,dv], Z [B,H,n])
    in float32, the layout decode_step continues from (all passes only).
    family, g: the PSD feature family ("full", "sigma" = KATA-Sigma g, "block" = KATA-M g);
    the reduced families run all passes in one call.
    lengths: optional int32 device tensor [B]; sequence b then uses its first lengths[b]
    tokens (padded layout), output rows past it are not written, and the returned state is
    the one after its last token."""
    lib = load()
    dev = _dev(q, k, v)
    B, H, T, p = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("shape mismatch between q, k and v")
    _same_dtype(q, k, v)
    sc = _scan_code(scan)
    out = _out(out, (B, H, T, dv), out_dtype or v.dtype, dev)
    fam = _fam(family, g)
    need = int(lib.kata_chunked_workspace_bytes_family(B, H, T, p, dv, C, sc, _dt(q), fam, g))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if lengths is not None:
        if passes != PASS_ALL:
            raise ValueError("ragged sequences run all passes in one call")
        if lengths.dtype != torch.int32 or tuple(lengths.shape) != (B,):
            raise ValueError("lengths must be an int32 tensor of shape [B]")
        _dev(lengths, q)
        S = Z = None
        if return_state:
            n = feature_dim(p, family, g)
            S = torch.empty((B, H, n, dv), dtype=torch.float32, device=dev)
            Z = torch.empty((B, H, n), dtype=torch.float32, device=dev)
        with torch.cuda.device(dev):
            _check(lib.kata_chunked_fwd_ragged(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q),
                                               out.data_ptr(), _dt(out), B, H, T, p, dv, C, sc, fam, g,
                                               lengths.data_ptr(), ws_ptr, ws_bytes,
                                               S.data_ptr() if S is not None else None,
                                               Z.data_ptr() if Z is not None else None, _stream(dev)),
                   "kata_chunked_fwd_ragged")
        return (out, S, Z) if return_state else out
    if family != "full":
        if passes != PASS_ALL:
            raise ValueError("the reduced families run all passes in one call")
        S = Z = None
        if return_state:
            n = feature_dim(p, family, g)
            S = torch.empty((B, H, n, dv), dtype=torch.float32, device=dev)
            Z = torch.empty((B, H, n), dtype=torch.float32, device=dev)
        with torch.cuda.device(dev):
            _check(lib.kata_chunked_fwd_family(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q),
                                               out.data_ptr(), _dt(out), B, H, T, p, dv, C, sc, fam, g,
                                               ws_ptr, ws_bytes, S.data_ptr() if S is not None else None,
                                               Z.data_ptr() if Z is not None else None, _stream(dev)),
                   "kata_chunked_fwd_family")
        return (out, S, Z) if return_state else out
    if return_state:
        if passes != PASS_ALL:
            raise ValueError("return_state needs all passes in one call")
        n = packed_dim(p)
        S = torch.empty((B, H, n, dv), dtype=torch.float32, device=dev)
        Z = torch.empty((B, H, n), dtype=torch.float32, device=dev)
        with torch.cuda.device(dev):
            _check(lib.kata_chunked_fwd_state(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q),
                                              out.data_ptr(), _dt(out), B, H, T, p, dv, C, sc,
                                              ws_ptr, ws_bytes, S.data_ptr(), Z.data_ptr(),
                                              _stream(dev)), "kata_chunked_fwd_state")
        return out, S, Z
    with torch.cuda.device(dev):
        if passes == PASS_ALL:
            _check(lib.kata_chunked_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q),
                                        out.data_ptr(), _dt(out), B, H, T, p, dv, C, sc, ws_ptr,
                                        ws_bytes, _stream(dev)), "kata_chunked_fwd")
        else:
            _check(lib.kata_chunked_fwd_passes(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q),
                                               out.data_ptr(), _dt(out), B, H, T, p, dv, C, sc,
                                               ws_ptr, ws_bytes, int(passes), _stream(dev)),
                   "kata_chunked_fwd_passes")
    return out


def quadratic_fwd(q, k, v, out_dtype=None, out=None, family: str = "full", g: int = 1, order: int = 1):
    """Flash-style quadratic forward (no state). q, k: [B,H,T,p]; v: [B,H,T,dv].
    family, g: the PSD feature family of the weights (see chunked_fwd); order = r > 1:
    weights (q_hat . k_hat)^(2r) of the even-order lift psi_2r (full map)."""
    lib = load()
    dev = _dev(q, k, v)
    B, H, T, p = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("shape mismatch between q, k and v")
    _same_dtype(q, k, v)
    out = _out(out, (B, H, T, dv), out_dtype or v.dtype, dev)
    with torch.cuda.device(dev):
        if order != 1:
            if family != "full":
                raise ValueError("higher orders apply to the full map")
            _check(lib.kata_quadratic_fwd_order(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q),
                                                out.data_ptr(), _dt(out), B, H, T, p, dv, order, _stream(dev)),
                   "kata_quadratic_fwd_order")
        elif family == "full":
            _check(lib.kata_quadratic_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q),
                                          out.data_ptr(), _dt(out), B, H, T, p, dv, _stream(dev)),
                   "kata_quadratic_fwd")
        else:
            _check(lib.kata_quadratic_fwd_family(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q),
                                                 out.data_ptr(), _dt(out), B, H, T, p, dv,
                                                 _fam(family, g), g, _stream(dev)),
                   "kata_quadratic_fwd_family")
    return out


def decode_step(q, k, v, S, Z, out_dtype=None, out=None, family: str = "full", g: int = 1):
    """One recurrent step: S += psi(k) v^T, Z += psi(k), o = psi(q)^T S / psi(q)^T Z.
    q, k: [N,H,p]; v: [N,H,dv]; S: [N,H,n,dv] fp32 and Z: [N,H,n] fp32 updated in place;
    family, g: the PSD feature family of psi (n = feature_dim(p, family, g))."""
    lib = load()
    dev = _dev(q, k, v, S, Z)
    N, H, p = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("shape mismatch between q, k and v")
    _same_dtype(q, k, v)
    n = feature_dim(p, family, g)
    if S.dtype != torch.float32 or Z.dtype != torch.float32:
        raise TypeError("S and Z must be float32")
    if tuple(S.shape) != (N, H, n, dv) or tuple(Z.shape) != (N, H, n):
        raise ValueError("state shape mismatch")
    out = _out(out, (N, H, dv), out_dtype or v.dtype, dev)
    with torch.cuda.device(dev):
        if family == "full":
            _check(lib.kata_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q),
                                        S.data_ptr(), Z.data_ptr(), out.data_ptr(), _dt(out), N, H,
                                        p, dv, _stream(dev)), "kata_decode_step")
        else:
            _check(lib.kata_decode_step_family(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q),
                                               _fam(family, g), g, S.data_ptr(), Z.data_ptr(),
                                               out.data_ptr(), _dt(out), N, H, p, dv, _stream(dev)),
                   "kata_decode_step_family")
    return out


def quadratic_bwd(q, k, v, grad_o, family: str = "full", g: int = 1):
    """Gradients (dq, dk, dv) in float32 of the causal forward with dL/do = grad_o.
    q, k: [B,H,T,p]; v, grad_o: [B,H,T,dv], in the dtype of q (float32 or bfloat16)."""
    lib = load()
    dev = _dev(q, k, v, grad_o)
    B, H, T, p = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or grad_o.shape != v.shape:
        raise ValueError("shape mismatch between q, k, v and grad_o")
    if not (k.dtype == v.dtype == grad_o.dtype == q.dtype):
        raise TypeError("q, k, v and grad_o must share one dtype")
    dq = torch.empty((B, H, T, p), dtype=torch.float32, device=dev)
    dk = torch.empty_like(dq)
    dvv = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    need = int(lib.kata_quadratic_bwd_workspace_bytes(B, H, T))
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(lib.kata_quadratic_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), grad_o.data_ptr(), _dt(q),
                                      B, H, T, p, dv, _fam(family, g), g, dq.data_ptr(), dk.data_ptr(),
                                      dvv.data_ptr(), ws.data_ptr(), need, _stream(dev)), "kata_quadratic_bwd")
    return dq, dk, dvv


def quadratic_bwd_varlen(q, k, v, grad_o, cu_seqlens, max_len: int):
    """Flash-style gradients (dq, dk, dv), float32, of the full-map forward over B sequences
    packed without padding (the layout of quadratic_fwd_varlen): q, k [total, H, p]; v,
    grad_o [total, H, dv], one dtype (bf16 or fp32), p and dv <= 64: bf16 MFMA kernels for
    p, dv in {32, 64}, else the VALU kernels. Rows outside every sequence come back as
    zeros."""
    lib = load()
    dev = _dev(q, k, v, grad_o)
    total, H, p = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:2] != q.shape[:2] or grad_o.shape != v.shape:
        raise ValueError("shape mismatch between q, k, v and grad_o")
    if not (q.dtype == k.dtype == v.dtype == grad_o.dtype):
        raise TypeError("q, k, v and grad_o must share one dtype")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d int32 tensor [B + 1]")
    _dev(cu_seqlens, q)
    B = cu_seqlens.numel() - 1
    dq = torch.zeros((total, H, p), dtype=torch.float32, device=dev)
    dk = torch.zeros_like(dq)
    dvv = torch.zeros((total, H, dv), dtype=torch.float32, device=dev)
    need = int(lib.kata_quadratic_bwd_varlen_workspace_bytes(B, H, total))
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(lib.kata_quadratic_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), grad_o.data_ptr(), _dt(q), B,
                                             H, total, max_len, p, dv, cu_seqlens.data_ptr(), dq.data_ptr(),
                                             dk.data_ptr(), dvv.data_ptr(), ws.data_ptr(), need, _stream(dev)),
               "kata_quadratic_bwd_varlen")
    return dq, dk, dvv


def chunked_bwd(q, k, v, grad_o, C: int = 32, scan="associative", workspace=None):
    """O(T) gradients (dq, dk, dv) of the causal full-map forward, float32, from the state form:
    bf16 MFMA kernels for bf16 inputs with p in {16, 32} and dv in {32, 64}, fp32 VALU kernels
    (chunk C) otherwise. q, k: [B,H,T,p]; v, grad_o: [B,H,T,dv], one dtype."""
    lib = load()
    dev = _dev(q, k, v, grad_o)
    B, H, T, p = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or grad_o.shape != v.shape:
        raise ValueError("shape mismatch between q, k, v and grad_o")
    if not (q.dtype == k.dtype == v.dtype == grad_o.dtype):
        raise TypeError("q, k, v and grad_o must share one dtype")
    sc = _scan_code(scan)
    dq = torch.empty((B, H, T, p), dtype=torch.float32, device=dev)
    dk = torch.empty_like(dq)
    dvv = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    need = int(lib.kata_chunked_bwd_workspace_bytes(B, H, T, p, dv, C, sc))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(lib.kata_chunked_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), grad_o.data_ptr(), _dt(q), B, H, T, p,
                                    dv, C, sc, dq.data_ptr(), dk.data_ptr(), dvv.data_ptr(), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(dev)),
               "kata_chunked_bwd")
    return dq, dk, dvv


# From this length on, bf16 gradients of the full map (p in {16, 32}, dv in {32, 64}) come from
# the O(T) state form: it costs about 1.7 ns per head-token against 1.3 ps per causal pair for
# the flash form on one MI355X, which puts the crossover near T = 2600.
STATE_BWD_MIN_T = 3072


def chunked_bwd_varlen(q, k, v, grad_o, cu_seqlens, max_len: int, scan="associative", workspace=None):
    """O(T) gradients (dq, dk, dv), float32, of the forward over B sequences packed without
    padding (the layout of chunked_fwd_varlen): q, k [total, H, p]; v, grad_o [total, H, dv],
    one dtype: the bf16 MFMA state form for bf16 with p in {16, 32}, dv in {32, 64}, else the
    fp32 VALU kernels (p, dv <= 64, the largest chunk of 64, 32, 16 that fits LDS). Rows
    outside every sequence come back as zeros."""
    lib = load()
    dev = _dev(q, k, v, grad_o)
    total, H, p = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:2] != q.shape[:2] or grad_o.shape != v.shape:
        raise ValueError("shape mismatch between q, k, v and grad_o")
    if not (q.dtype == k.dtype == v.dtype == grad_o.dtype):
        raise TypeError("q, k, v and grad_o must share one dtype")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d int32 tensor [B + 1]")
    _dev(cu_seqlens, q)
    B = cu_seqlens.numel() - 1
    sc = _scan_code(scan)
    dq = torch.zeros((total, H, p), dtype=torch.float32, device=dev)
    dk = torch.zeros_like(dq)
    dvv = torch.zeros((total, H, dv), dtype=torch.float32, device=dev)
    need = int(lib.kata_chunked_bwd_varlen_workspace_bytes(B, H, total, max(max_len, 1), p, dv, sc))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(lib.kata_chunked_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), grad_o.data_ptr(), _dt(q), B, H,
                                           total, max_len, p, dv, sc, cu_seqlens.data_ptr(), dq.data_ptr(),
                                           dk.data_ptr(), dvv.data_ptr(), workspace.data_ptr(),
                                           workspace.numel() * workspace.element_size(), _stream(dev)),
               "kata_chunked_bwd_varlen")
    return dq, dk, dvv


class _KataAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, C, family, g):
        ctx.save_for_backward(q, k, v)
        ctx.family, ctx.g = family, g
        try:  # the O(T) chunked form where its kernels cover the shape, else the quadratic form
            return chunked_fwd(q, k, v, C=C, family=family, g=g)
        except KataError as e:
            if e.status != 4:  # KATA_ERR_UNSUPPORTED
                raise
        return quadratic_fwd(q, k, v, family=family, g=g)

    @staticmethod
    def backward(ctx, grad_o):
        q, k, v = ctx.saved_tensors
        go = grad_o.contiguous().to(q.dtype)
        if (ctx.family == "full" and q.dtype == torch.bfloat16 and q.shape[-1] in (16, 32)
                and v.shape[-1] in (32, 64) and q.shape[2] >= STATE_BWD_MIN_T):
            dq, dk, dvv = chunked_bwd(q, k, v, go, C=32)  # O(T): the bf16 MFMA state form
        else:
            dq, dk, dvv = quadratic_bwd(q, k, v, go, family=ctx.family, g=ctx.g)
        return dq.to(q.dtype), dk.to(k.dtype), dvv.to(v.dtype), None, None, None


class _KataAttentionVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, max_len, C):
        ctx.save_for_backward(q, k, v, cu_seqlens)
        ctx.max_len = max_len
        try:  # the O(T) chunked form where its kernels cover the shape, else the quadratic form
            return chunked_fwd_varlen(q, k, v, cu_seqlens, max_len, C=C)
        except KataError as e:
            if e.status != 4:  # KATA_ERR_UNSUPPORTED
                raise
        return quadratic_fwd_varlen(q, k, v, cu_seqlens, max_len)

    @staticmethod
    def backward(ctx, grad_o):
        q, k, v, cu = ctx.saved_tensors
        go = grad_o.contiguous().to(q.dtype)
        p, dv = q.shape[-1], v.shape[-1]
        state_form = q.dtype == torch.bfloat16 and p in (16, 32) and dv in (32, 64)
        if state_form and not (ctx.max_len < STATE_BWD_MIN_T and p == 32):
            dq, dk, dvv = chunked_bwd_varlen(q, k, v, go, cu, ctx.max_len)  # O(T): bf16 MFMA
        else:  # flash style: bf16 MFMA for p, dv in {32, 64}, else the VALU kernels
            dq, dk, dvv = quadratic_bwd_varlen(q, k, v, go, cu, ctx.max_len)
        return dq.to(q.dtype), dk.to(k.dtype), dvv.to(v.dtype), None, None, None


def kata_attention_varlen(q, k, v, cu_seqlens, max_len: int, C: int = 64):
    """Differentiable causal KATA attention (full map) over B sequences packed without
    padding (the layout of chunked_fwd_varlen: q, k [total, H, p]; v [total, H, dv];
    cu_seqlens int32 [B + 1]), bf16 or fp32 inputs. Forward: the packed chunked form, or the
    packed quadratic form where the chunked kernels do not cover the shape. Backward: the O(T)
    bf16 MFMA state form for bf16 with p in {16, 32} and dv in {32, 64} (except p = 32 with
    max_len < STATE_BWD_MIN_T), else the packed flash-style form (bf16 MFMA for p, dv in
    {32, 64}, else the VALU kernels, p, dv <= 64). Rows outside every sequence get zero
    gradients."""
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("kata_attention_varlen takes q, k, v of one dtype, bf16 or float32")
    return _KataAttentionVarlen.apply(q, k, v, cu_seqlens, max_len, C)


def kata_attention(q, k, v, C: int = 64, family: str = "full", g: int = 1):
    """Differentiable causal KATA attention: the chunked forward (quadratic form where the
    chunked kernels do not cover the shape); gradients from kata_chunked_bwd's bf16 MFMA
    state form for long bf16 sequences (T >= STATE_BWD_MIN_T, full map, p in {16, 32}, dv in
    {32, 64}), else from kata_quadratic_bwd."""
    return _KataAttention.apply(q, k, v, C, family, g)

