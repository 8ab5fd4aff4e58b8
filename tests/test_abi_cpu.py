"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every entry
point declared in include/kata.h, and validates arguments before any HIP call.

Only validation paths are exercised: every call below returns an error (or is a zero-size
no-op) before the library touches the device; the fake pointers are never dereferenced.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import kernelized_linear_attention_normalize_amd as kata
from kernelized_linear_attention_normalize_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
F32, BF16 = 0, 1
SEQ, ASSOC = 0, 1
OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_ALIAS, E_WS, E_HIP, E_SCAN, E_PASS, E_FEAT, E_SCRATCH = range(13)
A = 0x7F0000000000  # fake, 16-byte aligned device addresses (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kata.library_path()):
        build_lib.build()
    return kata.load()


def _declared_functions():
    txt = open(os.path.join(ROOT, "include", "kata.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(kata_[a-z_0-9]+)\s*\(", txt)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) >= {"kata_lift", "kata_chunked_fwd", "kata_quadratic_fwd", "kata_decode_step",
                          "kata_packed_dim", "kata_status_string", "kata_chunked_workspace_bytes"}
    for nm in names:
        assert hasattr(lib, nm), nm


def test_no_unresolved_library_symbols():
    """Every kata symbol the library references is defined in it (a template declared in one
    translation unit and instantiated in another under a different signature would only
    fail when the loader binds it)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", kata.library_path()], capture_output=True, text=True,
                         check=True).stdout
    assert "kata" not in out, [l for l in out.splitlines() if "kata" in l]


def test_packed_dim_and_status_strings(lib):
    assert lib.kata_packed_dim(32) == 528 and lib.kata_packed_dim(64) == 2080
    assert lib.kata_packed_dim(0) == -1
    for s in range(13):
        assert lib.kata_status_string(s).startswith(b"KATA_")


def _chunked(lib, q=A, k=A + 4096, v=A + 8192, in_dt=BF16, o=A + (1 << 30), o_dt=BF16, B=1, H=1, T=128,
             p=32, dv=64, C=64, scan=SEQ, ws=None, wsb=0):
    return lib.kata_chunked_fwd(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, C, scan, ws, wsb, None)


def test_chunked_validation(lib):
    assert _chunked(lib, in_dt=7) == E_DTYPE
    assert _chunked(lib, o_dt=-1) == E_DTYPE
    assert _chunked(lib, scan=5) == E_SCAN
    assert _chunked(lib, T=-1) == E_SHAPE
    assert _chunked(lib, C=0) == E_SHAPE
    assert _chunked(lib, p=0) == E_SHAPE
    assert _chunked(lib, T=0, q=None, k=None, v=None, o=None) == OK       # zero-size no-op
    assert _chunked(lib, B=0) == OK
    assert _chunked(lib, q=None) == E_NULL
    assert _chunked(lib, o=None) == E_NULL
    assert _chunked(lib, k=A + 4) == E_ALIGN
    assert _chunked(lib, p=24) == E_UNSUP
    assert _chunked(lib, p=64) == E_UNSUP
    assert _chunked(lib, dv=48) == E_UNSUP
    assert _chunked(lib, C=16) == E_UNSUP
    assert _chunked(lib, o=A + 4096) == E_ALIAS                          # o overlaps k
    # associative mode needs the workspace
    need = lib.kata_chunked_workspace_bytes(1, 16, 131072, 32, 64, 64, ASSOC, BF16)
    assert need > 0
    kw = dict(B=1, H=16, T=131072, scan=ASSOC, o=A + (1 << 34))
    assert _chunked(lib, **kw) == E_WS
    assert _chunked(lib, ws=A + (1 << 36), wsb=need - 1, **kw) == E_WS
    assert _chunked(lib, ws=A + (1 << 36) + 8, wsb=need, **kw) == E_ALIGN
    assert _chunked(lib, ws=A + (1 << 34), wsb=need, **kw) == E_ALIAS    # workspace overlaps o
    # fp32 inputs are supported on the whole advertised set (p = 32, dv = 64 in two
    # value-column parts): no shape of it is rejected as unsupported
    for C in (32, 64, 128):
        assert lib.kata_chunked_workspace_bytes(1, 16, 131072, 32, 64, C, ASSOC, F32) > 0


def test_chunked_passes_validation(lib):
    def passes(mask, **kw):
        a = dict(q=A, k=A + 4096, v=A + 8192, in_dt=BF16, o=A + (1 << 30), o_dt=BF16, B=1, H=1, T=128,
                 p=32, dv=64, C=64, scan=SEQ, ws=None, wsb=0)
        a.update(kw)
        return lib.kata_chunked_fwd_passes(a["q"], a["k"], a["v"], a["in_dt"], a["o"], a["o_dt"], a["B"],
                                           a["H"], a["T"], a["p"], a["dv"], a["C"], a["scan"], a["ws"],
                                           a["wsb"], mask, None)
    for bad in (0, 8, -1, 15):
        assert passes(bad) == E_PASS
    assert passes(7, scan=5) == E_SCAN           # shared validation, checked in the same order
    assert passes(4, in_dt=9) == E_DTYPE
    assert passes(1, q=None) == E_NULL
    kw = dict(B=1, H=16, T=131072, scan=ASSOC, o=A + (1 << 34))
    assert passes(2, **kw) == E_WS                # every pass needs the workspace of its plan


def test_chunked_state_validation(lib):
    """kata_chunked_fwd_state: the checks of kata_chunked_fwd plus those of the state outputs."""
    def st(S=A + (1 << 40), Z=A + (1 << 41), **kw):
        a = dict(q=A, k=A + 4096, v=A + 8192, in_dt=BF16, o=A + (1 << 30), o_dt=BF16, B=1, H=1, T=128,
                 p=32, dv=64, C=64, scan=SEQ, ws=None, wsb=0)
        a.update(kw)
        return lib.kata_chunked_fwd_state(a["q"], a["k"], a["v"], a["in_dt"], a["o"], a["o_dt"], a["B"],
                                          a["H"], a["T"], a["p"], a["dv"], a["C"], a["scan"], a["ws"],
                                          a["wsb"], S, Z, None)
    assert st(in_dt=7) == E_DTYPE
    assert st(scan=3) == E_SCAN
    assert st(B=0, S=None, Z=None) == OK             # no sequences: nothing to write
    assert st(S=None) == E_NULL
    assert st(Z=None) == E_NULL
    assert st(p=64) == E_UNSUP
    assert st(S=A + (1 << 40) + 4) == E_ALIGN
    n = lib.kata_packed_dim(32)
    assert st(Z=A + (1 << 40) + n * 64 * 4 - 64) == E_ALIAS      # Z inside S
    assert st(S=A + 4096) == E_ALIAS                             # S over k
    assert st(Z=A + (1 << 30)) == E_ALIAS                        # Z over o
    assert st(q=None) == E_NULL
    need = lib.kata_chunked_workspace_bytes(1, 16, 131072, 32, 64, 64, ASSOC, BF16)
    kw = dict(B=1, H=16, T=131072, scan=ASSOC, o=A + (1 << 34), ws=A + (1 << 36), wsb=need)
    assert st(S=A + (1 << 36) + 1024, **kw) == E_ALIAS           # S inside the workspace


def test_feature_families(lib):
    """kata_feature_dim matches the widths of the oracle; a bad (family, g) is
    KATA_ERR_FEATURE before anything else touches the device."""
    from oracle import kata_families as kf
    FULL, SIGMA, BLOCK = 0, 1, 2
    for p, fam, g in [(32, SIGMA, 2), (32, BLOCK, 2), (64, SIGMA, 2), (64, BLOCK, 4), (12, SIGMA, 3), (16, BLOCK, 16)]:
        assert lib.kata_feature_dim(p, fam, g) == kf.family_dim(p, ("full", "sigma", "block")[fam], g)
    assert lib.kata_feature_dim(32, FULL, 1) == 528
    assert lib.kata_feature_dim(32, FULL, 2) == -1 and lib.kata_feature_dim(32, SIGMA, 3) == -1
    assert lib.kata_feature_dim(32, 7, 1) == -1 and lib.kata_feature_dim(32, SIGMA, 0) == -1
    fwd = dict(q=A, k=A + 4096, v=A + 8192, o=A + (1 << 30))
    assert lib.kata_quadratic_fwd_family(fwd["q"], fwd["k"], fwd["v"], BF16, fwd["o"], BF16, 1, 1, 64, 32, 64,
                                         SIGMA, 3, None) == E_FEAT
    assert lib.kata_quadratic_fwd_family(fwd["q"], fwd["k"], fwd["v"], BF16, fwd["o"], BF16, 1, 1, 64, 128, 64,
                                         SIGMA, 2, None) == E_UNSUP
    assert lib.kata_decode_step_family(A, A + 4096, A + 8192, BF16, BLOCK, 5, A + (1 << 30), A + (1 << 31),
                                       A + (1 << 32), BF16, 2, 2, 32, 64, None) == E_FEAT
    assert lib.kata_lift_family(A, F32, 4, 32, FULL, 4, A + (1 << 30), F32, None) == E_FEAT

    def ch(fam=SIGMA, g=2, S=None, Z=None, **kw):
        a = dict(q=A, k=A + 4096, v=A + 8192, in_dt=BF16, o=A + (1 << 30), o_dt=BF16, B=1, H=1, T=128,
                 p=32, dv=64, C=64, scan=SEQ, ws=None, wsb=0)
        a.update(kw)
        return lib.kata_chunked_fwd_family(a["q"], a["k"], a["v"], a["in_dt"], a["o"], a["o_dt"], a["B"],
                                           a["H"], a["T"], a["p"], a["dv"], a["C"], a["scan"], fam, g,
                                           a["ws"], a["wsb"], S, Z, None)
    assert ch(g=5) == E_FEAT
    assert ch(S=A + (1 << 40)) == E_NULL               # S without Z
    assert ch(p=128, g=2) == E_UNSUP
    assert ch(C=16) == E_UNSUP
    # associative: the family's summaries need the workspace of their own width
    need = lib.kata_chunked_workspace_bytes_family(1, 4, 65536, 32, 64, 64, ASSOC, BF16, SIGMA, 2)
    assert need == 4 * 63 * (136 * 64 + 136) * 4     # 4 heads x 63 summaries (64 segments each)
    assert lib.kata_chunked_workspace_bytes_family(1, 4, 65536, 32, 64, 64, ASSOC, BF16, FULL, 1) == \
        lib.kata_chunked_workspace_bytes(1, 4, 65536, 32, 64, 64, ASSOC, BF16)
    assert ch(B=1, H=4, T=65536, scan=ASSOC, o=A + (1 << 34)) == E_WS


def test_sequence_length_limit(lib):
    """One sequence is addressed with 32-bit byte offsets: T * max(p, dv) * 4 < 2^31."""
    T = (1 << 31) // (64 * 4)  # exactly at the limit for dv = 64
    assert lib.kata_quadratic_fwd(A, A + 4096, A + 8192, BF16, A + (1 << 40), BF16, 1, 1, T, 32, 64, None) == E_SHAPE
    assert lib.kata_chunked_fwd(A, A + 4096, A + 8192, BF16, A + (1 << 40), BF16, 1, 1, T, 32, 64, 64, SEQ, None, 0,
                                None) == E_SHAPE


def test_varlen_validation(lib):
    """kata_chunked_fwd_varlen: argument errors come back before any device access."""
    FULL, SIGMA = 0, 1

    def vl(fam=FULL, g=1, cu=A + (1 << 36), S=None, Z=None, **kw):
        a = dict(q=A, k=A + 4096, v=A + 8192, in_dt=BF16, o=A + (1 << 30), o_dt=BF16, B=2, H=2, total=300,
                 max_len=200, p=32, dv=64, C=64, scan=SEQ, ws=None, wsb=0)
        a.update(kw)
        return lib.kata_chunked_fwd_varlen(a["q"], a["k"], a["v"], a["in_dt"], a["o"], a["o_dt"], a["B"],
                                           a["H"], a["total"], a["max_len"], a["p"], a["dv"], a["C"], a["scan"],
                                           fam, g, cu, a["ws"], a["wsb"], S, Z, None)
    assert vl(cu=None) == E_NULL
    assert vl(cu=A + (1 << 36) + 2) == E_ALIGN               # int32 array: 4-byte aligned
    assert vl(total=-1) == E_SHAPE and vl(max_len=-5) == E_SHAPE
    assert vl(S=A + (1 << 40)) == E_NULL                     # S without Z
    assert vl(g=3, fam=SIGMA) == E_FEAT
    assert vl(total=0) == OK and vl(max_len=0) == OK and vl(B=0) == OK   # nothing to do
    assert vl(dv=48) == E_UNSUP
    # Sigma 2 at p = 64, dv = 64 takes the packed layout on the two-block fp16 kernels: the
    # call gets as far as its (missing) segment-summary workspace
    assert vl(fam=SIGMA, g=2, p=64, dv=64, C=128, scan=ASSOC, max_len=200 * 64) == E_WS
    assert vl(fam=SIGMA, g=2, p=64, dv=48, C=128) == E_UNSUP
    # 32-bit offsets of one packed sequence: max_len * H * max(p, dv) * 4 must stay below 2^31
    assert vl(H=1024, max_len=1 << 14, total=1 << 14) == E_SHAPE
    # the associative scan's workspace is that of the padded call with T = max_len
    need = lib.kata_chunked_workspace_bytes(2, 2, 200 * 64, 32, 64, 64, ASSOC, BF16)
    assert need > 0 and vl(scan=ASSOC, max_len=200 * 64, total=300) == E_WS


def test_chunked_bwd_validation(lib):
    need = lib.kata_chunked_bwd_workspace_bytes(1, 2, 1000, 32, 64, 16, ASSOC)
    # covers the bf16 MFMA path: stats and two sets of segment summaries (8 segments of 128
    # tokens per head here, 34,816 floats each at p = 32, dv = 64)
    assert need >= (2 * 1000 * 2 + 2 * 2 * 7 * 34816) * 4
    # p = 32, dv = 64 at C = 32: the bf16 MFMA path runs it (any C in {16, 32, 64}), the fp32
    # VALU path does not (its LDS holds that state with C = 16 only)
    assert lib.kata_chunked_bwd_workspace_bytes(1, 2, 1000, 32, 64, 32, ASSOC) > 0
    assert lib.kata_chunked_bwd_workspace_bytes(1, 2, 1000, 32, 64, 8, ASSOC) == 0
    assert lib.kata_chunked_bwd_workspace_bytes(1, 2, 1000, 96, 64, 16, ASSOC) == 0
    assert lib.kata_chunked_bwd_workspace_bytes(1, 2, 1000, 48, 48, 32, ASSOC) == 0  # neither path
    args = lambda **kw: dict(dict(q=A, k=A + 4096, v=A + 8192, g=A + 12288, dt=BF16, B=1, H=2, T=1000, p=32, dv=64,
                                  C=16, scan=ASSOC, dq=A + (1 << 30), dk=A + (2 << 30), dvo=A + (3 << 30),
                                  ws=A + (4 << 30), wsb=need), **kw)

    def call(**kw):
        a = args(**kw)
        return lib.kata_chunked_bwd(a["q"], a["k"], a["v"], a["g"], a["dt"], a["B"], a["H"], a["T"], a["p"], a["dv"],
                                    a["C"], a["scan"], a["dq"], a["dk"], a["dvo"], a["ws"], a["wsb"], None)
    assert call(C=32, dt=F32) == E_UNSUP and call(C=8) == E_UNSUP
    assert call(scan=7) == E_SCAN and call(dt=5) == E_DTYPE
    assert call(dq=None) == E_NULL and call(wsb=need - 1) == E_WS and call(ws=None) == E_WS
    assert call(dk=A + (1 << 30)) == E_ALIAS                       # dk on top of dq
    assert call(T=0) == OK and call(B=0) == OK


def test_chunked_bwd_varlen_validation(lib):
    """kata_chunked_bwd_varlen: argument errors come back before any device access."""
    need = lib.kata_chunked_bwd_varlen_workspace_bytes(2, 2, 300, 200, 32, 64, ASSOC)
    assert need >= 300 * 2 * 2 * 4                                  # at least D_t, delta_t per row
    # p = dv = 64: no MFMA form, and the fp32 state does not fit LDS at any chunk
    assert lib.kata_chunked_bwd_varlen_workspace_bytes(2, 2, 300, 200, 64, 64, ASSOC) == 0
    assert lib.kata_chunked_bwd_varlen_workspace_bytes(2, 2, 300, 200, 32, 96, ASSOC) == 0
    # dv = 16: the fp32 VALU form (chunk 64), D_t and delta_t per row plus its summaries
    assert lib.kata_chunked_bwd_varlen_workspace_bytes(2, 2, 300, 200, 32, 16, ASSOC) >= 300 * 2 * 2 * 4
    # D_t, delta_t are kept for every row of the packed tensor, including rows past the last sequence
    assert lib.kata_chunked_bwd_varlen_workspace_bytes(2, 2, 3000, 200, 32, 64, ASSOC) > need

    def vb(cu=A + (1 << 36), **kw):
        a = dict(q=A, k=A + 4096, v=A + 8192, g=A + 12288, dt=BF16, B=2, H=2, total=300, max_len=200, p=32, dv=64,
                 scan=ASSOC, dq=A + (1 << 30), dk=A + (2 << 30), dvo=A + (3 << 30), ws=A + (4 << 30), wsb=need)
        a.update(kw)
        return lib.kata_chunked_bwd_varlen(a["q"], a["k"], a["v"], a["g"], a["dt"], a["B"], a["H"], a["total"],
                                           a["max_len"], a["p"], a["dv"], a["scan"], cu, a["dq"], a["dk"], a["dvo"],
                                           a["ws"], a["wsb"], None)
    assert vb(p=64) == E_UNSUP and vb(dv=96) == E_UNSUP and vb(p=80, dv=16) == E_UNSUP
    # fp32 inputs and other shapes take the VALU form: accepted up to the later checks
    assert vb(dt=F32, wsb=need - 1) == E_WS and vb(dt=F32, dq=None) == E_NULL
    assert vb(dv=48, dq=None) == E_NULL and vb(p=16, dv=16, ws=None) == E_WS
    assert vb(scan=7) == E_SCAN and vb(dt=5) == E_DTYPE
    assert vb(cu=None) == E_NULL and vb(cu=A + (1 << 36) + 2) == E_ALIGN
    assert vb(total=-1) == E_SHAPE and vb(max_len=-3) == E_SHAPE
    assert vb(wsb=need - 1) == E_WS and vb(ws=None) == E_WS and vb(dq=None) == E_NULL
    assert vb(dk=A + (1 << 30)) == E_ALIAS                        # dk on top of dq
    assert vb(H=1024, max_len=1 << 14, total=1 << 14) == E_SHAPE  # 32-bit offsets of one sequence
    assert vb(total=0) == OK and vb(max_len=0) == OK and vb(B=0) == OK


def test_quadratic_bwd_varlen_validation(lib):
    """kata_quadratic_bwd_varlen: argument errors come back before any device access."""
    need = lib.kata_quadratic_bwd_varlen_workspace_bytes(2, 2, 300)
    assert need == 300 * 2 * 2 * 4                                 # D_t, delta_t per packed row
    assert lib.kata_quadratic_bwd_varlen_workspace_bytes(2, 2, 0) == 0
    assert lib.kata_quadratic_bwd_varlen_workspace_bytes(0, 2, 300) == 0

    def qb(cu=A + (1 << 36), **kw):
        a = dict(q=A, k=A + 4096, v=A + 8192, g=A + 12288, dt=BF16, B=2, H=2, total=300, max_len=200, p=32, dv=64,
                 dq=A + (1 << 30), dk=A + (2 << 30), dvo=A + (3 << 30), ws=A + (4 << 30), wsb=need)
        a.update(kw)
        return lib.kata_quadratic_bwd_varlen(a["q"], a["k"], a["v"], a["g"], a["dt"], a["B"], a["H"], a["total"],
                                             a["max_len"], a["p"], a["dv"], cu, a["dq"], a["dk"], a["dvo"], a["ws"],
                                             a["wsb"], None)
    assert qb(p=65) == E_UNSUP and qb(dv=80) == E_UNSUP              # p, dv <= 64
    # fp32 and the non-MFMA shapes run the VALU kernels: accepted up to the later checks
    assert qb(dt=F32, wsb=need - 1) == E_WS and qb(p=16, dq=None) == E_NULL and qb(dv=48, ws=None) == E_WS
    assert qb(dt=5) == E_DTYPE
    assert qb(cu=None) == E_NULL and qb(cu=A + (1 << 36) + 2) == E_ALIGN
    assert qb(total=-1) == E_SHAPE and qb(max_len=-3) == E_SHAPE and qb(H=-1) == E_SHAPE
    assert qb(wsb=need - 1) == E_WS and qb(ws=None) == E_WS and qb(dq=None) == E_NULL and qb(v=A + 8) == E_ALIGN
    assert qb(dk=A + (1 << 30)) == E_ALIAS                        # dk on top of dq
    assert qb(dvo=A + 4096) == E_ALIAS                            # dv_out on top of k
    assert qb(H=1024, max_len=1 << 14, total=1 << 14) == E_SHAPE  # 32-bit offsets of one sequence
    assert qb(H=16, max_len=(1 << 19) - 256, total=100) == E_SHAPE  # a block past the end counts
    assert qb(total=0) == OK and qb(max_len=0) == OK and qb(B=0) == OK and qb(H=0) == OK


def test_quadratic_varlen_validation(lib):
    """kata_quadratic_fwd_varlen: argument errors come back before any device access."""
    def qv(cu=A + (1 << 36), **kw):
        a = dict(q=A, k=A + 4096, v=A + 8192, dt=BF16, o=A + (1 << 30), odt=BF16, B=2, H=2, total=300,
                 max_len=200, p=32, dv=64, fam=0, g=1)
        a.update(kw)
        return lib.kata_quadratic_fwd_varlen(a["q"], a["k"], a["v"], a["dt"], a["o"], a["odt"], a["B"], a["H"],
                                             a["total"], a["max_len"], a["p"], a["dv"], a["fam"], a["g"], cu, None)
    assert qv(p=48) == E_UNSUP and qv(dv=8) == E_UNSUP                  # full map: p, dv in {16, 32, 64}
    assert qv(fam=1, g=2, p=128) == E_UNSUP and qv(fam=2, g=4, p=64, dv=80) == E_UNSUP   # families: p, dv <= 64
    # fp32 inputs and the families without MFMA kernels run the VALU kernels: accepted up to
    # the later checks
    assert qv(dt=F32, q=None) == E_NULL and qv(fam=1, g=2, o=None) == E_NULL and qv(fam=2, g=4, p=64, v=A + 8) == E_ALIGN
    assert qv(fam=1, g=3) == E_FEAT and qv(fam=0, g=2) == E_FEAT and qv(fam=9) == E_FEAT
    assert qv(dt=5) == E_DTYPE and qv(odt=2) == E_DTYPE
    assert qv(cu=None) == E_NULL and qv(cu=A + (1 << 36) + 2) == E_ALIGN
    assert qv(total=-1) == E_SHAPE and qv(max_len=-3) == E_SHAPE and qv(H=-1) == E_SHAPE
    assert qv(q=None) == E_NULL and qv(o=None) == E_NULL and qv(v=A + 8) == E_ALIGN
    assert qv(o=A + 4096) == E_ALIAS                              # o on top of k
    assert qv(H=1024, max_len=1 << 14, total=1 << 14) == E_SHAPE  # 32-bit offsets of one sequence
    assert qv(H=16, max_len=(1 << 19) - 256, total=100) == E_SHAPE  # a query block past the end counts
    assert qv(total=0) == OK and qv(max_len=0) == OK and qv(B=0) == OK and qv(H=0) == OK


def test_higher_orders(lib):
    from oracle import kata_families as kf
    for p, r in [(4, 2), (16, 2), (3, 3), (8, 4), (64, 1)]:
        assert lib.kata_order_dim(p, r) == kf.order_dim(p, r)
    assert lib.kata_order_dim(8, 5) == -1 and lib.kata_order_dim(0, 2) == -1
    assert lib.kata_lift_order(A, F32, 4, 16, 5, A + (1 << 30), F32, None) == E_FEAT
    assert lib.kata_lift_order(A, F32, 4, 200, 2, A + (1 << 30), F32, None) == E_UNSUP
    assert lib.kata_quadratic_fwd_order(A, A + 4096, A + 8192, BF16, A + (1 << 30), BF16, 1, 1, 64, 32, 64, 0,
                                        None) == E_FEAT
    assert lib.kata_quadratic_fwd_order(A, A + 4096, A + 8192, BF16, A + (1 << 30), BF16, 1, 1, 64, 128, 64, 2,
                                        None) == E_UNSUP


def test_workspace_bytes(lib):
    # sequential mode and single-segment problems need none
    assert lib.kata_chunked_workspace_bytes(1, 16, 131072, 32, 64, 64, SEQ, BF16) == 0
    assert lib.kata_chunked_workspace_bytes(1, 1, 64, 32, 64, 64, ASSOC, BF16) == 0
    assert lib.kata_chunked_workspace_bytes(1, 1, 64, 33, 64, 64, ASSOC, BF16) == 0   # unsupported
    # long config (fp16-operand kernels): 16 heads x 16 segments, 15 summaries each of
    # 18 feature tiles x 2 value tiles x 1024 floats plus the 1024-float Gram tile
    assert lib.kata_chunked_workspace_bytes(1, 16, 131072, 32, 64, 64, ASSOC, BF16) == 16 * 15 * (18 * 2 * 1024 + 1024) * 4
    assert lib.kata_chunked_workspace_bytes(1, 16, 131072, 32, 64, 128, ASSOC, BF16) == 16 * 15 * (18 * 2 * 1024 + 1024) * 4
    # bf16 MFMA kernels of the other shapes: (33 tiles x dv/16 + 4) x 256 floats
    assert lib.kata_chunked_workspace_bytes(1, 16, 131072, 32, 32, 64, ASSOC, BF16) == 16 * 15 * (33 * 2 * 256 + 4 * 256) * 4
    # fp32 layout: n*dv + n floats per summary
    w = lib.kata_chunked_workspace_bytes(1, 1, 256, 16, 16, 32, ASSOC, F32)
    assert w == 7 * (136 * 16 + 136) * 4
    # fp32 at p = 32, dv = 64, C = 128: the state fits LDS only per half of the value columns,
    # so each summary is two parts of n*dv/2 + n floats
    assert lib.kata_chunked_workspace_bytes(1, 16, 131072, 32, 64, 128, ASSOC, F32) == 16 * 15 * 2 * (528 * 32 + 528) * 4
    assert lib.kata_chunked_workspace_bytes(1, 16, 131072, 32, 64, 32, ASSOC, F32) == 16 * 15 * (528 * 64 + 528) * 4


def test_quadratic_and_lift_and_decode_validation(lib):
    q = lambda **kw: lib.kata_quadratic_fwd(kw.get("q", A), A + 4096, A + 8192, kw.get("dt", BF16),
                                            kw.get("o", A + (1 << 30)), BF16, 1, 1, kw.get("T", 64),
                                            kw.get("p", 64), kw.get("dv", 64), None)
    assert q(dt=3) == E_DTYPE and q(T=-2) == E_SHAPE and q(T=0) == OK
    assert q(p=48) == E_UNSUP and q(q=None) == E_NULL and q(o=A + 8192) == E_ALIAS
    assert lib.kata_lift(A, F32, 10, 129, A + (1 << 30), F32, None) == E_UNSUP
    assert lib.kata_lift(A, F32, -1, 8, A + (1 << 30), F32, None) == E_SHAPE
    assert lib.kata_lift(A, F32, 0, 8, None, F32, None) == OK
    assert lib.kata_lift(A, F32, 10, 8, A + 64, F32, None) == E_ALIAS
    assert lib.kata_lift(A, 2, 10, 8, A + (1 << 30), F32, None) == E_DTYPE
    d = lambda **kw: lib.kata_decode_step(A, A + 4096, A + 8192, BF16, kw.get("S", A + (1 << 30)),
                                          kw.get("Z", A + (1 << 31)), kw.get("o", A + (1 << 32)), BF16,
                                          kw.get("N", 4), 2, kw.get("p", 32), kw.get("dv", 64), None)
    assert d(N=0) == OK and d(p=65) == E_UNSUP and d(dv=62) == E_UNSUP
    assert d(S=None) == E_NULL and d(Z=A + (1 << 30) + 16) == E_ALIAS
    assert d(o=A + 4096) == E_ALIAS and d(S=A + (1 << 30) + 4) == E_ALIGN


def _noalloc(lib, q=A, k=A + 4096, v=A + 8192, in_dt=BF16, o=A + (1 << 30), o_dt=BF16, B=1, H=1, T=128,
             p=32, dv=64, C=64, scan=ASSOC):
    return lib.kata_chunked_fwd_noalloc(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, C, scan, None)


def test_noalloc_validates_before_any_hip_call(lib):
    """kata_chunked_fwd_noalloc rejects bad arguments exactly as kata_chunked_fwd does, before
    it resolves its scratch array (no HIP call happens on these paths: there is no GPU here)."""
    assert _noalloc(lib, in_dt=7) == E_DTYPE
    assert _noalloc(lib, scan=5) == E_SCAN
    assert _noalloc(lib, T=-1) == E_SHAPE
    assert _noalloc(lib, q=None) == E_NULL
    assert _noalloc(lib, o=A + 8) == E_ALIGN
    assert _noalloc(lib, o=A) == E_ALIAS
    assert _noalloc(lib, p=48) == E_UNSUP
    assert _noalloc(lib, T=0, q=None, k=None, v=None, o=None) == OK


def test_noalloc_scratch_covers_every_supported_shape(lib):
    """The fixed scratch (64 MiB) holds the workspace of every supported shape: the segment
    plan keeps B*H*(segments-1) near one workgroup per compute unit, so the largest need is a
    few hundred summaries whatever B, H and T are."""
    cap = kata.NOALLOC_SCRATCH_BYTES
    worst = 0
    for p in (16, 32):
        for dv in (16, 32, 64):
            for C in (32, 64, 128):
                for dt in (F32, BF16):
                    for BH in (1, 2, 3, 5, 8, 16, 31, 64, 100, 128, 200, 255, 256, 257, 1000):
                        for T in (C + 1, 4096, 131072, 1 << 20):
                            need = lib.kata_chunked_workspace_bytes(1, BH, T, p, dv, C, ASSOC, dt)
                            worst = max(worst, need)
    assert 0 < worst <= cap, worst
