"""The C ABI on the CPU: libfa_amd.so loads, exports every function
include/fa.h declares, and rejects bad arguments with the documented status
before touching the GPU (no kernel is launched by these tests)."""
import ctypes

import pytest

import flashattention_attention_fa_amd as fa

OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP, INTERNAL, VALUE = range(9)
A = 0x10000          # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10008        # 8-byte aligned only


@pytest.fixture(scope="module")
def L():
    return fa.lib()


def test_exports_every_declared_function(L):
    names = fa.declared_functions()
    assert set(names) >= {"fa_fwd", "fa_fwd_varlen", "fa_fwd_fp8", "fa_bwd", "fa_bwd_varlen",
                          "fa_bwd_workspace_bytes", "fa_decode", "fa_decode_ex", "fa_decode_paged",
                          "fa_decode_noalloc",
                          "fa_decode_workspace_bytes",
                          "fa_status_string", "fa_version"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(9):
        assert fa.status_string(s)
    assert fa.status_string(99) == "unknown status"
    assert L.fa_version() >= 100


def fwd(L, q=A, k=A, v=A, o=A, lse=None, B=1, H=1, N=16, d=64, causal=0, scale=0.125, dtype=0):
    return L.fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, None, dtype)


def test_fwd_validation(L):
    assert fwd(L, q=None) == NULL
    assert fwd(L, o=None) == NULL
    assert fwd(L, B=-1) == SHAPE
    assert fwd(L, N=-5) == SHAPE
    assert fwd(L, d=96) == UNSUP
    assert fwd(L, d=256) == UNSUP
    assert fwd(L, dtype=7) == UNSUP
    assert fwd(L, k=MIS) == ALIGN
    assert fwd(L, o=MIS) == ALIGN
    assert fwd(L, lse=A + 2) == ALIGN
    assert fwd(L, scale=float("nan")) == VALUE
    assert fwd(L, scale=float("inf")) == VALUE
    assert fwd(L, N=(1 << 23) + 1) == SHAPE
    assert fwd(L, B=65536, H=65536) == SHAPE


def bwd(L, q=A, k=A, v=A, o=A, do=A, lse=A, dq=A, dk=A, dv=A, B=1, H=2, N=100, d=64, causal=0,
        scale=0.125, dtype=0, ws=0x100000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.fa_bwd_workspace_bytes(B, H, N)
    return L.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, causal, scale, None, dtype, ws,
                    ws_bytes)


def test_bwd_validation(L):
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert bwd(L, **{name: None}) == NULL, name
    for name in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
        assert bwd(L, **{name: MIS}) == ALIGN, name
    assert bwd(L, lse=A + 2) == ALIGN
    assert bwd(L, B=-1) == SHAPE
    assert bwd(L, N=-1) == SHAPE
    assert bwd(L, d=96) == UNSUP
    assert bwd(L, dtype=3) == UNSUP
    assert bwd(L, scale=float("nan")) == VALUE
    assert bwd(L, N=(1 << 23) + 1) == SHAPE
    assert bwd(L, B=65536, H=65536) == SHAPE
    assert bwd(L, ws=None) == WS
    assert bwd(L, ws=0x100080) == WS
    assert bwd(L, ws_bytes=L.fa_bwd_workspace_bytes(1, 2, 100) - 1) == WS
    # empty problems return before any pointer is looked at
    assert bwd(L, q=None, ws=None, B=0) == OK
    assert bwd(L, q=None, ws=None, N=0) == OK


def bwdv(L, q=A, k=A, v=A, o=A, do=A, lse=A, dq=A, dk=A, dv=A, cu=A, B=2, H=2, T=100, maxs=60,
         d=64, causal=0, scale=0.125, dtype=0, ws=0x100000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.fa_bwd_workspace_bytes(1, H, T)
    return L.fa_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, cu, B, H, T, maxs, d, causal, scale,
                           None, dtype, ws, ws_bytes)


def test_bwd_varlen_validation(L):
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "cu"):
        assert bwdv(L, **{name: None}) == NULL, name
    for name in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
        assert bwdv(L, **{name: MIS}) == ALIGN, name
    assert bwdv(L, cu=A + 2) == ALIGN
    assert bwdv(L, B=-1) == SHAPE
    assert bwdv(L, maxs=-1) == SHAPE
    assert bwdv(L, d=80) == UNSUP
    assert bwdv(L, dtype=5) == UNSUP
    assert bwdv(L, scale=float("inf")) == VALUE
    assert bwdv(L, maxs=1 << 22, H=4) == SHAPE
    assert bwdv(L, ws=None) == WS
    assert bwdv(L, ws_bytes=L.fa_bwd_workspace_bytes(1, 2, 100) - 1) == WS
    assert bwdv(L, q=None, cu=None, ws=None, B=0) == OK
    assert bwdv(L, q=None, cu=None, ws=None, T=0) == OK


def test_bwd_workspace_bytes(L):
    # two fp32 arrays [B, H, N], each rounded up to 256 bytes
    assert L.fa_bwd_workspace_bytes(2, 3, 100) == 2 * 2560
    assert L.fa_bwd_workspace_bytes(1, 1, 1) == 512
    assert L.fa_bwd_workspace_bytes(0, 3, 100) == 0
    assert L.fa_bwd_workspace_bytes(-1, 3, 100) == 0


def fwd8(L, q=A, k=A, v=A, o=A, lse=None, B=1, H=1, N=16, d=64, causal=0, scale=0.125,
         dq=1.0, dk=1.0, dv=1.0):
    return L.fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, causal, scale, dq, dk, dv, None)


def test_fwd_fp8_validation(L):
    assert fwd8(L, q=None) == NULL
    assert fwd8(L, v=None) == NULL
    assert fwd8(L, B=-1) == SHAPE
    assert fwd8(L, d=32) == UNSUP
    assert fwd8(L, q=MIS) == ALIGN
    assert fwd8(L, lse=A + 1) == ALIGN
    assert fwd8(L, scale=float("nan")) == VALUE
    assert fwd8(L, dq=float("inf")) == VALUE
    assert fwd8(L, dk=float("nan")) == VALUE
    assert fwd8(L, dv=float("-inf")) == VALUE
    assert fwd8(L, N=(1 << 23) + 1) == SHAPE
    assert fwd8(L, q=None, k=None, v=None, o=None, B=0) == OK


def decp(L, q=A, kp=A, vp=A, bt=A, sl=A, o=A, lse=None, B=1, Hq=4, Hkv=2, page=32, pps=4,
         npages=8, d=128, nsplit=4, dtype=0, ws=A, ws_bytes=1 << 20):
    P = ctypes.c_void_p
    return L.fa_decode_paged(q, kp, vp, P(bt) if bt else None, P(sl) if sl else None, o, lse,
                             B, Hq, Hkv, page, pps, npages, d, nsplit, None, dtype, ws, ws_bytes)


def test_decode_paged_validation(L):
    assert decp(L, page=0) == SHAPE
    assert decp(L, page=24) == SHAPE
    assert decp(L, page=8) == SHAPE
    assert decp(L, pps=0) == SHAPE
    assert decp(L, npages=0) == SHAPE
    assert decp(L, Hkv=3) == SHAPE
    assert decp(L, bt=None) == NULL
    assert decp(L, sl=None) == NULL
    assert decp(L, d=96) == UNSUP
    assert decp(L, bt=A + 2) == ALIGN
    assert decp(L, kp=MIS) == ALIGN
    assert decp(L, ws=None) == WS
    assert decp(L, ws_bytes=16) == WS
    assert decp(L, pps=1 << 20, page=16) == SHAPE
    assert decp(L, q=None, B=0) == OK


def fwdv(L, q=A, k=A, v=A, o=A, lse=None, cu=A, B=2, H=2, T=64, maxs=32, d=128, causal=0,
         scale=0.1, dtype=0):
    return L.fa_fwd_varlen(q, k, v, o, lse, ctypes.c_void_p(cu) if cu else None, B, H, T, maxs,
                           d, causal, scale, None, dtype)


def test_fwd_varlen_validation(L):
    assert fwdv(L, cu=None) == NULL
    assert fwdv(L, q=None) == NULL
    assert fwdv(L, B=-1) == SHAPE
    assert fwdv(L, maxs=-1) == SHAPE
    assert fwdv(L, d=80) == UNSUP
    assert fwdv(L, dtype=5) == UNSUP
    assert fwdv(L, cu=A + 2) == ALIGN
    assert fwdv(L, o=MIS) == ALIGN
    assert fwdv(L, scale=float("nan")) == VALUE
    assert fwdv(L, maxs=1 << 22, H=4) == SHAPE
    assert fwdv(L, q=None, k=None, v=None, o=None, cu=None, B=0) == OK
    assert fwdv(L, q=None, k=None, v=None, o=None, cu=None, T=0) == OK


def test_fwd_empty_is_noop(L):
    # no pointer is needed when there is nothing to compute
    assert fwd(L, q=None, k=None, v=None, o=None, B=0) == OK
    assert fwd(L, q=None, k=None, v=None, o=None, H=0) == OK
    assert fwd(L, q=None, k=None, v=None, o=None, N=0) == OK


def dec(L, q=A, k=A, v=A, o=A, B=1, Hq=4, Hkv=2, Lk=100, d=128, nsplit=4, dtype=0):
    return L.fa_decode(q, k, v, o, B, Hq, Hkv, Lk, d, nsplit, None, dtype)


def dec_ex(L, ws=A, ws_bytes=1 << 20, lse=None, **kw):
    a = dict(q=A, k=A, v=A, o=A, B=1, Hq=4, Hkv=2, Lk=100, d=128, nsplit=4, dtype=0)
    a.update(kw)
    return L.fa_decode_ex(a["q"], a["k"], a["v"], a["o"], lse, a["B"], a["Hq"], a["Hkv"],
                          a["Lk"], a["d"], a["nsplit"], None, a["dtype"], ws, ws_bytes)


def test_decode_validation(L):
    assert dec(L, q=None) == NULL
    assert dec(L, v=None) == NULL
    assert dec(L, Hq=6, Hkv=4) == SHAPE
    assert dec(L, Hkv=0) == SHAPE
    assert dec(L, Lk=0) == SHAPE
    assert dec(L, nsplit=0) == SHAPE
    assert dec(L, d=80) == UNSUP
    assert dec(L, dtype=3) == UNSUP
    assert dec(L, k=MIS) == ALIGN
    assert dec(L, B=70000) == SHAPE
    assert dec(L, Lk=(1 << 23) + 1) == SHAPE
    assert dec(L, q=None, B=0) == OK
    assert dec(L, q=None, Hq=0) == OK


def test_decode_ex_workspace(L):
    need = L.fa_decode_workspace_bytes(1, 4, 128, 4)
    # ws_o = 1*4*4*128*4 = 8192 bytes, ws_lse = 64 -> 256: 8448 bytes
    assert need == 8192 + 256
    assert L.fa_decode_workspace_bytes(1, 4, 100, 4) == 0
    assert L.fa_decode_workspace_bytes(1, 4, 128, 0) == 0
    assert dec_ex(L, ws=None) == WS
    assert dec_ex(L, ws_bytes=need - 1) == WS
    assert dec_ex(L, ws=A + 16) == WS           # not 256-byte aligned
    assert dec_ex(L, lse=A + 1) == ALIGN
    # nsplit larger than L is clamped to L before sizing the workspace
    assert L.fa_decode_workspace_bytes(1, 4, 128, 100) < L.fa_decode_workspace_bytes(1, 4, 128, 200)
    assert dec_ex(L, Lk=3, nsplit=50, ws_bytes=L.fa_decode_workspace_bytes(1, 4, 128, 3) - 1) == WS


def dec_noalloc(L, lse=None, **kw):
    a = dict(q=A, k=A, v=A, o=A, B=1, Hq=4, Hkv=2, Lk=100, d=128, nsplit=4, dtype=0)
    a.update(kw)
    return L.fa_decode_noalloc(a["q"], a["k"], a["v"], a["o"], lse, a["B"], a["Hq"], a["Hkv"],
                               a["Lk"], a["d"], a["nsplit"], None, a["dtype"])


def test_decode_noalloc_validation(L):
    """Every rejection happens before the library looks up its device buffer
    (no HIP call), including a call whose partials would not fit in it."""
    assert fa.DECODE_NOALLOC_MAX_BYTES == 8 << 20
    assert dec_noalloc(L, q=None) == NULL
    assert dec_noalloc(L, o=None) == NULL
    assert dec_noalloc(L, Hq=6, Hkv=4) == SHAPE
    assert dec_noalloc(L, Lk=0) == SHAPE
    assert dec_noalloc(L, nsplit=0) == SHAPE
    assert dec_noalloc(L, d=96) == UNSUP
    assert dec_noalloc(L, dtype=2) == UNSUP
    assert dec_noalloc(L, v=MIS) == ALIGN
    assert dec_noalloc(L, lse=A + 2) == ALIGN
    assert dec_noalloc(L, q=None, B=0) == OK
    # partials of B*Hq*nsplit rows x (d + 1) floats must fit in 8 MiB
    fits = L.fa_decode_workspace_bytes(8, 32, 128, 16)
    assert fits <= fa.DECODE_NOALLOC_MAX_BYTES
    big = L.fa_decode_workspace_bytes(8, 32, 128, 64)
    assert big > fa.DECODE_NOALLOC_MAX_BYTES
    assert dec_noalloc(L, B=8, Hq=32, Hkv=8, Lk=32768, nsplit=64) == WS


def test_python_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q.float())
    with pytest.raises(ValueError):
        fa.fwd(q, q, q[:, :1])
    with pytest.raises(ValueError):      # CPU tensors are rejected before any call
        fa.fwd(q, q, q)
    with pytest.raises(ValueError):
        fa.decode(q[:, :, 0], q, q.half(), nsplit=2)
    o = torch.zeros(1, 2, 8, 64)
    lse = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):      # o must be fp32
        fa.bwd(q, q, q, o.half(), lse, q)
    with pytest.raises(ValueError):      # lse shape
        fa.bwd(q, q, q, o, lse[:, :1], q)
    with pytest.raises(ValueError):      # dout dtype differs
        fa.bwd(q, q, q, o, lse, q.half())
    with pytest.raises(ValueError):      # CPU tensors
        fa.bwd(q, q, q, o, lse, q)
    p = torch.zeros(16, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 16], dtype=torch.int32)
    with pytest.raises(ValueError):      # lse must be [H, T]
        fa.bwd_varlen(p, p, p, torch.zeros(16, 2, 64), torch.zeros(16, 2), p, cu, 16)
    with pytest.raises(ValueError):      # cu_seqlens must be int32
        fa.bwd_varlen(p, p, p, torch.zeros(16, 2, 64), torch.zeros(2, 16), p, cu.long(), 16)


def test_ceiling_library_exports_and_rejects():
    """libfa_ceiling.so (the benchmark's measurement kernels) exports what
    include/fa_ceiling.h declares and rejects bad arguments before any launch."""
    import re
    from pathlib import Path
    path = Path(fa.LIB_PATH).with_name("libfa_ceiling.so")
    C = ctypes.CDLL(str(path))
    text = re.sub(r"/\*.*?\*/", "", (Path(fa.HEADER_PATH).with_name("fa_ceiling.h")).read_text(),
                  flags=re.S)
    names = re.findall(r"^\s*int\s+(fa_[a-z0-9_]+)\s*\(", text, flags=re.M)
    assert names == ["fa_ceiling_mfma", "fa_ceiling_lds", "fa_ceiling_read"]
    for n in names:
        assert hasattr(C, n), n
    P, I = ctypes.c_void_p, ctypes.c_int
    C.fa_ceiling_mfma.argtypes = [P, P, I, I, I, P]
    C.fa_ceiling_read.argtypes = [P, ctypes.c_size_t, P, I, I, P]
    C.fa_ceiling_lds.argtypes = [P, I, I, I, P]
    bad = 1                                               # hipErrorInvalidValue
    assert C.fa_ceiling_mfma(None, A, 1, 1, 1, None) == bad
    assert C.fa_ceiling_mfma(A, A, 0, 1, 1, None) == bad
    assert C.fa_ceiling_mfma(A, A, 1, 1, 5, None) == bad
    assert C.fa_ceiling_mfma(A, A, 1, 1, -1, None) == bad
    assert C.fa_ceiling_mfma(MIS, A, 1, 1, 1, None) == bad
    assert C.fa_ceiling_lds(None, 1, 1, 0, None) == bad
    assert C.fa_ceiling_lds(A, 0, 1, 0, None) == bad
    assert C.fa_ceiling_lds(A, 1, 0, 0, None) == bad
    assert C.fa_ceiling_lds(A, 1, 1, 2, None) == bad
    assert C.fa_ceiling_read(A, 0, A, 1, 1, None) == bad
    assert C.fa_ceiling_read(A, 24, A, 1, 1, None) == bad
    assert C.fa_ceiling_read(A, 1 << 32, A, 1, 1, None) == bad    # a 4 GiB chunk
