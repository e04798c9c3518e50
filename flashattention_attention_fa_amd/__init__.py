"""MI355X-native exact attention: FlashAttention forward and split-KV
flash-decode, hand-written HIP kernels for gfx950.

This module is the Python binding of libfa_amd.so (C ABI in include/fa.h).
It only marshals arguments: it checks tensor shapes, dtypes and devices,
allocates outputs and workspaces with torch (device memory and streams are
all torch is used for) and calls the library.  Anything allocated here is
allocated on the stream the call is launched on, so torch's caching
allocator cannot hand it to other work before the kernels are done with it.  Every step of the computation runs in the
library's kernels; if the library is missing the calls raise instead of
falling back to anything else.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import re
from pathlib import Path

import torch

__all__ = ["fwd", "fwd_varlen", "fwd_fp8", "bwd", "bwd_varlen", "bwd_workspace_bytes", "decode",
           "decode_noalloc", "decode_paged", "decode_workspace_bytes", "lib", "FAError", "LIB_PATH",
           "HEADER_PATH", "status_string"]

LIB_PATH = Path(__file__).resolve().parent / "libfa_amd.so"
HEADER_PATH = Path(__file__).resolve().parent.parent / "include" / "fa.h"

_DTYPE = {torch.bfloat16: 0, torch.float16: 1}
_lib = None


class FAError(RuntimeError):
    """A library call returned a non-OK status."""


def lib() -> ctypes.CDLL:
    """The loaded libfa_amd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m flashattention_attention_fa_amd.build`")
        L = ctypes.CDLL(str(LIB_PATH))
        P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, F, P, I]
        L.fa_fwd.restype = I
        L.fa_fwd_varlen.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, P, I]
        L.fa_fwd_varlen.restype = I
        L.fa_fwd_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, F, F, F, F, P]
        L.fa_fwd_fp8.restype = I
        L.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, P, I, P, S]
        L.fa_bwd.restype = I
        L.fa_bwd_varlen.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, I, P,
                                    S]
        L.fa_bwd_varlen.restype = I
        L.fa_bwd_workspace_bytes.argtypes = [I, I, I]
        L.fa_bwd_workspace_bytes.restype = S
        L.fa_decode.argtypes = [P, P, P, P, I, I, I, I, I, I, P, I]
        L.fa_decode.restype = I
        L.fa_decode_ex.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, I, P, S]
        L.fa_decode_ex.restype = I
        L.fa_decode_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, I]
        L.fa_decode_noalloc.restype = I
        L.fa_decode_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P, I, P, S]
        L.fa_decode_paged.restype = I
        L.fa_decode_workspace_bytes.argtypes = [I, I, I, I]
        L.fa_decode_workspace_bytes.restype = S
        L.fa_status_string.argtypes = [I]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_version.argtypes = []
        L.fa_version.restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def declared_functions() -> list[str]:
    """Names of the functions include/fa.h declares."""
    text = re.sub(r"/\*.*?\*/", "", HEADER_PATH.read_text(), flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(fa_[a-z0-9_]+)\s*\(",
                      text, flags=re.M)


def _check(status: int, what: str):
    if status != 0:
        raise FAError(f"{what}: {status_string(status)} (status {status})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _alloc_on(stream):
    """Context in which torch allocations belong to the launch stream: a
    buffer freed when the binding returns is then reused only by later work
    on that same stream, which runs after the kernels that use it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _check_out(t, shape, device, what):
    _need(t.shape == tuple(shape) and t.dtype == torch.float32 and t.is_contiguous()
          and t.device == device, f"{what} must be a contiguous fp32 {list(shape)} tensor on {device}")


# Bytes of fa_decode_noalloc's fixed per-device buffer (FA_DECODE_NOALLOC_MAX_BYTES).
DECODE_NOALLOC_MAX_BYTES = 8 << 20


def fwd(q, k, v, *, causal: bool = False, scale: float | None = None, out=None, lse=None,
        return_lse: bool = True, stream=None):
    """Exact attention forward.  q, k, v: [B, H, N, d] bf16/fp16 CUDA tensors.
    Returns (o [B, H, N, d] fp32, lse [B, H, N] fp32 or None)."""
    _need(q.dim() == 4 and q.shape == k.shape == v.shape, "q, k, v must share a [B,H,N,d] shape")
    _need(q.dtype in _DTYPE and q.dtype == k.dtype == v.dtype, "q, k, v must all be bf16 or fp16")
    _need(q.is_cuda and k.device == q.device and v.device == q.device, "tensors must be on one GPU")
    _need(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(), "tensors must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with _alloc_on(stream):
        if out is None:
            out = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
        if lse is None and return_lse:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_out(out, (B, H, N, d), q.device, "out")
    if lse is not None:
        _check_out(lse, (B, H, N), q.device, "lse")
    st = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                      int(bool(causal)), float(scale), _stream(stream, q.device), _DTYPE[q.dtype])
    _check(st, "fa_fwd")
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, *, causal: bool = False,
               scale: float | None = None, out=None, lse=None, return_lse: bool = True,
               stream=None):
    """Attention over a packed batch of variable-length sequences.
    q, k, v: [T, H, d] bf16/fp16; cu_seqlens: [B+1] int32 on the GPU (sequence
    b = rows cu[b]..cu[b+1]); max_seqlen: host int >= every length.
    Returns (o [T, H, d] fp32, lse [H, T] fp32 or None)."""
    _need(q.dim() == 3 and q.shape == k.shape == v.shape, "q, k, v must share a [T,H,d] shape")
    _need(q.dtype in _DTYPE and q.dtype == k.dtype == v.dtype, "q, k, v must all be bf16 or fp16")
    _need(cu_seqlens.dim() == 1 and cu_seqlens.dtype == torch.int32 and cu_seqlens.numel() >= 1,
          "cu_seqlens must be int32 [B+1]")
    _need(q.is_cuda and q.is_contiguous(), "q must be a contiguous GPU tensor")
    for t in (k, v, cu_seqlens):
        _need(t.device == q.device and t.is_contiguous(), "contiguous tensors on one GPU")
    T, H, d = q.shape
    B = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with _alloc_on(stream):
        if out is None:
            out = torch.empty((T, H, d), dtype=torch.float32, device=q.device)
        if lse is None and return_lse:
            lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    _check_out(out, (T, H, d), q.device, "out")
    if lse is not None:
        _check_out(lse, (H, T), q.device, "lse")
    st = lib().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens),
                             B, H, T, int(max_seqlen), d, int(bool(causal)), float(scale),
                             _stream(stream, q.device), _DTYPE[q.dtype])
    _check(st, "fa_fwd_varlen")
    return out, lse


def fwd_fp8(q, k, v, *, q_descale: float, k_descale: float, v_descale: float,
            causal: bool = False, scale: float | None = None, out=None, lse=None,
            return_lse: bool = True, stream=None):
    """Attention forward on FP8 E4M3 inputs: q, k, v are [B, H, N, d] CUDA
    tensors of E4M3 bytes (torch.uint8, or torch.float8_e4m3fn); the result
    is the attention of q_descale*q, k_descale*k, v_descale*v.
    Returns (o [B, H, N, d] fp32, lse [B, H, N] fp32 or None)."""
    _need(q.dim() == 4 and q.shape == k.shape == v.shape, "q, k, v must share a [B,H,N,d] shape")
    _need(all(t.dtype in (torch.uint8, torch.float8_e4m3fn) for t in (q, k, v)),
          "q, k, v must hold E4M3 bytes (uint8 or float8_e4m3fn)")
    _need(q.is_cuda and k.device == q.device and v.device == q.device, "tensors must be on one GPU")
    _need(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(), "tensors must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with _alloc_on(stream):
        if out is None:
            out = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
        if lse is None and return_lse:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_out(out, (B, H, N, d), q.device, "out")
    if lse is not None:
        _check_out(lse, (B, H, N), q.device, "lse")
    st = lib().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                          int(bool(causal)), float(scale), float(q_descale), float(k_descale),
                          float(v_descale), _stream(stream, q.device))
    _check(st, "fa_fwd_fp8")
    return out, lse


def bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H, N))


def _grads(shape, device, given, stream):
    outs = []
    with _alloc_on(stream):
        for g in given:
            if g is None:
                g = torch.empty(shape, dtype=torch.float32, device=device)
            _check_out(g, shape, device, "gradients")
            outs.append(g)
    return outs


def _workspace(workspace, nbytes, device, stream):
    if workspace is None:
        with _alloc_on(stream):
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _need(workspace.is_cuda and workspace.device == device and workspace.is_contiguous(),
          "workspace must be a contiguous tensor on the inputs' GPU")
    return workspace, workspace.numel() * workspace.element_size()


def bwd(q, k, v, o, lse, dout, *, causal: bool = False, scale: float | None = None,
        dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Attention backward.  q, k, v, dout: [B, H, N, d] bf16/fp16 CUDA
    tensors (one dtype); o [B, H, N, d] and lse [B, H, N]: fp32 outputs of
    ``fwd`` for the same q, k, v, causal and scale.  Returns
    (dq, dk, dv), each [B, H, N, d] fp32."""
    _need(q.dim() == 4 and q.shape == k.shape == v.shape == dout.shape,
          "q, k, v, dout must share a [B,H,N,d] shape")
    _need(q.dtype in _DTYPE and q.dtype == k.dtype == v.dtype == dout.dtype,
          "q, k, v, dout must all be bf16 or all fp16")
    B, H, N, d = q.shape
    _need(o.shape == q.shape and o.dtype == torch.float32, "o must be fp32 [B,H,N,d]")
    _need(lse.shape == (B, H, N) and lse.dtype == torch.float32, "lse must be fp32 [B,H,N]")
    ts = (q, k, v, dout, o, lse)
    _need(all(t.is_cuda and t.device == q.device for t in ts), "tensors must be on one GPU")
    _need(all(t.is_contiguous() for t in ts), "tensors must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs = _grads((B, H, N, d), q.device, (dq, dk, dv), stream)
    workspace, ws_bytes = _workspace(workspace, bwd_workspace_bytes(B, H, N), q.device, stream)
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(outs[0]),
                      _ptr(outs[1]), _ptr(outs[2]), B, H, N, d, int(bool(causal)), float(scale),
                      _stream(stream, q.device), _DTYPE[q.dtype], _ptr(workspace), ws_bytes)
    _check(st, "fa_bwd")
    return tuple(outs)


def bwd_varlen(q, k, v, o, lse, dout, cu_seqlens, max_seqlen: int, *, causal: bool = False,
               scale: float | None = None, dq=None, dk=None, dv=None, workspace=None,
               stream=None):
    """Backward of ``fwd_varlen``.  q, k, v, dout: packed [T, H, d] bf16/fp16;
    o [T, H, d] and lse [H, T] fp32 from ``fwd_varlen``; cu_seqlens: int32
    [B + 1] on the device.  Returns (dq, dk, dv), each [T, H, d] fp32 (rows
    outside every sequence are left as allocated)."""
    _need(q.dim() == 3 and q.shape == k.shape == v.shape == dout.shape,
          "q, k, v, dout must share a [T,H,d] shape")
    _need(q.dtype in _DTYPE and q.dtype == k.dtype == v.dtype == dout.dtype,
          "q, k, v, dout must all be bf16 or all fp16")
    T, H, d = q.shape
    _need(o.shape == q.shape and o.dtype == torch.float32, "o must be fp32 [T,H,d]")
    _need(lse.shape == (H, T) and lse.dtype == torch.float32, "lse must be fp32 [H,T]")
    _need(cu_seqlens.dim() == 1 and cu_seqlens.dtype == torch.int32, "cu_seqlens: int32 [B+1]")
    ts = (q, k, v, dout, o, lse, cu_seqlens)
    _need(all(t.is_cuda and t.device == q.device for t in ts), "tensors must be on one GPU")
    _need(all(t.is_contiguous() for t in ts), "tensors must be contiguous")
    B = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs = _grads((T, H, d), q.device, (dq, dk, dv), stream)
    workspace, ws_bytes = _workspace(workspace, bwd_workspace_bytes(1, H, T), q.device, stream)
    st = lib().fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                             _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _ptr(cu_seqlens), B, H,
                             T, int(max_seqlen), d, int(bool(causal)), float(scale),
                             _stream(stream, q.device), _DTYPE[q.dtype], _ptr(workspace),
                             ws_bytes)
    _check(st, "fa_bwd_varlen")
    return tuple(outs)


def decode_workspace_bytes(B: int, Hq: int, d: int, nsplit: int) -> int:
    return int(lib().fa_decode_workspace_bytes(B, Hq, d, nsplit))


def _decode_args(q, kcache, vcache):
    _need(q.dim() == 3 and kcache.dim() == 4 and kcache.shape == vcache.shape,
          "q must be [B,Hq,d] and the caches [B,Hkv,L,d]")
    B, Hq, d = q.shape
    Bk, Hkv, L, dk = kcache.shape
    _need(Bk == B and dk == d, "batch / head_dim mismatch between q and the caches")
    _need(q.dtype in _DTYPE and q.dtype == kcache.dtype == vcache.dtype, "bf16 or fp16 inputs")
    _need(q.is_cuda and kcache.device == q.device and vcache.device == q.device, "one GPU")
    _need(q.is_contiguous() and kcache.is_contiguous() and vcache.is_contiguous(), "contiguous")
    return B, Hq, Hkv, L, d


def decode(q, kcache, vcache, *, nsplit: int, out=None, lse=None, return_lse: bool = False,
           workspace=None, stream=None):
    """Split-KV flash-decode.  q: [B, Hq, d]; kcache, vcache: [B, Hkv, L, d].
    With return_lse, an lse buffer or a workspace given, the call goes through
    fa_decode_ex (caller-owned workspace, allocated here with torch if not
    given); otherwise through fa_decode (library-managed workspace).
    Returns (o [B, Hq, d] fp32, lse [B, Hq] fp32 or None)."""
    B, Hq, Hkv, L, d = _decode_args(q, kcache, vcache)
    with _alloc_on(stream):
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        if lse is None and return_lse:
            lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check_out(out, (B, Hq, d), q.device, "out")
    if lse is not None:
        _check_out(lse, (B, Hq), q.device, "lse")
    s = _stream(stream, q.device)
    if lse is None and workspace is None:
        st = lib().fa_decode(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(out), B, Hq, Hkv, L, d,
                             int(nsplit), s, _DTYPE[q.dtype])
        _check(st, "fa_decode")
        return out, None
    nbytes = decode_workspace_bytes(B, Hq, d, max(1, min(int(nsplit), L)))
    workspace, ws_bytes = _workspace(workspace, nbytes, q.device, stream)
    st = lib().fa_decode_ex(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(out), _ptr(lse), B, Hq,
                            Hkv, L, d, int(nsplit), s, _DTYPE[q.dtype], _ptr(workspace), ws_bytes)
    _check(st, "fa_decode_ex")
    return out, lse


def decode_noalloc(q, kcache, vcache, *, nsplit: int, out, lse=None, stream=None):
    """Split-KV flash-decode through fa_decode_noalloc: the library allocates
    nothing (its shard partials live in a fixed per-device buffer of
    DECODE_NOALLOC_MAX_BYTES), and this binding allocates nothing either, so
    the caller passes ``out`` [B, Hq, d] fp32 (and optionally ``lse`` [B, Hq]
    fp32).  Calls that overlap in time on one GPU share that buffer and race.
    Returns (out, lse)."""
    B, Hq, Hkv, L, d = _decode_args(q, kcache, vcache)
    _check_out(out, (B, Hq, d), q.device, "out")
    if lse is not None:
        _check_out(lse, (B, Hq), q.device, "lse")
    st = lib().fa_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(out), _ptr(lse), B,
                                 Hq, Hkv, L, d, int(nsplit), _stream(stream, q.device),
                                 _DTYPE[q.dtype])
    _check(st, "fa_decode_noalloc")
    return out, lse


def decode_paged(q, kpages, vpages, block_table, seq_lens, *, nsplit: int, out=None, lse=None,
                 return_lse: bool = True, workspace=None, stream=None):
    """Split-KV flash-decode over a paged cache.  q: [B, Hq, d];
    kpages, vpages: [num_pages, page_size, Hkv, d] (bf16/fp16);
    block_table: [B, pages_per_seq] int32; seq_lens: [B] int32 (all on the GPU).
    Returns (o [B, Hq, d] fp32, lse [B, Hq] fp32 or None)."""
    _need(q.dim() == 3 and kpages.dim() == 4 and kpages.shape == vpages.shape,
          "q must be [B,Hq,d] and the page pools [num_pages,page_size,Hkv,d]")
    B, Hq, d = q.shape
    num_pages, page_size, Hkv, dk = kpages.shape
    _need(dk == d, "head_dim mismatch between q and the page pools")
    _need(q.dtype in _DTYPE and q.dtype == kpages.dtype == vpages.dtype, "bf16 or fp16 inputs")
    _need(block_table.dim() == 2 and block_table.shape[0] == B and block_table.dtype == torch.int32,
          "block_table must be int32 [B, pages_per_seq]")
    _need(seq_lens.shape == (B,) and seq_lens.dtype == torch.int32, "seq_lens must be int32 [B]")
    _need(q.is_cuda and q.is_contiguous(), "q must be a contiguous GPU tensor")
    for t in (kpages, vpages, block_table, seq_lens):
        _need(t.device == q.device and t.is_contiguous(), "contiguous tensors on one GPU")
    with _alloc_on(stream):
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        if lse is None and return_lse:
            lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check_out(out, (B, Hq, d), q.device, "out")
    if lse is not None:
        _check_out(lse, (B, Hq), q.device, "lse")
    workspace, ws_bytes = _workspace(workspace, decode_workspace_bytes(B, Hq, d, int(nsplit)),
                                     q.device, stream)
    st = lib().fa_decode_paged(_ptr(q), _ptr(kpages), _ptr(vpages), _ptr(block_table),
                               _ptr(seq_lens), _ptr(out), _ptr(lse), B, Hq, Hkv, page_size,
                               block_table.shape[1], num_pages, d, int(nsplit),
                               _stream(stream, q.device), _DTYPE[q.dtype], _ptr(workspace),
                               ws_bytes)
    _check(st, "fa_decode_paged")
    return out, lse
