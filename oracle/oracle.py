"""fp64 CPU oracle for exact attention, split-KV partials and their combine,
and the gradients of attention.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path never
imports this module, and this module imports nothing from the product.

The arithmetic lives in ``fa_oracle.c`` (plain C, fp64, OpenMP over rows);
this file builds it with gcc and marshals numpy arrays through ctypes.

Inputs are bit patterns of the values a GPU kernel would consume: 16-bit
(``numpy.uint16``) bf16 or fp16, or bytes (``numpy.uint8``) of FP8 E4M3 with
per-tensor dequantization factors; the C code widens them exactly to
double.  Layouts follow the (batch, heads, seq_len, head_dim) convention of
the benchmark listing on the dailyaiworld page "FlashAttention-3 vs Triton
Kernels", section "Benchmarking Triton vs FlashAttention-3 Kernels".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "fa_oracle.c"
_LIB_PATH = _HERE / "libfa_oracle.so"

DTYPES = {"bf16": 0, "fp16": 1, "fp8": 2}


def build(out: Path | None = None, mutant: int = 0) -> Path:
    """Compile fa_oracle.c with gcc (fp64, no fast-math).  ``mutant`` > 0
    plants one deliberate mistake; only the pin-sensitivity test uses it."""
    out = Path(out) if out is not None else _LIB_PATH
    tmp = f"{out}.tmp{os.getpid():x}"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-o", tmp, str(_SRC), "-lm"]
    if mutant:
        cmd.insert(1, f"-DORACLE_MUTANT={int(mutant)}")
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one build of fa_oracle.c."""

    def __init__(self, path: Path | None = None):
        path = Path(path) if path is not None else _LIB_PATH
        if not path.exists() or (path == _LIB_PATH and
                                 path.stat().st_mtime < _SRC.stat().st_mtime):
            build(path)
        self.lib = ctypes.CDLL(str(path))
        L, P, D, I = ctypes.c_long, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
        self.lib.oracle_attention_rows.argtypes = [P, P, P, I, L, L, L, L, L, L,
                                                   I, D, L, L, P, L, P, P]
        self.lib.oracle_attention_rows.restype = I
        self.lib.oracle_attention_rows_dq.argtypes = [P, P, P, I, D, D, D, L, L, L, L, L,
                                                      L, I, D, L, L, P, L, P, P]
        self.lib.oracle_attention_rows_dq.restype = I
        self.lib.oracle_combine.argtypes = [P, P, L, L, P, P]
        self.lib.oracle_combine.restype = None
        self.lib.oracle_decode.argtypes = [P, P, P, I, L, L, L, L, L, P, P]
        self.lib.oracle_decode.restype = I
        self.lib.oracle_widen.argtypes = [ctypes.c_uint16, I]
        self.lib.oracle_widen.restype = D
        self.lib.oracle_attention_bwd.argtypes = [P, P, P, P, I, L, L, L, L, I, D, P, L, P, L,
                                                  P, P, P, P, P]
        self.lib.oracle_attention_bwd.restype = I

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _bits(a: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(a)
        if a.dtype != np.uint16:
            raise TypeError("oracle inputs are uint16 bit patterns")
        return a

    @staticmethod
    def _ptr(a: np.ndarray) -> int:
        return a.ctypes.data

    def widen(self, bits: int, dtype: str) -> float:
        return self.lib.oracle_widen(int(bits), DTYPES[dtype])

    def widen_many(self, bits, dtype: str) -> np.ndarray:
        """oracle_widen of every pattern in ``bits``, one call each."""
        f, t = self.lib.oracle_widen, DTYPES[dtype]
        return np.array([f(int(b), t) for b in np.asarray(bits).ravel()], dtype=np.float64)

    # -- attention over explicit rows ---------------------------------------
    def attention_rows(self, q, k, v, dtype: str, rows, causal: bool,
                       scale: float, klo: int = 0, khi: int | None = None):
        """q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] (uint16 bits); rows: (n,3) int
        array of (b, hq, i).  Returns (o [n,d] float64, lse [n] float64)."""
        q, k, v = self._bits(q), self._bits(k), self._bits(v)
        B, Hq, Nq, d = q.shape
        Bk, Hkv, Nk, dk = k.shape
        if v.shape != k.shape or Bk != B or dk != d:
            raise ValueError("shape mismatch")
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        n = rows.shape[0]
        o = np.zeros((n, d), np.float64)
        lse = np.zeros(n, np.float64)
        khi = Nk if khi is None else khi
        rc = self.lib.oracle_attention_rows(
            self._ptr(q), self._ptr(k), self._ptr(v), DTYPES[dtype], B, Hq, Hkv,
            Nq, Nk, d, int(bool(causal)), float(scale), int(klo), int(khi),
            self._ptr(rows), n, self._ptr(o), self._ptr(lse))
        if rc != 0:
            raise ValueError("oracle_attention_rows rejected its arguments")
        return o, lse

    def attention_rows_fp8(self, q, k, v, rows, causal: bool, scale: float,
                           dq: float, dk: float, dv: float):
        """FP8 E4M3 inputs (uint8 bytes) with dequantization factors: the
        attention of dq*q, dk*k, dv*v over explicit rows."""
        arrs = []
        for a in (q, k, v):
            a = np.ascontiguousarray(a)
            if a.dtype != np.uint8:
                raise TypeError("FP8 oracle inputs are uint8 bytes")
            arrs.append(a.astype(np.uint16))
        q, k, v = arrs
        B, Hq, Nq, d = q.shape
        Bk, Hkv, Nk, dk_ = k.shape
        if v.shape != k.shape or Bk != B or dk_ != d:
            raise ValueError("shape mismatch")
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        n = rows.shape[0]
        o = np.zeros((n, d), np.float64)
        lse = np.zeros(n, np.float64)
        rc = self.lib.oracle_attention_rows_dq(
            self._ptr(q), self._ptr(k), self._ptr(v), DTYPES["fp8"], float(dq), float(dk),
            float(dv), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), float(scale), 0, Nk,
            self._ptr(rows), n, self._ptr(o), self._ptr(lse))
        if rc != 0:
            raise ValueError("oracle_attention_rows_dq rejected its arguments")
        return o, lse

    def attention_fp8(self, q, k, v, causal: bool, scale: float, dq: float, dk: float,
                      dv: float):
        """Every row of a [B,H,N,d] FP8 problem."""
        B, H, N, d = q.shape
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
        o, lse = self.attention_rows_fp8(q, k, v, rows, causal, scale, dq, dk, dv)
        return o.reshape(B, H, N, d), lse.reshape(B, H, N)

    def attention(self, q, k, v, dtype: str, causal: bool, scale: float):
        """Every row of a [B,H,N,d] problem: (o [B,H,N,d], lse [B,H,N])."""
        B, H, N, d = q.shape
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(H), np.arange(N),
                                 indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
        o, lse = self.attention_rows(q, k, v, dtype, rows, causal, scale)
        return o.reshape(B, H, N, d), lse.reshape(B, H, N)

    def combine(self, part_o, part_lse):
        """part_o [nsplit, d], part_lse [nsplit] -> (o [d], lse)."""
        part_o = np.ascontiguousarray(part_o, dtype=np.float64)
        part_lse = np.ascontiguousarray(part_lse, dtype=np.float64)
        ns, d = part_o.shape
        o = np.zeros(d, np.float64)
        lse = ctypes.c_double(0.0)
        self.lib.oracle_combine(self._ptr(part_o), self._ptr(part_lse), ns, d,
                                self._ptr(o), ctypes.addressof(lse))
        return o, lse.value

    def decode(self, q, kc, vc, dtype: str):
        """q [B,Hq,d], caches [B,Hkv,L,d] -> (o [B,Hq,d], lse [B,Hq]);
        scale 1/sqrt(d), every cached key visible."""
        q, kc, vc = self._bits(q), self._bits(kc), self._bits(vc)
        B, Hq, d = q.shape
        _, Hkv, L, _ = kc.shape
        o = np.zeros((B, Hq, d), np.float64)
        lse = np.zeros((B, Hq), np.float64)
        rc = self.lib.oracle_decode(self._ptr(q), self._ptr(kc), self._ptr(vc),
                                    DTYPES[dtype], B, Hq, Hkv, L, d,
                                    self._ptr(o), self._ptr(lse))
        if rc != 0:
            raise ValueError("oracle_decode rejected its arguments")
        return o, lse

    # -- gradients -----------------------------------------------------------
    def attention_bwd(self, q, k, v, dout, dtype: str, causal: bool, scale: float,
                      qrows=None, kcols=None):
        """Gradients of self-attention with upstream gradient ``dout``.

        q, k, v, dout: [B,H,N,d] uint16 bit patterns of ``dtype``, or float64
        arrays with ``dtype="f64"``.  qrows / kcols: (n,3) arrays of
        (b, h, i); None means every row.  Returns a dict with dq, o, lse (for
        qrows) and dk, dv (for kcols); with both None the arrays have the
        shapes [B,H,N,d] and [B,H,N]."""
        if dtype == "f64":
            code = 3
            arrs = [np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v, dout)]
        else:
            code = DTYPES[dtype]
            arrs = [self._bits(a) for a in (q, k, v, dout)]
        q, k, v, dout = arrs
        if not (q.shape == k.shape == v.shape == dout.shape) or q.ndim != 4:
            raise ValueError("shape mismatch")
        B, H, N, d = q.shape
        full = qrows is None and kcols is None
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
        every = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
        qrows = every if qrows is None else qrows
        kcols = every if kcols is None else kcols
        qrows = np.ascontiguousarray(np.asarray(qrows, dtype=np.int64).reshape(-1, 3))
        kcols = np.ascontiguousarray(np.asarray(kcols, dtype=np.int64).reshape(-1, 3))
        nq, nk = qrows.shape[0], kcols.shape[0]
        dq = np.zeros((nq, d)); o = np.zeros((nq, d)); lse = np.zeros(nq)
        dk = np.zeros((nk, d)); dv = np.zeros((nk, d))
        rc = self.lib.oracle_attention_bwd(
            self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(dout), code, B, H, N, d,
            int(bool(causal)), float(scale), self._ptr(qrows), nq, self._ptr(kcols), nk,
            self._ptr(dq), self._ptr(o), self._ptr(lse), self._ptr(dk), self._ptr(dv))
        if rc != 0:
            raise ValueError("oracle_attention_bwd rejected its arguments")
        out = {"dq": dq, "o": o, "lse": lse, "dk": dk, "dv": dv}
        if full:
            for key in ("dq", "o", "dk", "dv"):
                out[key] = out[key].reshape(B, H, N, d)
            out["lse"] = lse.reshape(B, H, N)
        return out


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from fa_oracle.c (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
