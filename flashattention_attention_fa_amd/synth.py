"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and picks row indices; it holds none of the
attention arithmetic, so both the HIP path and the fp64 oracle can consume
what it produces without sharing any of the method's code.

Recipe (the benchmark listing on the dailyaiworld page "FlashAttention-3 vs
Triton Kernels", section "Benchmarking Triton vs FlashAttention-3 Kernels",
draws ``randn`` tensors of shape (batch, heads, seq_len, head_dim)):
values are i.i.d. N(0, 1) drawn in fp32 from a seeded ``torch.Generator``
and rounded to the 16-bit storage type (round to nearest even).  The
causal stress workload additionally multiplies every key row (b, h, j) by a
factor drawn i.i.d. from U[0.5, 4] in fp32 before the rounding.
"""
from __future__ import annotations

import numpy as np
import torch

TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


def normal(shape, seed: int, dtype: str = "bf16", device="cpu") -> torch.Tensor:
    g = torch.Generator(device=device).manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.to(TORCH_DTYPES[dtype])


def uniform(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    g = torch.Generator(device=device).manual_seed(int(seed))
    x = torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return lo + (hi - lo) * x


def fwd_inputs(B, H, N, d, dtype="bf16", seed=0, device="cpu",
               krow_scale: tuple[float, float] | None = None):
    """q, k, v of shape [B, H, N, d]; seeds seed*16 + {0: q, 1: k, 2: v, 3: key-row factor}."""
    base = int(seed) * 16
    q = normal((B, H, N, d), base + 0, dtype, device)
    if krow_scale is None:
        k = normal((B, H, N, d), base + 1, dtype, device)
    else:
        g = torch.Generator(device=device).manual_seed(base + 1)
        kf = torch.randn((B, H, N, d), generator=g, device=device, dtype=torch.float32)
        f = uniform((B, H, N, 1), krow_scale[0], krow_scale[1], base + 3, device)
        k = (kf * f).to(TORCH_DTYPES[dtype])
        del kf, f
    v = normal((B, H, N, d), base + 2, dtype, device)
    return q, k, v


def bwd_inputs(B, H, N, d, dtype="bf16", seed=0, device="cpu"):
    """q, k, v as fwd_inputs, plus the upstream gradient dout [B, H, N, d]
    (i.i.d. N(0, 1), seed seed*16 + 4, rounded to the storage type)."""
    q, k, v = fwd_inputs(B, H, N, d, dtype, seed, device)
    dout = normal((B, H, N, d), int(seed) * 16 + 4, dtype, device)
    return q, k, v, dout


def fp8_inputs(B, H, N, d, seed=0, device="cpu", amp=8.0):
    """FP8 (E4M3) q, k, v of shape [B, H, N, d] as uint8 tensors holding the
    E4M3 bytes, and their per-tensor dequantization factor 1/amp: each
    tensor is amp * N(0, 1) drawn in fp32 (seeds as fwd_inputs) and rounded
    to E4M3 (nearest even), so the dequantized values follow N(0, 1)."""
    base = int(seed) * 16
    out = []
    for i in range(3):
        g = torch.Generator(device=device).manual_seed(base + i)
        x = torch.randn((B, H, N, d), generator=g, device=device, dtype=torch.float32)
        out.append((x * amp).to(torch.float8_e4m3fn).view(torch.uint8))
    return out[0], out[1], out[2], 1.0 / amp


def fp8_bits(t: torch.Tensor) -> np.ndarray:
    """uint8 E4M3 tensor -> host numpy uint8 (what the oracle reads)."""
    if t.dtype != torch.uint8:
        raise TypeError("expected a uint8 tensor of E4M3 bytes")
    return t.detach().contiguous().cpu().numpy()


def decode_inputs(B, Hq, Hkv, L, d, dtype="bf16", seed=0, device="cpu"):
    """q [B, Hq, d] (one new token per sequence), kcache/vcache [B, Hkv, L, d]."""
    base = int(seed) * 16
    q = normal((B, Hq, d), base + 0, dtype, device)
    k = normal((B, Hkv, L, d), base + 1, dtype, device)
    v = normal((B, Hkv, L, d), base + 2, dtype, device)
    return q, k, v


def varlen_inputs(lens, H, d, dtype="bf16", seed=0, device="cpu"):
    """A packed batch of len(lens) sequences: q, k, v [T, H, d] i.i.d. N(0,1)
    with T = sum(lens) (seeds as fwd_inputs), and cu_seqlens [B+1] int32."""
    base = int(seed) * 16
    T = int(sum(lens))
    q, k, v = (normal((T, H, d), base + i, dtype, device) for i in range(3))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=device)
    return q, k, v, cu


def paged_decode_inputs(B, Hq, Hkv, L, d, page, dtype="bf16", seed=0, device="cpu"):
    """Decode inputs with the caches in pages: q [B, Hq, d]; K and V pools
    [B*L/page, page, Hkv, d] i.i.d. N(0,1); a block table [B, L/page] int32
    holding a seeded permutation of the pools' pages (key j of sequence b is
    slot j % page of page table[b, j // page]); seq_lens [B] int32, all L."""
    if L % page:
        raise ValueError("L must be a multiple of the page size")
    pps = L // page
    base = int(seed) * 16
    rng = np.random.default_rng(int(seed))
    table = torch.from_numpy(rng.permutation(B * pps).astype(np.int32).reshape(B, pps)).to(device)
    q = normal((B, Hq, d), base + 0, dtype, device)
    kp = normal((B * pps, page, Hkv, d), base + 1, dtype, device)
    vp = normal((B * pps, page, Hkv, d), base + 2, dtype, device)
    seq = torch.full((B,), L, dtype=torch.int32, device=device)
    return q, kp, vp, table, seq


def to_bits(t: torch.Tensor) -> np.ndarray:
    """16-bit tensor -> host numpy uint16 bit patterns (what the oracle reads)."""
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("expected a 16-bit tensor")
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sample_rows(B, H, N, n, seed) -> np.ndarray:
    """n distinct (b, h, i) triples, uniform without replacement."""
    rng = np.random.default_rng(int(seed))
    total = B * H * N
    n = min(int(n), total)
    flat = rng.choice(total, size=n, replace=False)
    b, rem = np.divmod(flat, H * N)
    h, i = np.divmod(rem, N)
    return np.stack([b, h, i], axis=1).astype(np.int64)


def boundary_rows(B, H, N, seed, tiles=(16, 32, 64, 128, 256), n_random=64,
                  per_head=False) -> np.ndarray:
    """First, second, last rows, rows on both sides of tile boundaries (a few
    near the start and the end of the sequence for every tile size), plus
    n_random random rows; spread over heads and batches."""
    idx = {0, 1, N - 2, N - 1}
    for T in tiles:
        for kk in (1, 2, 3):
            for i in (kk * T - 1, kk * T, N - kk * T - 1, N - kk * T):
                idx.add(i)
        mid = (N // 2 // T) * T
        idx.update({mid - 1, mid})
    idx = sorted(i for i in idx if 0 <= i < N)
    rng = np.random.default_rng(int(seed))
    rows = []
    heads = [(b, h) for b in range(B) for h in range(H)]
    for n, i in enumerate(idx):
        if per_head:
            rows.extend((b, h, i) for b, h in heads)
        else:
            b, h = heads[n % len(heads)]
            rows.append((b, h, i))
    for _ in range(int(n_random)):
        rows.append((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(N))))
    return np.unique(np.asarray(rows, dtype=np.int64), axis=0)


# The five workloads (shapes, dtypes, masks, input recipes).
CONFIGS = {
    "tiny": dict(kind="fwd", B=1, H=2, N=128, d=64, dtype="bf16", causal=False, seed=1001),
    "fwd_b8h32n8k": dict(kind="fwd", B=8, H=32, N=8192, d=128, dtype="fp16", causal=False, seed=1002),
    "causal_b4h32n16k_kscaled": dict(kind="fwd", B=4, H=32, N=16384, d=128, dtype="bf16", causal=True,
                                     seed=1003, krow_scale=(0.5, 4.0)),
    "causal_b1h32n128k": dict(kind="fwd", B=1, H=32, N=131072, d=128, dtype="bf16", causal=True, seed=1004),
    "decode_b8hq32hkv8l32k": dict(kind="decode", B=8, Hq=32, Hkv=8, L=32768, d=128, dtype="bf16",
                                  nsplit=16, seed=1005),
}

# The workloads of bench.py's variable-length legs: one packed batch of
# mixed lengths with the forward shape's 65536 tokens, and the decode shape
# in 16-token pages.
VARLEN_BENCH = dict(lens=(16384, 12288, 9216, 8192, 7168, 6144, 4096, 2048), H=32, d=128,
                    dtype="fp16", causal=False, seed=1007)
PAGED_BENCH = dict(B=8, Hq=32, Hkv=8, L=32768, d=128, dtype="bf16", nsplit=16, page=16, seed=1008)
