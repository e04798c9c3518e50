"""fa_fwd through the C ABI on an MI355X, against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import flashattention_attention_fa_amd as fa
from flashattention_attention_fa_amd import synth
from oracle import oracle as oracle_mod
from parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def orc():
    return oracle_mod.get()


def run_full(orc, B, H, N, d, dtype, causal, seed, scale=None, **kw):
    print(f"case fwd B{B} H{H} N{N} d{d} {dtype} causal={causal} seed={seed}", flush=True)
    q, k, v = synth.fwd_inputs(B, H, N, d, dtype, seed=seed, device=DEV, **kw)
    scale = 1 / math.sqrt(d) if scale is None else scale
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = orc.attention(synth.to_bits(q), synth.to_bits(k), synth.to_bits(v), dtype, causal, scale)
    return assert_close(o.cpu().numpy(), ro, lse.cpu().numpy(), rl,
                        f"fwd B{B} H{H} N{N} d{d} {dtype} causal={causal}")


def run_rows(orc, cfg, rows):
    c = dict(cfg)
    print(f"case fwd {c}", flush=True)
    q, k, v = synth.fwd_inputs(c["B"], c["H"], c["N"], c["d"], c["dtype"], seed=c["seed"],
                               device=DEV, krow_scale=c.get("krow_scale"))
    scale = 1 / math.sqrt(c["d"])
    o, lse = fa.fwd(q, k, v, causal=c["causal"], scale=scale)
    torch.cuda.synchronize()
    r = torch.as_tensor(rows)
    og = o[r[:, 0], r[:, 1], r[:, 2]].cpu().numpy()
    lg = lse[r[:, 0], r[:, 1], r[:, 2]].cpu().numpy()
    del o, lse
    qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
    del q, k, v
    torch.cuda.empty_cache()
    ro, rl = orc.attention_rows(qb, kb, vb, c["dtype"], rows, c["causal"], scale)
    return assert_close(og, ro, lg, rl, f"fwd sampled {len(rows)} rows")


# -- the workloads --------------------------------------------------------------

def test_tiny_config(orc):
    c = synth.CONFIGS["tiny"]
    run_full(orc, c["B"], c["H"], c["N"], c["d"], c["dtype"], False, c["seed"])
    run_full(orc, c["B"], c["H"], c["N"], c["d"], c["dtype"], True, c["seed"])


def test_bench_shape_sampled(orc):
    c = synth.CONFIGS["fwd_b8h32n8k"]
    rows = synth.sample_rows(c["B"], c["H"], c["N"], 256, seed=c["seed"])
    run_rows(orc, c, rows)


def test_causal_kscaled_sampled(orc):
    c = synth.CONFIGS["causal_b4h32n16k_kscaled"]
    rows = synth.boundary_rows(c["B"], c["H"], c["N"], seed=c["seed"], n_random=96)
    run_rows(orc, c, rows)


def test_causal_kscaled_full_heads(orc):
    """Eight complete heads (131072 rows, every row of each) of the key-scaled
    causal workload: the workload whose rows are the most peaked (a few keys
    scaled up to 4x dominate them), so the rounding of a dominant weight
    shows here first.  Heads spread over all four batches."""
    c = synth.CONFIGS["causal_b4h32n16k_kscaled"]
    heads = [(0, 5), (0, 11), (0, 24), (1, 0), (1, 17), (2, 9), (2, 30), (3, 21)]
    N = c["N"]
    rows = np.concatenate([np.stack([np.full(N, b), np.full(N, h), np.arange(N)], 1)
                           for b, h in heads]).astype(np.int64)
    run_rows(orc, c, rows)


def test_long_causal_sampled(orc):
    c = synth.CONFIGS["causal_b1h32n128k"]
    rows = synth.boundary_rows(c["B"], c["H"], c["N"], seed=c["seed"], n_random=64)
    run_rows(orc, c, rows)


def test_long_single_head_causal(orc):
    """A 2M-token head: per-head offsets past 2^29 bytes, 32768 key tiles."""
    c = dict(B=1, H=1, N=1 << 21, d=128, dtype="bf16", causal=True, seed=1006)
    rows = synth.boundary_rows(1, 1, c["N"], seed=c["seed"], tiles=(64, 128, 256), n_random=8)
    run_rows(orc, c, rows)


# -- several tiles with ragged tails, both dtypes and head dims ---------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_multi_tile(orc, dtype, causal, d):
    run_full(orc, 2, 3, 333, d, dtype, causal, seed=40 + d)


@pytest.mark.parametrize("N", [1, 2, 31, 63, 64, 65, 127, 128, 129, 191, 257])
@pytest.mark.parametrize("causal", [False, True])
def test_lengths(orc, N, causal):
    run_full(orc, 1, 2, N, 128, "bf16", causal, seed=N)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale_mul", [1.0, 8.0])
def test_running_max_raised_mid_row(orc, dtype, causal, scale_mul):
    """Keys whose norm grows 8x along the sequence: later key tiles beat the
    first tile's maximum by far more than 10 (log2 units), so the kernel must
    raise its running max mid-row (rescaling O and l) on many tiles."""
    B, H, N, d = 1, 2, 1024, 128
    print(f"case fwd ramped keys {dtype} causal={causal} scale x{scale_mul}", flush=True)
    q, k, v = synth.fwd_inputs(B, H, N, d, dtype, seed=77, device=DEV)
    ramp = torch.linspace(1.0, 8.0, N, device=DEV)[None, None, :, None]
    k = (k.float() * ramp).to(k.dtype)
    scale = scale_mul / math.sqrt(d)
    # The input property the test relies on, checked in fp64 on the CPU.
    qc, kc = q.double().cpu(), k.double().cpu()
    s = scale * math.log2(math.e) * (qc @ kc.transpose(-1, -2).contiguous())
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    gap = (s[..., 64:].amax(-1) - s[..., :64].amax(-1))[..., 64:]
    assert (gap > 10).float().mean() > 0.5, gap.median()
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = orc.attention(synth.to_bits(q), synth.to_bits(k), synth.to_bits(v), dtype, causal,
                           scale)
    assert_close(o.cpu().numpy(), ro, lse.cpu().numpy(), rl, f"ramped keys {dtype} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_dominant_weight_rounding_cancels(orc, causal):
    """bf16: one key of the second tile outweighs the first tile's 64 keys
    8-13 times over, with weights between 2^9 and 2^10 relative to the
    running max (below the kernel's bound for raising it), so the kernel keeps them and
    rounds each to bf16 for the PV product, off by up to 2^-8 of itself.
    Dividing by the rounded weights of such a tile cancels most of it: with
    w the key's weight and L = 64 + w the row sum, O's error is at most
    2^-8 (w/L)(64/L) max|v_64 - mean(v_0..63)|, where dividing by the exact
    sum would leave 2^-8 (w/L)|v_64|."""
    N, d = 128, 128
    print(f"case fwd dominant bf16 weight causal={causal}", flush=True)
    g = torch.Generator().manual_seed(91)
    a = torch.linspace(0.9, 1.05, N).to(torch.bfloat16)           # query i: a_i e_0
    q = torch.zeros(1, 1, N, d, dtype=torch.bfloat16)
    q[0, 0, :, 0] = a
    k = torch.zeros(1, 1, N, d, dtype=torch.bfloat16)               # tile 0: scores 0
    k[0, 0, 64, 0] = 6.4375                                          # the dominant key
    k[0, 0, 65:, 0] = -20.0                                          # the rest of tile 1: ~0
    v = torch.randn(1, 1, N, d, generator=g).to(torch.bfloat16)
    v[0, 0, 64] = 4.0 * torch.sign(torch.randn(d, generator=g)).to(torch.bfloat16)
    o, lse = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=1.0)
    torch.cuda.synchronize()
    ro, rl = orc.attention(synth.to_bits(q), synth.to_bits(k), synth.to_bits(v), "bf16", causal, 1.0)
    og = o.cpu().numpy()
    assert_close(og, ro, lse.cpu().numpy(), rl, f"dominant bf16 weight causal={causal}")
    # rows that see the dominant key
    rows = np.arange(64, N)
    w = np.exp2(a[rows].double().numpy() * 6.4375 * math.log2(math.e))
    assert w.min() > 256 and w.max() < 1024
    L = 64.0 + w
    vd = v[0, 0, 64].double().numpy()
    spread = np.abs(vd - v[0, 0, :64].double().numpy().mean(0)).max()
    bound = 2.0 ** -8 * (w / L) * (64.0 / L) * spread + 1e-5
    err = np.abs(og[0, 0, rows] - ro[0, 0, rows]).max(1)
    assert (err <= bound).all(), (err / bound).max()
    # dividing by the exact sum would leave (w~ - w) v_64 / L: far above the bound
    wr = torch.tensor(w).float().to(torch.bfloat16).double().numpy()
    uncorrected = np.abs(wr - w) * np.abs(vd).max() / L
    assert uncorrected.max() > 3 * bound.max()


def test_single_key_returns_v(orc):
    q, k, v = synth.fwd_inputs(2, 4, 1, 128, "bf16", seed=3, device=DEV)
    o, lse = fa.fwd(q, k, v, scale=0.1)
    torch.cuda.synchronize()
    # P is rounded to 16 bits while l sums the fp32 weights: O = V within 1 ulp-ish
    np.testing.assert_allclose(o[:, :, 0].cpu().numpy(), v[:, :, 0].float().cpu().numpy(),
                               rtol=1e-6, atol=1e-6)
    ref = 0.1 * (q.double() * k.double()).sum(-1)
    np.testing.assert_allclose(lse.cpu().numpy(), ref.cpu().numpy(), atol=1e-3)


def test_causal_row0_and_uniform(orc):
    N = 300
    _, k, v = synth.fwd_inputs(1, 2, N, 128, "fp16", seed=5, device=DEV)
    q = torch.zeros_like(k)
    o, lse = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    vf = v.double()
    mean = torch.cumsum(vf, dim=2) / torch.arange(1, N + 1, device=DEV, dtype=torch.float64)[:, None]
    np.testing.assert_allclose(o.cpu().numpy(), mean.cpu().numpy(), atol=2e-3, rtol=0)
    np.testing.assert_allclose(lse.cpu().numpy()[0, 0], np.log(np.arange(1, N + 1)), atol=1e-4)
    np.testing.assert_allclose(o[:, :, 0].cpu().numpy(), v[:, :, 0].float().cpu().numpy(),
                               rtol=1e-6, atol=1e-6)


def test_constant_v(orc):
    q, k, _ = synth.fwd_inputs(1, 2, 200, 64, "bf16", seed=6, device=DEV)
    v = torch.full_like(q, 1.5)
    for causal in (False, True):
        o, _ = fa.fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert (o - 1.5).abs().max().item() < 1e-2


def test_scale_sign_and_zero(orc):
    for scale in (-0.2, 0.0, 0.5):
        run_full(orc, 1, 2, 150, 128, "bf16", True, seed=8, scale=scale)


def test_lse_optional_and_deterministic(orc):
    q, k, v = synth.fwd_inputs(2, 2, 500, 128, "fp16", seed=9, device=DEV)
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k, v, causal=True, return_lse=False)
    o3, l3 = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert l2 is None
    assert torch.equal(o1, o2) and torch.equal(o1, o3) and torch.equal(l1, l3)


def test_empty_batch_is_noop():
    q = torch.empty(0, 2, 16, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = fa.fwd(q, q, q)
    assert o.numel() == 0 and lse.numel() == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_score_dot_products_keep_fp32_range(dtype):
    """One key per head (N = 1, scale 1: lse = q.k).  A product 2^16 next to
    127 products of 2^-6 in the same group of dims: the exact sum
    65536 + 127/64 is representable in fp32, and the 16-bit matrix cores keep
    it (products 22 binades below the largest survive), unlike the FP8 form,
    which drops products 14 binades down; the 1e-3 lse bar of the 16-bit
    path rests on this."""
    H = 8
    q = torch.ones(1, H, 1, 128)
    k = torch.full((1, H, 1, 128), 2.0 ** -6)
    for h in range(H):
        q[0, h, 0, 8 * h % 128] = 256.0
        k[0, h, 0, 8 * h % 128] = 256.0
    t = torch.bfloat16 if dtype == "bf16" else torch.float16
    assert torch.equal(q.to(t).float(), q) and torch.equal(k.to(t).float(), k)
    print(f"case fwd score range {dtype}", flush=True)
    _, lse = fa.fwd(q.to(t).to(DEV), k.to(t).to(DEV), q.to(t).to(DEV), scale=1.0)
    torch.cuda.synchronize()
    exact = 65536.0 + 127 / 64
    # fp32 rounding of c*s and of the final product: a few ulp of 9.5e4
    np.testing.assert_allclose(lse.cpu().double().numpy(), exact, rtol=0, atol=0.05)
