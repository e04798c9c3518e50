"""fa_bwd through the C ABI on an MI355X, against the fp64 oracle's gradients.

The forward that feeds the backward (O, lse) is this library's fa_fwd on the
same inputs, as a training step would run it.  Bar per gradient tensor:
rel-L2 <= 5e-3 and max |g - g_ref| <= 2e-2 * max |g_ref| (the weights P and
dS are rounded to the 16-bit storage type for their products, a relative
error of at most 2^-8 for bf16 and 2^-11 for fp16 per element (round to
nearest with 8 and 11 significant bits), accumulated in fp32).
"""
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
GRAD_REL_L2 = 5e-3
GRAD_MAX_ABS_REL = 2e-2


@pytest.fixture(scope="module")
def orc():
    return oracle_mod.get()


def check_grads(got, ref, what):
    top = max(float(np.abs(np.asarray(ref[n])).max()) for n in ("dq", "dk", "dv"))
    for name in ("dq", "dk", "dv"):
        g = np.asarray(got[name], np.float64)
        r = np.asarray(ref[name], np.float64)
        if not r.any():
            # Closed form zero (one visible key, or constant V): only fp32
            # rounding of dP - D remains; bound it by the largest gradient.
            assert np.isfinite(g).all(), (what, name)
            print(f"{what} {name}: reference is zero, max |g| {np.abs(g).max():.3e}", flush=True)
            assert np.abs(g).max() <= 1e-5 * top, (what, name, float(np.abs(g).max()))
            continue
        bound = GRAD_MAX_ABS_REL * float(np.abs(r).max())
        assert_close(g, r, what=f"{what} {name}", o_max_abs=bound, o_rel_l2=GRAD_REL_L2)


def gpu_grads(q, k, v, do, causal, scale):
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def run_full(orc, B, H, N, d, dtype, causal, seed, scale=None):
    what = f"bwd B{B} H{H} N{N} d{d} {dtype} causal={causal} scale={scale}"
    print(f"case {what} seed={seed}", flush=True)
    q, k, v, do = synth.bwd_inputs(B, H, N, d, dtype, seed=seed, device=DEV)
    scale = 1 / math.sqrt(d) if scale is None else scale
    dq, dk, dv = gpu_grads(q, k, v, do, causal, scale)
    got = {"dq": dq.cpu().numpy(), "dk": dk.cpu().numpy(), "dv": dv.cpu().numpy()}
    ref = orc.attention_bwd(*(synth.to_bits(t) for t in (q, k, v, do)), dtype, causal, scale)
    check_grads(got, ref, what)


@pytest.mark.parametrize("B,H,N,d,dtype,causal", [
    (1, 2, 300, 128, "bf16", False),   # several 128-row tiles, ragged tail
    (1, 2, 300, 128, "fp16", True),
    (2, 1, 257, 64, "bf16", True),
    (1, 2, 200, 64, "fp16", False),
    (1, 1, 128, 128, "bf16", True),    # exactly one workgroup tile
    (1, 1, 64, 128, "fp16", False),    # exactly one streamed tile
    (1, 3, 33, 128, "bf16", False),    # shorter than a tile
    (1, 1, 1, 64, "fp16", True),       # one key: dQ = dK = 0, dV = dO
    (1, 1, 1, 128, "bf16", False),
])
def test_small_shapes(orc, B, H, N, d, dtype, causal):
    run_full(orc, B, H, N, d, dtype, causal, seed=2000 + N)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.5])
def test_scale_values(orc, scale):
    run_full(orc, 1, 2, 150, 64, "fp16", True, seed=2100, scale=scale)
    run_full(orc, 1, 1, 190, 128, "bf16", False, seed=2101, scale=scale)


def test_key_scaled_causal(orc):
    """Key rows scaled by U[0.5, 4] (peaked softmax rows), causal, bf16."""
    print("case bwd key-scaled causal B1 H2 N384 d128 bf16", flush=True)
    B, H, N, d = 1, 2, 384, 128
    q, k, v = synth.fwd_inputs(B, H, N, d, "bf16", seed=2200, device=DEV, krow_scale=(0.5, 4.0))
    do = synth.normal((B, H, N, d), 2200 * 16 + 4, "bf16", DEV)
    scale = 1 / math.sqrt(d)
    dq, dk, dv = gpu_grads(q, k, v, do, True, scale)
    got = {"dq": dq.cpu().numpy(), "dk": dk.cpu().numpy(), "dv": dv.cpu().numpy()}
    ref = orc.attention_bwd(*(synth.to_bits(t) for t in (q, k, v, do)), "bf16", True, scale)
    check_grads(got, ref, "bwd key-scaled causal")


def run_sampled(orc, B, H, N, d, dtype, causal, seed, heads, per_head=12):
    what = f"bwd sampled B{B} H{H} N{N} d{d} {dtype} causal={causal}"
    print(f"case {what} seed={seed}", flush=True)
    q, k, v, do = synth.bwd_inputs(B, H, N, d, dtype, seed=seed, device=DEV)
    scale = 1 / math.sqrt(d)
    dq, dk, dv = gpu_grads(q, k, v, do, causal, scale)
    # Rows: first, last, tile boundaries and seeded random rows of each head.
    g = np.random.default_rng(seed)
    sel = []
    for (b, h) in heads:
        idx = {0, N - 1, 127, 128, N // 2, N - 129}
        idx |= set(g.integers(0, N, per_head - len(idx)).tolist())
        sel += [(b, h, i) for i in sorted(idx) if 0 <= i < N]
    sel = np.array(sel, np.int64)
    r = torch.as_tensor(sel)
    got = {"dq": dq[r[:, 0], r[:, 1], r[:, 2]].cpu().numpy(),
           "dk": dk[r[:, 0], r[:, 1], r[:, 2]].cpu().numpy(),
           "dv": dv[r[:, 0], r[:, 1], r[:, 2]].cpu().numpy()}
    # Properties over every head: sum_j dV_j = sum_i dO_i (each query's
    # weights sum to one) and sum_j dK_j = 0 (each row of dS sums to zero).
    sdv = dv.double().sum(dim=2)
    sdo = do.double().sum(dim=2)
    err_v = (sdv - sdo).norm() / sdo.norm()
    rms_k = dk.double().pow(2).mean().sqrt()
    err_k = dk.double().sum(dim=2).norm() / (rms_k * math.sqrt(N) * math.sqrt(B * H * d))
    print(f"{what} sum dV vs sum dO rel {err_v.item():.2e}; |sum dK| / (sqrt(N) rms) {err_k.item():.2e}",
          flush=True)
    assert err_v.item() < 5e-3
    assert err_k.item() < 2e-2
    bits = [synth.to_bits(t) for t in (q, k, v, do)]
    del q, k, v, do, dq, dk, dv
    torch.cuda.empty_cache()
    ref = orc.attention_bwd(*bits, dtype, causal, scale, qrows=sel, kcols=sel)
    check_grads(got, ref, what)


def test_bench_shape_sampled(orc):
    run_sampled(orc, 8, 32, 8192, 128, "fp16", False, seed=2300, heads=[(3, 17), (7, 31)])


def test_bench_shape_causal_sampled(orc):
    run_sampled(orc, 8, 32, 8192, 128, "bf16", True, seed=2301, heads=[(0, 0), (5, 9)])


def test_long_single_head_causal(orc):
    """One causal head of 2^21 tokens (512 MiB per 16-bit tensor): 32-bit
    buffer offsets near their range.  dQ on sampled rows against the oracle;
    dK and dV through properties that hold at any size."""
    B, H, N, d = 1, 1, 1 << 21, 128
    print(f"case bwd long causal B{B} H{H} N{N} d{d} bf16", flush=True)
    q, k, v, do = synth.bwd_inputs(B, H, N, d, "bf16", seed=2600, device=DEV)
    scale = 1 / math.sqrt(d)
    dq, dk, dv = gpu_grads(q, k, v, do, True, scale)
    rows = [0, 1, 63, 64, 127, 128, 4095, 4096, N // 2, N - 129, N - 128, N - 2, N - 1]
    sel = np.array([(0, 0, i) for i in rows], np.int64)
    got = dq[0, 0, torch.as_tensor(rows)].cpu().numpy()
    sdv = dv.double().sum(dim=2)
    sdo = do.double().sum(dim=2)
    err_v = ((sdv - sdo).norm() / sdo.norm()).item()
    err_k = (dk.double().sum(dim=2).norm() /
             (dk.double().pow(2).mean().sqrt() * math.sqrt(N) * math.sqrt(d))).item()
    print(f"long causal: sum dV vs sum dO rel {err_v:.2e}; |sum dK| / (sqrt(N) rms) {err_k:.2e}",
          flush=True)
    assert err_v < 5e-3 and err_k < 2e-2
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
    bits = [synth.to_bits(t) for t in (q, k, v, do)]
    del q, k, v, do, dq, dk, dv
    torch.cuda.empty_cache()
    ref = orc.attention_bwd(*bits, "bf16", True, scale, qrows=sel, kcols=np.zeros((0, 3)))
    bound = GRAD_MAX_ABS_REL * float(np.abs(ref["dq"]).max())
    assert_close(got, ref["dq"], what="bwd long causal dq rows", o_max_abs=bound,
                 o_rel_l2=GRAD_REL_L2)


def test_deterministic(orc):
    """No atomics: two runs give bitwise identical gradients."""
    print("case bwd determinism B2 H4 N1000 d128 bf16 causal", flush=True)
    q, k, v, do = synth.bwd_inputs(2, 4, 1000, 128, "bf16", seed=2400, device=DEV)
    a = gpu_grads(q, k, v, do, True, 0.1)
    b = gpu_grads(q, k, v, do, True, 0.1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_workspace_reuse(orc):
    """One workspace serves a call and then a smaller one."""
    print("case bwd workspace reuse", flush=True)
    ws = torch.empty(fa.bwd_workspace_bytes(1, 2, 700), dtype=torch.uint8, device=DEV)
    for N, seed in ((700, 2500), (333, 2501)):
        q, k, v, do = synth.bwd_inputs(1, 2, N, 64, "fp16", seed=seed, device=DEV)
        o, lse = fa.fwd(q, k, v, causal=False)
        dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=False, workspace=ws)
        dq2, dk2, dv2 = fa.bwd(q, k, v, o, lse, do, causal=False)
        torch.cuda.synchronize()
        for x, y in ((dq, dq2), (dk, dk2), (dv, dv2)):
            assert torch.equal(x, y)
    ref = orc.attention_bwd(*(synth.to_bits(t) for t in (q, k, v, do)), "fp16", False,
                            1 / math.sqrt(64))
    check_grads({"dq": dq.cpu().numpy(), "dk": dk.cpu().numpy(), "dv": dv.cpu().numpy()}, ref,
                "bwd workspace reuse")
