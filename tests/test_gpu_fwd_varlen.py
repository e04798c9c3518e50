"""fa_fwd_varlen through the C ABI on an MI355X: packed [T, H, d] batches of
variable-length sequences, against the fp64 oracle run on each sequence."""
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


def run(orc, lens, H, d, dtype, causal, seed, max_seqlen=None):
    print(f"case fwd_varlen lens={lens} H{H} d{d} {dtype} causal={causal}", flush=True)
    T = sum(lens)
    q, k, v = (synth.normal((T, H, d), seed * 16 + i, dtype, DEV) for i in range(3))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(d)
    o, lse = fa.fwd_varlen(q, k, v, cu, max_seqlen or max(lens), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
    ro = np.zeros(o.shape, np.float64)
    rl = np.zeros(lse.shape, np.float64)
    start = 0
    for N in lens:
        if N:
            sl = slice(start, start + N)
            per = [np.ascontiguousarray(x[sl].transpose(1, 0, 2)[None]) for x in (qb, kb, vb)]
            rob, rlb = orc.attention(*per, dtype, causal, scale)        # [1, H, N, d], [1, H, N]
            ro[sl] = rob[0].transpose(1, 0, 2)
            rl[:, sl] = rlb[0]
        start += N
    return assert_close(o, ro, lse, rl, f"fwd_varlen lens={lens} {dtype} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
def test_mixed_lengths(orc, causal, dtype, d):
    run(orc, [1, 17, 128, 300, 0, 1000, 64, 257], 3, d, dtype, causal, seed=3000 + d)


def test_grid_larger_than_longest(orc):
    """max_seqlen above every length: the extra workgroups leave at once."""
    run(orc, [40, 513], 2, 128, "bf16", True, seed=3010, max_seqlen=2000)


def test_long_sequences(orc):
    run(orc, [4096, 1500, 8192], 4, 128, "fp16", False, seed=3011)


def test_equal_lengths_match_dense():
    """All lengths equal: the packed call reproduces fa_fwd bit for bit."""
    B, H, N, d = 3, 4, 700, 128
    q, k, v = synth.fwd_inputs(B, H, N, d, "bf16", seed=3020, device=DEV)
    for causal in (False, True):
        o_d, l_d = fa.fwd(q, k, v, causal=causal)
        pk = [x.permute(0, 2, 1, 3).reshape(B * N, H, d).contiguous() for x in (q, k, v)]
        cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device=DEV)
        o_p, l_p = fa.fwd_varlen(*pk, cu, N, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o_p, o_d.permute(0, 2, 1, 3).reshape(B * N, H, d))
        assert torch.equal(l_p, l_d.permute(1, 0, 2).reshape(H, B * N))


def test_bench_batch_sampled(orc):
    """The batch bench.py's varlen_fwd leg times (8 packed sequences, 65536
    tokens, H32 d128 fp16, the same launch): boundary and random rows of
    every sequence against the oracle run on that sequence alone."""
    c = synth.VARLEN_BENCH
    lens, H, d = c["lens"], c["H"], c["d"]
    print(f"case fwd_varlen bench batch lens={lens} H{H} d{d} {c['dtype']}", flush=True)
    q, k, v, cu = synth.varlen_inputs(lens, H, d, c["dtype"], seed=c["seed"], device=DEV)
    scale = 1 / math.sqrt(d)
    o, lse = fa.fwd_varlen(q, k, v, cu, max(lens), causal=c["causal"], scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
    del q, k, v
    got_o, got_l, ref_o, ref_l = [], [], [], []
    start = 0
    for n, L in enumerate(lens):
        rows = synth.boundary_rows(1, H, L, seed=c["seed"] + n, tiles=(64, 128, 256), n_random=24)
        sl = slice(start, start + L)
        per = [np.ascontiguousarray(x[sl].transpose(1, 0, 2)[None]) for x in (qb, kb, vb)]
        ro, rl = orc.attention_rows(*per, c["dtype"], rows, c["causal"], scale)
        got_o.append(o[start + rows[:, 2], rows[:, 1]])
        got_l.append(lse[rows[:, 1], start + rows[:, 2]])
        ref_o.append(ro)
        ref_l.append(rl)
        start += L
    assert_close(np.concatenate(got_o), np.concatenate(ref_o), np.concatenate(got_l),
                 np.concatenate(ref_l), f"fwd_varlen bench batch {sum(len(x) for x in got_o)} rows")
