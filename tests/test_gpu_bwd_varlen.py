"""fa_bwd_varlen through the C ABI on an MI355X: gradients of packed [T, H, d]
batches of variable-length sequences (o and lse from fa_fwd_varlen), against
the fp64 oracle's gradients of each sequence on its own.  Bar per gradient
tensor as for fa_bwd: rel-L2 <= 5e-3, max-abs <= 2e-2 * max |ref|."""
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
    print(f"case bwd_varlen lens={lens} H{H} d{d} {dtype} causal={causal}", flush=True)
    T = sum(lens)
    q, k, v, do = (synth.normal((T, H, d), seed * 16 + i, dtype, DEV) for i in range(4))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(d)
    ms = max_seqlen or max(lens)
    o, lse = fa.fwd_varlen(q, k, v, cu, ms, causal=causal, scale=scale)
    grads = fa.bwd_varlen(q, k, v, o, lse, do, cu, ms, causal=causal, scale=scale)
    torch.cuda.synchronize()
    got = [g.cpu().numpy() for g in grads]
    bits = [synth.to_bits(x) for x in (q, k, v, do)]
    ref = [np.zeros(got[0].shape) for _ in range(3)]
    start = 0
    for N in lens:
        if N:
            sl = slice(start, start + N)
            per = [np.ascontiguousarray(x[sl].transpose(1, 0, 2)[None]) for x in bits]
            r = orc.attention_bwd(*per, dtype, causal, scale)          # [1, H, N, d]
            for i, name in enumerate(("dq", "dk", "dv")):
                ref[i][sl] = r[name][0].transpose(1, 0, 2)
        start += N
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        bound = 2e-2 * float(np.abs(r).max())
        assert_close(g, r, what=f"bwd_varlen lens={lens} {dtype} causal={causal} {name}",
                     o_max_abs=bound, o_rel_l2=5e-3)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
def test_mixed_lengths(orc, causal, dtype, d):
    run(orc, [1, 17, 128, 300, 0, 700, 64, 257], 3, d, dtype, causal, seed=3100 + d)


def test_grid_larger_than_longest(orc):
    """max_seqlen above every length: the extra workgroups leave at once."""
    run(orc, [40, 513], 2, 128, "bf16", True, seed=3110, max_seqlen=2000)


def test_equal_lengths_match_dense():
    """All lengths equal: the packed call reproduces fa_bwd bit for bit."""
    B, H, N, d = 3, 4, 700, 128
    q, k, v, do = synth.bwd_inputs(B, H, N, d, "bf16", seed=3120, device=DEV)
    pack = lambda x: x.permute(0, 2, 1, 3).reshape(B * N, H, d).contiguous()
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device=DEV)
    for causal in (False, True):
        print(f"case bwd_varlen equal lengths causal={causal}", flush=True)
        o, lse = fa.fwd(q, k, v, causal=causal)
        dense = fa.bwd(q, k, v, o, lse, do, causal=causal)
        packed = fa.bwd_varlen(pack(q), pack(k), pack(v), pack(o),
                               lse.permute(1, 0, 2).reshape(H, B * N).contiguous(), pack(do), cu,
                               N, causal=causal)
        torch.cuda.synchronize()
        for a, b in zip(dense, packed):
            assert torch.equal(pack(a), b)
