"""fa_decode_noalloc through the C ABI: the entry point for callers that
cannot allocate (its partials live in the library's fixed per-device
buffer).  Two calls in a row, the second smaller, each against fa_decode_ex
with a caller-owned workspace on the same inputs: the kernels and the shard
partition are the same, so the results must match bit for bit (which is
tighter than the oracle bar both already meet)."""
import pytest
import torch

import flashattention_attention_fa_amd as fa
from flashattention_attention_fa_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(B, Hq, Hkv, L, d, dtype, nsplit, seed):
    print(f"case decode_noalloc B{B} Hq{Hq} Hkv{Hkv} L{L} d{d} {dtype} nsplit{nsplit}", flush=True)
    q, kc, vc = synth.decode_inputs(B, Hq, Hkv, L, d, dtype, seed=seed, device=DEV)
    ref_o, ref_l = fa.decode(q, kc, vc, nsplit=nsplit, return_lse=True)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    fa.decode_noalloc(q, kc, vc, nsplit=nsplit, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o)
    assert torch.equal(lse, ref_l)
    return out


def test_noalloc_two_calls_second_smaller():
    # the decode workload's shape, then a smaller call whose partials occupy
    # only the front of the buffer the first call filled
    _case(8, 32, 8, 32768, 128, "bf16", 16, seed=5100)
    _case(2, 8, 2, 1000, 64, "fp16", 7, seed=5101)


def test_noalloc_without_lse_and_clamped_shards():
    _case(3, 4, 4, 5, 128, "bf16", 64, seed=5102)          # nsplit clamped to L = 5
    out = torch.empty(1, 4, 128, device=DEV)
    q, kc, vc = synth.decode_inputs(1, 4, 1, 300, 128, "bf16", seed=5103, device=DEV)
    fa.decode_noalloc(q, kc, vc, nsplit=3, out=out)
    ref, _ = fa.decode(q, kc, vc, nsplit=3, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_noalloc_rejects_partials_beyond_its_buffer():
    q, kc, vc = synth.decode_inputs(8, 32, 8, 4096, 128, "bf16", seed=5104, device=DEV)
    out = torch.empty(8, 32, 128, device=DEV)
    assert fa.decode_workspace_bytes(8, 32, 128, 64) > fa.DECODE_NOALLOC_MAX_BYTES
    with pytest.raises(fa.FAError):
        fa.decode_noalloc(q, kc, vc, nsplit=64, out=out)
