"""Every entry point enqueues its work on the caller's stream.

On a side stream (default priority) the inputs are first copied into fresh
buffers, then the library is called on that stream and only that stream is
synchronised: work placed on any other stream could read the inputs before
the copies land.  Results must equal the same call on the default stream bit
for bit (the kernels are deterministic).
"""
import math

import numpy as np
import pytest
import torch

import flashattention_attention_fa_amd as fa
from flashattention_attention_fa_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def on_side_stream(fn, inputs):
    """Copy `inputs` on a fresh stream, run fn(copies, stream) there, wait
    for that stream only; returns fn's outputs."""
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(s):
        copies = [torch.empty_like(x) for x in inputs]
        for c, x in zip(copies, inputs):
            c.copy_(x, non_blocking=True)
        out = fn(copies, s)
    s.synchronize()
    return out


def same(a, b):
    a = a if isinstance(a, (tuple, list)) else (a,)
    b = b if isinstance(b, (tuple, list)) else (b,)
    for x, y in zip(a, b):
        if x is None and y is None:
            continue
        assert torch.equal(x, y)


def test_fwd_and_bwd_on_side_stream():
    print("case streams fwd/bwd B2 H4 N2000 d128 bf16", flush=True)
    q, k, v, do = synth.bwd_inputs(2, 4, 2000, 128, "bf16", seed=4000, device=DEV)
    ref_o, ref_l = fa.fwd(q, k, v, causal=True)
    ref_g = fa.bwd(q, k, v, ref_o, ref_l, do, causal=True)
    torch.cuda.synchronize()
    o, l = on_side_stream(lambda c, s: fa.fwd(c[0], c[1], c[2], causal=True, stream=s), [q, k, v])
    same((o, l), (ref_o, ref_l))
    g = on_side_stream(lambda c, s: fa.bwd(c[0], c[1], c[2], c[3], c[4], c[5], causal=True,
                                           stream=s), [q, k, v, ref_o, ref_l, do])
    same(g, ref_g)


def test_varlen_on_side_stream():
    print("case streams varlen", flush=True)
    lens = [100, 0, 777, 64]
    T, H, d = sum(lens), 2, 64
    q, k, v, do = (synth.normal((T, H, d), 4100 + i, "fp16", DEV) for i in range(4))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    ref_o, ref_l = fa.fwd_varlen(q, k, v, cu, max(lens), causal=False)
    ref_g = fa.bwd_varlen(q, k, v, ref_o, ref_l, do, cu, max(lens))
    torch.cuda.synchronize()
    o, l = on_side_stream(lambda c, s: fa.fwd_varlen(c[0], c[1], c[2], c[3], max(lens), stream=s),
                          [q, k, v, cu])
    same((o, l), (ref_o, ref_l))
    g = on_side_stream(lambda c, s: fa.bwd_varlen(c[0], c[1], c[2], c[3], c[4], c[5], c[6],
                                                  max(lens), stream=s),
                       [q, k, v, ref_o, ref_l, do, cu])
    same(g, ref_g)


def test_fp8_on_side_stream():
    print("case streams fp8", flush=True)
    q, k, v, ds = synth.fp8_inputs(1, 4, 1500, 128, seed=4200, device=DEV)
    kw = dict(q_descale=ds, k_descale=ds, v_descale=ds, causal=True)
    ref = fa.fwd_fp8(q, k, v, **kw)
    torch.cuda.synchronize()
    out = on_side_stream(lambda c, s: fa.fwd_fp8(c[0], c[1], c[2], stream=s, **kw), [q, k, v])
    same(out, ref)


def test_decode_on_side_stream():
    print("case streams decode", flush=True)
    q, kc, vc = synth.decode_inputs(4, 16, 2, 3000, 128, "bf16", seed=4300, device=DEV)
    ref_lib = fa.decode(q, kc, vc, nsplit=8)
    ref_ex = fa.decode(q, kc, vc, nsplit=8, return_lse=True)
    torch.cuda.synchronize()
    same(on_side_stream(lambda c, s: fa.decode(c[0], c[1], c[2], nsplit=8, stream=s), [q, kc, vc]),
         ref_lib)
    same(on_side_stream(lambda c, s: fa.decode(c[0], c[1], c[2], nsplit=8, return_lse=True,
                                               stream=s), [q, kc, vc]), ref_ex)


def test_decode_paged_on_side_stream():
    print("case streams paged decode", flush=True)
    B, Hq, Hkv, d, page, pps = 3, 8, 2, 128, 32, 20
    num_pages = B * pps
    kp = synth.normal((num_pages, page, Hkv, d), 4400, "fp16", DEV)
    vp = synth.normal((num_pages, page, Hkv, d), 4401, "fp16", DEV)
    q = synth.normal((B, Hq, d), 4402, "fp16", DEV)
    g = torch.Generator(device=DEV).manual_seed(4403)
    table = torch.randperm(num_pages, generator=g, device=DEV).to(torch.int32).reshape(B, pps)
    lens = torch.tensor([1, 333, page * pps], dtype=torch.int32, device=DEV)
    ref = fa.decode_paged(q, kp, vp, table, lens, nsplit=4)
    torch.cuda.synchronize()
    out = on_side_stream(lambda c, s: fa.decode_paged(c[0], c[1], c[2], c[3], c[4], nsplit=4,
                                                      stream=s), [q, kp, vp, table, lens])
    same(out, ref)


def test_stream_argument_outside_its_context():
    """stream= given while torch's current stream is another one: the binding
    must allocate its workspace and outputs on the launch stream.  Right after
    each call the current stream allocates same-sized buffers and overwrites
    them; if the binding had freed its workspace into the current stream's
    pool, those writes would land in it while the kernels still use it."""
    print("case streams: stream argument without entering its context", flush=True)
    q, kc, vc = synth.decode_inputs(8, 32, 8, 16384, 128, "bf16", seed=4500, device=DEV)
    ref = fa.decode(q, kc, vc, nsplit=16, return_lse=True)
    qb, kb, vb, do = synth.bwd_inputs(2, 8, 1024, 128, "bf16", seed=4501, device=DEV)
    o, lse = fa.fwd(qb, kb, vb)
    ref_g = fa.bwd(qb, kb, vb, o, lse, do)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=DEV)
    dec_ws = fa.decode_workspace_bytes(8, 32, 128, 16)
    bwd_ws = fa.bwd_workspace_bytes(2, 8, 1024)
    for _ in range(3):
        out = fa.decode(q, kc, vc, nsplit=16, return_lse=True, stream=s)
        junk = [torch.empty(dec_ws, dtype=torch.uint8, device=DEV).fill_(0x7f) for _ in range(4)]
        g = fa.bwd(qb, kb, vb, o, lse, do, stream=s)
        junk += [torch.empty(bwd_ws, dtype=torch.uint8, device=DEV).fill_(0x7f) for _ in range(4)]
        s.synchronize()
        torch.cuda.synchronize()
        same(out, ref)
        same(g, ref_g)
        del junk


def test_binding_rejects_bad_output_buffers():
    """Caller-supplied out/lse buffers are checked before any launch."""
    print("case binding rejects bad out/lse", flush=True)
    lens = [100, 28]
    q, k, v, cu = synth.varlen_inputs(lens, 2, 64, "bf16", seed=4600, device=DEV)
    T = sum(lens)
    with pytest.raises(ValueError):
        fa.fwd_varlen(q, k, v, cu, 100, out=torch.empty(T, 2, 64, device=DEV).half())
    with pytest.raises(ValueError):
        fa.fwd_varlen(q, k, v, cu, 100, lse=torch.empty(T, 2, device=DEV))      # must be [H, T]
    with pytest.raises(ValueError):
        fa.fwd_varlen(q, k, v, cu, 100, out=torch.empty(T, 2, 64))               # host memory
    qd, kc, vc = synth.decode_inputs(2, 4, 2, 50, 64, "bf16", seed=4601, device=DEV)
    with pytest.raises(ValueError):
        fa.decode(qd, kc, vc, nsplit=2, lse=torch.empty(2, 3, device=DEV))
    with pytest.raises(ValueError):
        fa.decode(qd, kc, vc, nsplit=2, out=torch.empty(2, 4, 64))
    with pytest.raises(ValueError):
        fa.decode_noalloc(qd, kc, vc, nsplit=2, out=torch.empty(2, 4, 32, device=DEV))
    kp = synth.normal((4, 16, 2, 64), 4602, "bf16", DEV)
    table = torch.zeros(2, 2, dtype=torch.int32, device=DEV)
    seq = torch.full((2,), 20, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        fa.decode_paged(qd, kp, kp, table, seq, nsplit=2, out=torch.empty(2, 4, 65, device=DEV))
    with pytest.raises(ValueError):
        fa.decode_paged(qd, kp, kp, table, seq, nsplit=2, lse=torch.empty(2, 4))
