"""Pins for the fp64 oracle: each checks it against something other than
itself (closed forms, hand-worked examples, invariants, a library routine,
pure-Python brute force).  A final test builds deliberately broken oracles
and checks that every planted mistake is caught by at least one pin.

Runs on the CPU only.
"""
import math
import re
from pathlib import Path

import numpy as np
import pytest
import torch

from flashattention_attention_fa_amd import synth
from oracle import oracle as oracle_mod

GOLDEN = Path(__file__).parent / "golden" / "worked_examples.txt"


def bits_of(values, dtype):
    t = torch.as_tensor(np.array(values, dtype=np.float32)).to(synth.TORCH_DTYPES[dtype])
    return synth.to_bits(t)


def widened(bits, dtype):
    """Library widening (torch), used only to build expected values."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(synth.TORCH_DTYPES[dtype])
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# pins: functions of an Oracle instance, so the mutation test can reuse them
# ---------------------------------------------------------------------------

def pin_widen_all_patterns(orc):
    """Every one of the 65536 bf16 and 65536 fp16 bit patterns widens to the
    value torch gives (NaN patterns to a NaN; signed zeros keep their sign)."""
    allbits = np.arange(65536, dtype=np.uint16)
    for dtype in ("bf16", "fp16"):
        ref = widened(allbits, dtype)
        got = orc.widen_many(allbits, dtype)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), dtype
        assert np.array_equal(got[~nan], ref[~nan]), dtype
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), dtype


def _parse_golden():
    blocks, cur = [], None
    for line in GOLDEN.read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, val = line.partition(":")
        val = val.strip()
        if key == "example":
            cur = {"name": val, "o": {}, "lse": {}}
            blocks.append(cur)
        elif key in ("q", "k", "v"):
            cur[key] = [[float(x) for x in row.split()] for row in val.split("|")]
        elif key in ("scale",):
            cur[key] = float(val)
        elif key == "causal":
            cur[key] = bool(int(val))
        else:
            m = re.fullmatch(r"expect_(o|lse)\[(\d+)\]", key)
            assert m, key
            exprs = [e.strip() for e in val.split(";")]
            env = {"math": math, "__builtins__": {}}
            vals = [eval(e, env) for e in exprs]  # closed forms over math.* only
            cur[m.group(1)][int(m.group(2))] = vals
    return blocks


def pin_worked_examples(orc):
    for ex in _parse_golden():
        for dtype in ("bf16", "fp16"):
            q = bits_of(ex["q"], dtype)[None, None]
            k = bits_of(ex["k"], dtype)[None, None]
            v = bits_of(ex["v"], dtype)[None, None]
            o, lse = orc.attention(q, k, v, dtype, ex["causal"], ex["scale"])
            for i, want in ex["o"].items():
                np.testing.assert_allclose(o[0, 0, i], want, rtol=1e-13, atol=1e-13,
                                           err_msg=ex["name"])
            for i, want in ex["lse"].items():
                np.testing.assert_allclose(lse[0, 0, i], want[0], rtol=1e-13, atol=1e-13,
                                           err_msg=ex["name"])


def pin_single_key(orc):
    """One key: softmax over a single element is 1, so O = v0 and
    lse = scale * <q, k0>."""
    for dtype in ("bf16", "fp16"):
        q, k, v = synth.fwd_inputs(2, 3, 1, 64, dtype, seed=11)
        qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
        scale = 0.125
        o, lse = orc.attention(qb, kb, vb, dtype, False, scale)
        np.testing.assert_array_equal(o[:, :, 0], widened(vb, dtype)[:, :, 0])
        dots = np.einsum("bhd,bhd->bh", widened(qb, dtype)[:, :, 0], widened(kb, dtype)[:, :, 0])
        np.testing.assert_allclose(lse[:, :, 0], scale * dots, rtol=1e-12, atol=1e-12)


def pin_causal_row0(orc):
    """Causal: query 0 sees only key 0, on any length."""
    q, k, v = synth.fwd_inputs(1, 2, 37, 32, "bf16", seed=12)
    qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
    o, lse = orc.attention(qb, kb, vb, "bf16", True, 0.3)
    np.testing.assert_array_equal(o[:, :, 0], widened(vb, "bf16")[:, :, 0])
    dots = np.einsum("bhd,bhd->bh", widened(qb, "bf16")[:, :, 0], widened(kb, "bf16")[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * dots, rtol=1e-12, atol=1e-12)


def pin_uniform_when_q_zero(orc):
    """Q = 0 makes every visible score 0: O_i is the mean of the visible V
    rows and lse_i = log(#visible) (log N non-causal, log(i+1) causal)."""
    N, d = 45, 16
    _, k, v = synth.fwd_inputs(2, 2, N, d, "fp16", seed=13)
    qb = np.zeros((2, 2, N, d), np.uint16)
    kb, vb = synth.to_bits(k), synth.to_bits(v)
    vw = widened(vb, "fp16")
    for causal in (False, True):
        o, lse = orc.attention(qb, kb, vb, "fp16", causal, 0.7)
        for i in (0, 1, 17, N - 1):
            n = i + 1 if causal else N
            np.testing.assert_allclose(o[:, :, i], vw[:, :, :n].mean(axis=2), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[:, :, i], math.log(n), rtol=1e-13, atol=1e-13)


def pin_constant_v(orc):
    """Every V row equal to c gives O = c whatever the weights."""
    q, k, _ = synth.fwd_inputs(1, 2, 50, 8, "bf16", seed=14)
    c = np.array([1.5, -2.0, 0.25, 3.0, 0.0, -0.5, 8.0, 1.0], np.float32)
    vb = bits_of(np.broadcast_to(c, (1, 2, 50, 8)), "bf16")
    for causal in (False, True):
        o, _ = orc.attention(synth.to_bits(q), synth.to_bits(k), vb, "bf16", causal, 0.9)
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=1e-12, atol=1e-12)


def pin_weights_sum_to_one(orc):
    """With V = identity (d = N), row i of O is the softmax weight vector of
    query i: non-negative, summing to 1, zero on keys a causal mask hides."""
    N = 24
    q, k, _ = synth.fwd_inputs(1, 1, N, N, "bf16", seed=15)
    vb = bits_of(np.eye(N)[None, None], "bf16")
    for causal in (False, True):
        o, _ = orc.attention(synth.to_bits(q), synth.to_bits(k), vb, "bf16", causal, 0.5)
        w = o[0, 0]
        assert (w >= 0).all()
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        if causal:
            assert np.all(np.triu(w, 1) == 0)


def pin_split_combine(orc):
    """Partials over disjoint key ranges, combined by their lse, equal the
    unsplit result; adding the partials (ignoring their denominators) does
    not (smzdm digest, section 5)."""
    B, H, N, d = 1, 2, 61, 16
    q, k, v = synth.fwd_inputs(B, H, N, d, "bf16", seed=16)
    qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
    rows = np.array([(0, h, i) for h in range(H) for i in (0, 5, 30, 60)])
    full_o, full_lse = orc.attention_rows(qb, kb, vb, "bf16", rows, False, 0.25)
    for bounds in ([0, 61], [0, 30, 61], [0, 1, 2, 61], [0, 20, 20, 40, 61],
                   [0, 7, 14, 21, 28, 35, 42, 49, 56, 61]):
        parts = [orc.attention_rows(qb, kb, vb, "bf16", rows, False, 0.25, lo, hi)
                 for lo, hi in zip(bounds[:-1], bounds[1:])]
        po = np.stack([p[0] for p in parts], axis=1)   # [rows, nsplit, d]
        pl = np.stack([p[1] for p in parts], axis=1)   # [rows, nsplit]
        for r in range(len(rows)):
            o, lse = orc.combine(po[r], pl[r])
            np.testing.assert_allclose(o, full_o[r], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse, full_lse[r], rtol=1e-13, atol=1e-13)
        if len(parts) > 1:
            naive = po.sum(axis=1)
            assert np.abs(naive - full_o).max() > 1e-2


def pin_permutation_invariance(orc):
    """Non-causal attention does not depend on the order of the key/value
    rows when K and V are permuted together."""
    q, k, v = synth.fwd_inputs(1, 1, 40, 16, "fp16", seed=17)
    qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
    perm = np.random.default_rng(0).permutation(40)
    o1, l1 = orc.attention(qb, kb, vb, "fp16", False, 0.25)
    o2, l2 = orc.attention(qb, kb[:, :, perm].copy(), vb[:, :, perm].copy(), "fp16", False, 0.25)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)


def _torch_reference(qb, kb, vb, dtype, causal, scale):
    q = torch.from_numpy(widened(qb, dtype))
    k = torch.from_numpy(widened(kb, dtype))
    v = torch.from_numpy(widened(vb, dtype))
    group = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(group, dim=1)
    v = v.repeat_interleave(group, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
    s = scale * (q @ k.transpose(-1, -2).contiguous())
    if causal:
        mask = torch.ones(s.shape[-2:], dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


def pin_library_routine(orc):
    """torch's CPU fp64 scaled_dot_product_attention and logsumexp."""
    for dtype, causal, shape, scale in (("bf16", False, (2, 2, 33, 64), 0.125),
                                        ("fp16", True, (1, 3, 70, 32), 1 / math.sqrt(32)),
                                        ("bf16", True, (1, 1, 128, 128), 1 / math.sqrt(128))):
        q, k, v = synth.fwd_inputs(*shape, dtype, seed=18)
        qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
        o, lse = orc.attention(qb, kb, vb, dtype, causal, scale)
        ro, rl = _torch_reference(qb, kb, vb, dtype, causal, scale)
        np.testing.assert_allclose(o, ro, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


def _brute(qw, kw, vw, causal, scale):
    """Pure Python, math.fsum, softmax as exp(s) / sum exp(s) directly."""
    Nq, d = len(qw), len(qw[0])
    out, lses = [], []
    for i in range(Nq):
        keys = [j for j in range(len(kw)) if (not causal or j <= i)]
        e = [math.exp(scale * math.fsum(qw[i][c] * kw[j][c] for c in range(d))) for j in keys]
        z = math.fsum(e)
        out.append([math.fsum(e[t] * vw[j][c] for t, j in enumerate(keys)) / z
                    for c in range(len(vw[0]))])
        lses.append(math.log(z))
    return out, lses


def pin_brute_force(orc):
    for dtype, causal, N, d in (("bf16", False, 9, 5), ("fp16", True, 12, 7), ("bf16", True, 16, 8)):
        q, k, v = synth.fwd_inputs(1, 2, N, d, dtype, seed=19)
        qb, kb, vb = synth.to_bits(q), synth.to_bits(k), synth.to_bits(v)
        o, lse = orc.attention(qb, kb, vb, dtype, causal, 0.4)
        qw, kw, vw = widened(qb, dtype), widened(kb, dtype), widened(vb, dtype)
        for h in range(2):
            bo, bl = _brute(qw[0, h].tolist(), kw[0, h].tolist(), vw[0, h].tolist(), causal, 0.4)
            np.testing.assert_allclose(o[0, h], np.array(bo), rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[0, h], np.array(bl), rtol=1e-13, atol=1e-13)


def pin_decode_gqa(orc):
    """Decode = the definition with one query per (b, hq) against KV head
    hq // (Hq/Hkv): KV heads made distinguishable by a constant V per head,
    so O[b, hq] = that head's constant; plus the forward row definition."""
    B, Hq, Hkv, L, d = 2, 8, 2, 19, 16
    q, k, _ = synth.decode_inputs(B, Hq, Hkv, L, d, "bf16", seed=20)
    vconst = np.zeros((B, Hkv, L, d), np.float32)
    for b in range(B):
        for g in range(Hkv):
            vconst[b, g] = 10 * b + g + 1
    vb = bits_of(vconst, "bf16")
    qb, kb = synth.to_bits(q), synth.to_bits(k)
    o, lse = orc.decode(qb, kb, vb, "bf16")
    for b in range(B):
        for hq in range(Hq):
            np.testing.assert_allclose(o[b, hq], 10 * b + hq // (Hq // Hkv) + 1, rtol=1e-12)
    # lse against the library routine with repeat_interleave'd heads
    _, rl = _torch_reference(qb[:, :, None], kb, vb, "bf16", False, 1 / math.sqrt(d))
    np.testing.assert_allclose(lse, rl[:, :, 0], rtol=1e-12, atol=1e-12)


def fp8_widened(b):
    """Library widening of E4M3 bytes (torch float8_e4m3fn), for expected values."""
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def pin_widen_fp8(orc):
    """All 256 E4M3 byte patterns widen to torch's float8_e4m3fn values."""
    bits = np.arange(256, dtype=np.uint8)
    ref = fp8_widened(bits)
    for b in bits:
        got = orc.widen(int(b), "fp8")
        if math.isnan(ref[b]):
            assert math.isnan(got), hex(b)
        else:
            assert got == ref[b], (hex(b), got, ref[b])


def pin_fp8_library_routine(orc):
    """FP8 attention = torch fp64 SDPA and logsumexp on the dequantized
    tensors dq*q8, dk*k8, dv*v8 (factors other than 1)."""
    for causal, shape in ((False, (1, 2, 40, 64)), (True, (1, 2, 50, 32))):
        q8, k8, v8, _ = synth.fp8_inputs(*shape, seed=22)
        qb, kb, vb = synth.fp8_bits(q8), synth.fp8_bits(k8), synth.fp8_bits(v8)
        dq, dk, dv, scale = 0.25, 0.5, 3.0, 1 / math.sqrt(shape[-1])
        o, lse = orc.attention_fp8(qb, kb, vb, causal, scale, dq, dk, dv)
        q = torch.from_numpy(dq * fp8_widened(qb))
        k = torch.from_numpy(dk * fp8_widened(kb))
        v = torch.from_numpy(dv * fp8_widened(vb))
        ro = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
        s = scale * (q @ k.transpose(-1, -2).contiguous())
        if causal:
            s = s.masked_fill(torch.ones(s.shape[-2:], dtype=torch.bool).triu(1), float("-inf"))
        np.testing.assert_allclose(o, ro.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def pin_fp8_single_key(orc):
    """One key: O = dv * v8[0] and lse = scale * dq * dk * <q8, k8[0]>."""
    q8, k8, v8, _ = synth.fp8_inputs(1, 2, 1, 16, seed=23)
    qb, kb, vb = synth.fp8_bits(q8), synth.fp8_bits(k8), synth.fp8_bits(v8)
    o, lse = orc.attention_fp8(qb, kb, vb, False, 0.3, 0.5, 0.25, 2.0)
    np.testing.assert_allclose(o, 2.0 * fp8_widened(vb), rtol=1e-15)
    want = 0.3 * 0.5 * 0.25 * (fp8_widened(qb) * fp8_widened(kb)).sum(-1)
    np.testing.assert_allclose(lse, want, rtol=1e-13)


# -- gradients ---------------------------------------------------------------

def pin_bwd_finite_difference(orc):
    """Central differences of f = sum(dout * O) with respect to every input
    element, on fp64 inputs (no storage rounding), with and without the
    causal mask."""
    rng = np.random.default_rng(31)
    B, H, N, d, h = 1, 2, 6, 4, 1e-5
    for causal in (False, True):
        q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
        g = orc.attention_bwd(q, k, v, do, "f64", causal, 0.7)

        def f(qq, kk, vv):
            return float((orc.attention_bwd(qq, kk, vv, do, "f64", causal, 0.7)["o"] * do).sum())

        for name, which in (("dq", 0), ("dk", 1), ("dv", 2)):
            num = np.zeros((B, H, N, d))
            for idx in np.ndindex(B, H, N, d):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][idx] += h
                args_m[which][idx] -= h
                num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
            np.testing.assert_allclose(g[name], num, rtol=0, atol=1e-7,
                                       err_msg=f"{name} causal={causal}")


def pin_bwd_library_routine(orc):
    """torch autograd through CPU fp64 scaled_dot_product_attention."""
    for dtype, causal, shape, scale in (("bf16", False, (1, 2, 40, 64), 0.125),
                                        ("fp16", True, (2, 1, 37, 32), 1 / math.sqrt(32))):
        q, k, v, do = synth.bwd_inputs(*shape, dtype, seed=32)
        bits = [synth.to_bits(t) for t in (q, k, v, do)]
        g = orc.attention_bwd(*bits, dtype, causal, scale)
        tq, tk, tv, tdo = (torch.from_numpy(widened(b, dtype)) for b in bits)
        for t in (tq, tk, tv):
            t.requires_grad_(True)
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                             scale=scale)
        (o * tdo).sum().backward()
        for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
            np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-9, atol=1e-11,
                                       err_msg=name)


def pin_bwd_invariants(orc):
    """Every row of dS sums to zero, so sum_j dK_j = 0; the weights of each
    query sum to one, so sum_j dV_j = sum_i dO_i; and scaling every score by
    t gives d/dt = sum_i <dQ_i, q_i> = sum_j <dK_j, k_j>."""
    for causal in (False, True):
        q, k, v, do = synth.bwd_inputs(2, 2, 50, 16, "fp16", seed=33)
        bits = [synth.to_bits(t) for t in (q, k, v, do)]
        g = orc.attention_bwd(*bits, "fp16", causal, 0.3)
        qw, kw, dow = widened(bits[0], "fp16"), widened(bits[1], "fp16"), widened(bits[3], "fp16")
        np.testing.assert_allclose(g["dk"].sum(axis=2), 0.0, atol=1e-11)
        np.testing.assert_allclose(g["dv"].sum(axis=2), dow.sum(axis=2), rtol=1e-12, atol=1e-11)
        np.testing.assert_allclose((g["dq"] * qw).sum(axis=(2, 3)),
                                   (g["dk"] * kw).sum(axis=(2, 3)), rtol=1e-10, atol=1e-10)


def pin_bwd_closed_forms(orc):
    """One key: the weight is 1 whatever q and k are, so dQ = dK = 0 and
    dV = dO.  Causal row 0 sees only key 0: dQ_0 = 0.  Value rows all equal:
    O does not depend on the weights, so dQ = dK = 0."""
    q, k, v, do = synth.bwd_inputs(1, 2, 1, 8, "bf16", seed=34)
    bits = [synth.to_bits(t) for t in (q, k, v, do)]
    g = orc.attention_bwd(*bits, "bf16", False, 0.9)
    assert not g["dq"].any() and not g["dk"].any()
    np.testing.assert_array_equal(g["dv"], widened(bits[3], "bf16"))
    q, k, v, do = synth.bwd_inputs(1, 1, 9, 8, "bf16", seed=35)
    bits = [synth.to_bits(t) for t in (q, k, v, do)]
    g = orc.attention_bwd(*bits, "bf16", True, 0.9)
    assert not g["dq"][0, 0, 0].any()
    vrow = np.repeat(bits[2][:, :, :1, :], 9, axis=2)
    g = orc.attention_bwd(bits[0], bits[1], vrow, bits[3], "bf16", False, 0.9)
    np.testing.assert_allclose(g["dq"], 0.0, atol=1e-13)
    np.testing.assert_allclose(g["dk"], 0.0, atol=1e-13)


def pin_bwd_forward_outputs(orc):
    """The O and lse the gradient routine recomputes are the forward's, and
    selected rows and columns equal the same rows of the full result."""
    q, k, v, do = synth.bwd_inputs(1, 3, 45, 32, "bf16", seed=36)
    bits = [synth.to_bits(t) for t in (q, k, v, do)]
    g = orc.attention_bwd(*bits, "bf16", True, 0.2)
    o, lse = orc.attention(*bits[:3], "bf16", True, 0.2)
    np.testing.assert_allclose(g["o"], o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(g["lse"], lse, rtol=1e-13, atol=1e-15)
    sel = np.array([(0, 2, 44), (0, 0, 0), (0, 1, 17)])
    gs = orc.attention_bwd(*bits, "bf16", True, 0.2, qrows=sel, kcols=sel[::-1])
    for r, (b, h, i) in enumerate(sel):
        np.testing.assert_array_equal(gs["dq"][r], g["dq"][b, h, i])
    for r, (b, h, j) in enumerate(sel[::-1]):
        np.testing.assert_array_equal(gs["dk"][r], g["dk"][b, h, j])
        np.testing.assert_array_equal(gs["dv"][r], g["dv"][b, h, j])
    # dQ rows alone (no key columns): only those rows' statistics are formed.
    gq = orc.attention_bwd(*bits, "bf16", True, 0.2, qrows=sel, kcols=np.zeros((0, 3)))
    for r, (b, h, i) in enumerate(sel):
        np.testing.assert_array_equal(gq["dq"][r], g["dq"][b, h, i])
        np.testing.assert_array_equal(gq["lse"][r], g["lse"][b, h, i])


PINS = [pin_widen_all_patterns, pin_worked_examples, pin_single_key, pin_causal_row0,
        pin_uniform_when_q_zero, pin_constant_v, pin_weights_sum_to_one, pin_split_combine,
        pin_permutation_invariance, pin_library_routine, pin_brute_force, pin_decode_gqa,
        pin_widen_fp8, pin_fp8_library_routine, pin_fp8_single_key,
        pin_bwd_finite_difference, pin_bwd_library_routine, pin_bwd_invariants,
        pin_bwd_closed_forms, pin_bwd_forward_outputs]


@pytest.fixture(scope="module")
def orc():
    return oracle_mod.get()


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_rejects_bad_arguments(orc):
    q = np.zeros((1, 2, 4, 8), np.uint16)
    with pytest.raises(ValueError):
        orc.attention_rows(q, q, q, "bf16", [(0, 5, 0)], False, 1.0)
    with pytest.raises(ValueError):
        orc.attention_rows(q, np.zeros((1, 3, 4, 8), np.uint16), np.zeros((1, 3, 4, 8), np.uint16),
                           "bf16", [(0, 0, 0)], False, 1.0)


def test_empty_key_range(orc):
    q, k, v = synth.fwd_inputs(1, 1, 8, 8, "bf16", seed=21)
    o, lse = orc.attention_rows(synth.to_bits(q), synth.to_bits(k), synth.to_bits(v), "bf16",
                                [(0, 0, 3)], False, 1.0, 5, 5)
    assert lse[0] == -np.inf and not o.any()
    o2, l2 = orc.combine(np.zeros((3, 8)), np.full(3, -np.inf))
    assert l2 == -np.inf and not o2.any()


MUTANTS = {
    1: "sign of the scale flipped",
    2: "causal visibility j < i instead of j <= i",
    3: "lse drops the running max",
    4: "scores computed against V instead of K",
    5: "grouped-query head map hq % Hkv",
    6: "output not divided by the softmax denominator",
    7: "combine adds the partial outputs",
    8: "fp16 exponent bias 14",
    9: "V row index off by one",
    10: "dot product drops the last head_dim term",
    11: "bf16 widening shifts by 15",
    12: "combine lse drops log of the weight sum",
    13: "E4M3 exponent bias 8",
    14: "value dequantization factor dropped",
    15: "softmax Jacobian drops the row term sum_k P_ik dP_ik",
    16: "dQ not multiplied by the scale",
    17: "dV weights not normalised (lse dropped)",
    18: "dK accumulates dO rows instead of q rows",
    19: "dK/dV ignore the causal mask",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_pins_catch_planted_mistake(tmp_path, mutant):
    path = oracle_mod.build(tmp_path / f"libfa_oracle_m{mutant}.so", mutant=mutant)
    bad = oracle_mod.Oracle(path)
    caught = []
    for pin in PINS:
        try:
            pin(bad)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {mutant}: {MUTANTS[mutant]}"
