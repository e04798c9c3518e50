"""fa_decode_paged through the C ABI on an MI355X: paged key/value pools,
block tables and a length per sequence, against the fp64 oracle applied to
each sequence's keys gathered through its block table."""
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


def make_paged(lens, Hq, Hkv, d, page, dtype, seed, spare_pages=5):
    """Random pools and block tables: every sequence gets distinct pages in a
    shuffled order; unused table entries hold out-of-range ids."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    pps = max(1, max((L + page - 1) // page for L in lens))
    need = sum((L + page - 1) // page for L in lens)
    num_pages = need + spare_pages
    perm = rng.permutation(num_pages)
    table = np.full((B, pps), 10 ** 6, dtype=np.int32)
    pos = 0
    for b, L in enumerate(lens):
        n = (L + page - 1) // page
        table[b, :n] = perm[pos:pos + n]
        pos += n
    q, kp, vp = synth.decode_inputs(1, Hq, Hkv, num_pages * page, d, dtype, seed=seed, device=DEV)
    q = synth.normal((B, Hq, d), seed * 16 + 5, dtype, DEV)
    # [1, Hkv, num_pages*page, d] -> pools [num_pages, page, Hkv, d]
    kpages = kp[0].reshape(Hkv, num_pages, page, d).permute(1, 2, 0, 3).contiguous()
    vpages = vp[0].reshape(Hkv, num_pages, page, d).permute(1, 2, 0, 3).contiguous()
    return q, kpages, vpages, torch.from_numpy(table).to(DEV), \
        torch.tensor(lens, dtype=torch.int32, device=DEV), table


def gather(pages_bits, table_row, L, page):
    """[num_pages, page, Hkv, d] bits -> [1, Hkv, L, d] keys of one sequence."""
    idx = np.arange(L)
    rows = pages_bits[table_row[idx // page], idx % page]          # [L, Hkv, d]
    return np.ascontiguousarray(rows.transpose(1, 0, 2)[None])


def run(orc, lens, Hq, Hkv, d, page, nsplit, dtype="bf16", seed=0):
    print(f"case decode_paged lens={lens} Hq{Hq} Hkv{Hkv} d{d} page{page} nsplit{nsplit} {dtype}",
          flush=True)
    q, kpages, vpages, table, seq, table_np = make_paged(lens, Hq, Hkv, d, page, dtype, seed)
    o, lse = fa.decode_paged(q, kpages, vpages, table, seq, nsplit=nsplit)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    qb, kb, vb = synth.to_bits(q), synth.to_bits(kpages), synth.to_bits(vpages)
    ro = np.zeros_like(o, dtype=np.float64)
    rl = np.zeros_like(lse, dtype=np.float64)
    for b, L in enumerate(lens):
        if L == 0:
            ro[b], rl[b] = 0.0, -np.inf
            continue
        kc, vc = gather(kb, table_np[b], L, page), gather(vb, table_np[b], L, page)
        rob, rlb = orc.decode(qb[b:b + 1], kc, vc, dtype)
        ro[b], rl[b] = rob[0], rlb[0]
    empty = np.array(lens) == 0
    assert not o[empty].any() and np.all(lse[empty] == -np.inf)
    if (~empty).any():
        assert_close(o[~empty], ro[~empty], lse[~empty], rl[~empty],
                     f"decode_paged page{page} nsplit{nsplit} {dtype}")


@pytest.mark.parametrize("page", [16, 32, 48, 64, 256])
def test_page_sizes(orc, page):
    run(orc, [1, 17, 100, 777, 2048, 0, 3000], 8, 2, 128, page, nsplit=5, seed=page)


@pytest.mark.parametrize("nsplit", [1, 3, 16, 24, 64])
def test_split_counts(orc, nsplit):
    run(orc, [5, 64, 1000, 4096], 8, 2, 128, 32, nsplit=nsplit, seed=100 + nsplit)


def test_dtypes_dims_groups(orc):
    run(orc, [300, 1500, 33], 16, 16, 64, 16, nsplit=4, dtype="fp16", seed=201)
    run(orc, [2000, 70], 32, 4, 128, 64, nsplit=8, dtype="bf16", seed=202)
    run(orc, [512, 513], 20, 1, 128, 128, nsplit=6, dtype="fp16", seed=203)


def test_four_head_groups(orc):
    """Shapes whose launch gives each workgroup four kv heads (two waves
    each): Hkv a multiple of 4 and at least 256 such workgroups.  Ragged
    lengths, an empty sequence, shards past a sequence's end."""
    run(orc, [1, 33, 500, 0, 1200, 64, 2049, 7], 16, 8, 128, 16, nsplit=40, seed=300)
    run(orc, [100, 3000, 1, 257], 16, 4, 64, 32, nsplit=64, dtype="fp16", seed=301)


def test_matches_dense_layout():
    """A paged cache holding the same keys as a dense one, one length for
    all sequences and shard boundaries on 32-key blocks: identical results."""
    B, Hq, Hkv, L, d, page = 2, 8, 2, 1024, 128, 64
    q, k, v = synth.decode_inputs(B, Hq, Hkv, L, d, "bf16", seed=210, device=DEV)
    o_d, l_d = fa.decode(q, k, v, nsplit=8, return_lse=True)
    npg = L // page
    kpages = k.reshape(B, Hkv, npg, page, d).permute(0, 2, 3, 1, 4).reshape(B * npg, page, Hkv, d).contiguous()
    vpages = v.reshape(B, Hkv, npg, page, d).permute(0, 2, 3, 1, 4).reshape(B * npg, page, Hkv, d).contiguous()
    table = torch.arange(B * npg, dtype=torch.int32, device=DEV).reshape(B, npg)
    seq = torch.full((B,), L, dtype=torch.int32, device=DEV)
    o_p, l_p = fa.decode_paged(q, kpages, vpages, table, seq, nsplit=8)
    torch.cuda.synchronize()
    assert torch.equal(o_d, o_p) and torch.equal(l_d, l_p)


def test_bench_shape(orc):
    """The workload bench.py's paged_decode leg times (B8 Hq32 Hkv8 L32768
    d128 bf16, 16-token pages in shuffled order, nsplit 16, the same launch):
    every query head of every sequence against the oracle on the keys
    gathered through the block table."""
    c = synth.PAGED_BENCH
    B, page = c["B"], c["page"]
    print(f"case decode_paged bench shape B{B} Hq{c['Hq']} Hkv{c['Hkv']} L{c['L']} page{page}",
          flush=True)
    q, kp, vp, table, seq = synth.paged_decode_inputs(B, c["Hq"], c["Hkv"], c["L"], c["d"], page,
                                                      c["dtype"], seed=c["seed"], device=DEV)
    o, lse = fa.decode_paged(q, kp, vp, table, seq, nsplit=c["nsplit"])
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    qb, kb, vb = synth.to_bits(q), synth.to_bits(kp), synth.to_bits(vp)
    del kp, vp
    table_np = table.cpu().numpy()
    ro = np.zeros(o.shape, np.float64)
    rl = np.zeros(lse.shape, np.float64)
    for b in range(B):
        kc, vc = gather(kb, table_np[b], c["L"], page), gather(vb, table_np[b], c["L"], page)
        rob, rlb = orc.decode(qb[b:b + 1], kc, vc, c["dtype"])
        ro[b], rl[b] = rob[0], rlb[0]
    assert_close(o, ro, lse, rl, f"decode_paged bench shape nsplit{c['nsplit']}")
