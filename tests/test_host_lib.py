"""CPU tests of the library's host side: symbols, block pool, validation and
argument checks that return before anything is enqueued.  No GPU is touched."""

import os
import random
import re

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_466_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(pkv_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 20
    for n in sorted(names):
        assert hasattr(pkv.lib, n), n
    assert "gfx950" in pkv.version()


def test_pool_reproduces_paging_example():
    """KV Cache Engineering, section 10: A=[0,1,2], B=[3,4], free [5,0,1,2], C=[5,0]."""
    p = pkv.BlockPool(6)
    a = p.allocate_sequence(3, 1)
    b = p.allocate_sequence(2, 1)
    assert a == [0, 1, 2] and b == [3, 4]
    p.release(a)
    assert p.free_list() == [5, 0, 1, 2]
    assert p.allocate_sequence(2, 1) == [5, 0]


def test_pool_matches_oracle_pool_on_random_operations():
    """Differential test: the same random sequence of allocations, forks,
    appends and releases on the library pool and the oracle pool."""
    rng = random.Random(5)
    for trial in range(20):
        nb = rng.randint(4, 40)
        order = list(range(nb))
        rng.shuffle(order)
        lp, op = pkv.BlockPool(nb, order), oracle.pool.BlockPool(nb, order)
        seqs = []          # (lib_table, oracle_table, length)
        for step in range(200):
            r = rng.random()
            try:
                if r < 0.2 or not seqs:
                    L = rng.randint(0, 40)
                    need = -(-L // 16)
                    if need > len(op.free_list):
                        continue
                    seqs.append([lp.allocate_sequence(L), op.allocate_sequence(L, 16), L])
                elif r < 0.35:
                    i = rng.randrange(len(seqs))
                    seqs.append([lp.fork(seqs[i][0]), op.fork(seqs[i][1]), seqs[i][2]])
                elif r < 0.9:
                    i = rng.randrange(len(seqs))
                    lt, ot, L = seqs[i]
                    try:
                        exp = op.append(ot, L, 16)
                    except oracle.pool.PoolExhausted:
                        with pytest.raises(pkv.PkvError) as e:
                            lp.append(lt, L, 16, capacity=len(lt) + 1)
                        assert e.value.status == 5
                        continue
                    got = lp.append(lt, L, 16, capacity=len(lt) + 1)
                    assert got == exp and lt == ot
                    seqs[i][2] = L + 1
                else:
                    i = rng.randrange(len(seqs))
                    lt, ot, L = seqs.pop(i)
                    lp.release(lt)
                    op.release(ot)
            finally:
                pass
            assert lp.free_list() == list(op.free_list)
            assert lp.stats() == op.stats()
            for b in range(nb):
                assert lp.refcount(b) == op.refcount[b]


def test_pool_errors():
    with pytest.raises(pkv.PkvError):
        pkv.BlockPool(3, [0, 0, 1])
    p = pkv.BlockPool(1)
    b = p.alloc()
    with pytest.raises(pkv.PkvError) as e:
        p.alloc()
    assert e.value.status == 5 and "exhausted" in str(e.value)
    p.decref(b)
    with pytest.raises(pkv.PkvError) as e:
        p.decref(b)
    assert e.value.status == 1
    assert p.refcount(99) == -1
    table = []
    with pytest.raises(pkv.PkvError):
        p.append(table, 5, 16)          # table does not cover 5 tokens


def test_validate_tables():
    import torch
    bt = torch.tensor([[7, 2, 14, -1]], dtype=torch.int32)
    pkv.validate_tables(bt, torch.tensor([40], dtype=torch.int32), 16)
    with pytest.raises(pkv.PkvError, match="block_tables"):
        pkv.validate_tables(bt, torch.tensor([40], dtype=torch.int32), 10)
    with pytest.raises(pkv.PkvError, match="seq_lens"):
        pkv.validate_tables(bt, torch.tensor([65], dtype=torch.int32), 16)
    with pytest.raises(pkv.PkvError, match="repeats"):
        pkv.validate_tables(bt, torch.tensor([40], dtype=torch.int32), 16,
                            slot_mapping=torch.tensor([3, 5, 3], dtype=torch.int32))
    pkv.validate_tables(bt, torch.tensor([0], dtype=torch.int32), 16,
                        slot_mapping=torch.tensor([3, -1, -1, 5], dtype=torch.int32))


def test_partition_and_workspace_sizes():
    # short bounds: one pass, no workspace
    assert pkv.paged_attn_num_partitions("bf16", 96) == 1
    assert pkv.paged_attn_workspace_bytes("bf16", 4, 8, 2, 64, 96) == 0
    # longer bounds: block granularity for 16-bit and code caches, 64 tokens for fp32
    assert pkv.paged_attn_partition_size("bf16", 4096) == 16
    assert pkv.paged_attn_partition_size("i8", 4096) == 16
    assert pkv.paged_attn_partition_size("f32", 4096) == 64
    # 128K tokens in 512-token partitions
    assert pkv.paged_attn_num_partitions("bf16", 131072 + 16, 512) == 257
    # fp32: a record per (sequence, KV head, partition)
    nbytes = pkv.paged_attn_workspace_bytes("f32", 4, 64, 8, 128, 131072, 512)
    n = 4 * 8 * 256
    assert nbytes >= n * (8 * 128 + 32) * 4
    # 16-bit: the plan area and two records per (workgroup, KV head); with 8
    # KV heads a workgroup per compute unit (256 on a host without a GPU)
    nbytes = pkv.paged_attn_workspace_bytes("bf16", 4, 64, 8, 128, 131072, 512)
    assert nbytes == 256 + 2 * 256 * 8 * (8 * 128 + 32) * 4
    assert pkv.paged_attn_num_partitions("bf16", 1000, 100) == 0     # not a multiple of 16


def test_argument_errors_return_before_launch():
    """Invalid arguments are rejected on the host with a status and message;
    no pointer is dereferenced (all null) and nothing is enqueued."""
    L = pkv.lib
    st = L.pkv_paged_attn_decode(None, None, 1, None, None, 1, None, None, None, 4, None, 2, 32, 8, 96, 16, 10,
                                 0.1, 0, 0, 0, 0, None, 0, None)
    assert st == 2 and "head_dim" in pkv.last_error()
    st = L.pkv_paged_attn_decode(None, None, 1, None, None, 1, None, None, None, 4, None, 2, 30, 8, 128, 16, 10,
                                 0.1, 0, 0, 0, 0, None, 0, None)
    assert st == 1 and "%" in pkv.last_error()
    st = L.pkv_paged_attn_decode(None, None, 1, None, None, 1, None, None, None, 4, None, 2, 32, 8, 128, 32, 10,
                                 0.1, 0, 0, 0, 0, None, 0, None)
    assert st == 2 and "block_size" in pkv.last_error()
    st = L.pkv_paged_attn_decode(None, None, 0, None, None, 3, None, None, None, 4, None, 2, 32, 8, 128, 16, 10,
                                 0.1, 0, 0, 0, 0, None, 0, None)
    assert st == 2                       # int8 codes need a 16-bit query
    st = L.pkv_paged_attn_decode(None, None, 1, None, None, 3, None, None, None, 4, None, 2, 32, 8, 128, 16, 10,
                                 0.1, 0, 0, 0, 0, None, 0, None)
    assert st == 1 and "scales" in pkv.last_error()
    st = L.pkv_paged_attn_decode(None, None, 1, None, None, 1, None, None, None, 4, None, 2, 32, 8, 128, 16, 10,
                                 0.1, 24, 0, 0, 0, None, 0, None)
    assert st == 1 and "partition_size" in pkv.last_error()
    # a 128K bound needs partials: missing workspace is reported
    st = L.pkv_paged_attn_decode(1, 1, 1, 1, 1, 1, None, None, 1, 8192, 1, 4, 64, 8, 128, 16, 32768,
                                 0.1, 512, 0, 0, 0, None, 0, None)
    assert st == 3 and "workspace" in pkv.last_error()
    st = L.pkv_paged_attn_decode(None, None, 1, None, None, 1, None, None, None, 4, None, 2, 64 * 17, 64, 128, 16,
                                 10, 0.1, 0, 0, 0, 0, None, 0, None)
    assert st == 2 and "group" in pkv.last_error()
    assert L.pkv_reshape_and_cache(None, None, None, None, 3, None, 4, 10, 16, 8, 128, None) == 2
    assert L.pkv_quantize_kv(None, 1, None, 1, None, None, 4, 10, 16, 8, 128, None) == 2
    assert L.pkv_copy_blocks(1, 1, 1, None, 1, 1, 1, 10, 16, 8, 128, None) == 1
    assert L.pkv_slot_mapping(1, 1, 4, None, 1, 8, 4, 16, 10, None) == 1
    st = L.pkv_paged_attn_decode(None, None, 1, None, None, 1, None, None, None, 4, None, 2, 32, 8, 128, 16, 10,
                                 0.1, 0, 0, 0, 2, None, 0, None)
    assert st == 1 and "flags" in pkv.last_error()
    # INT4 caches: head_dim 128 only; no raw slot write into codes
    st = L.pkv_paged_attn_decode(None, None, 1, None, None, 5, 1, 1, None, 4, None, 2, 32, 8, 64, 16, 10,
                                 0.1, 0, 0, 0, 0, None, 0, None)
    assert st == 2 and "INT4" in pkv.last_error()
    assert L.pkv_reshape_and_cache(None, None, None, None, 5, None, 4, 10, 16, 8, 128, None) == 2
    # fused slot write: 16-bit caches of the query dtype only
    st = L.pkv_paged_attn_decode_append(None, None, 1, None, None, 3, None, None, None, None, None, 4, None, 2, 32, 8,
                                        128, 16, 10, 0.1, 0, 0, 0, 0, None, 0, None)
    assert st == 2 and "fused" in pkv.last_error()
    st = L.pkv_paged_attn_decode_append(None, None, 1, None, None, 1, None, None, None, None, None, 4, None, 2, 32, 8,
                                        128, 16, 10, 0.1, 0, 0, 0, 0, None, 0, None)
    assert st == 1 and "null" in pkv.last_error()
    # grouped scales: i8 / i4 codes; scale pointers; scale group kind
    st = L.pkv_paged_attn_decode_grouped(None, None, 1, None, None, 4, 1, 1, 1, None, 4, None, 2, 32, 8, 128, 16, 10,
                                         0.1, 0, 0, None, 0, None)
    assert st == 2 and "grouped" in pkv.last_error()
    st = L.pkv_paged_attn_decode_grouped(None, None, 1, None, None, 3, None, 1, 1, None, 4, None, 2, 32, 8, 128, 16,
                                         10, 0.1, 0, 0, None, 0, None)
    assert st == 1 and "scale" in pkv.last_error()
    assert L.pkv_quantize_kv_grouped(1, 1, 1, 3, None, 1, 7, None, 4, 10, 16, 8, 128, None) == 1
    assert L.pkv_quantize_kv_grouped(1, 1, 1, 1, None, 1, 0, None, 4, 10, 16, 8, 128, None) == 2
    assert L.pkv_append_kv_quantized_grouped(1, 1, 1, 1, 1, 1, 1, 3, 1, None, 1, 1, 4, 1, 2, 10, 16, 8, 128,
                                             None) == 1
    # empty batches are no-ops
    assert L.pkv_paged_attn_decode(None, None, 1, None, None, 1, None, None, None, 4, None, 0, 32, 8, 128, 16, 10,
                                   0.1, 0, 0, 0, 0, None, 0, None) == 0
    assert L.pkv_reshape_and_cache(None, None, None, None, 1, None, 0, 10, 16, 8, 128, None) == 0


def test_shared_prefix_host_side():
    """pkv_paged_attn_decode_shared_prefix rejects bad arguments on the host;
    pkv_validate_shared_prefix checks its preconditions; the workspace is the
    prefix records plus the suffix decode's workspace."""
    L = pkv.lib
    f = L.pkv_paged_attn_decode_shared_prefix
    # (out, query, q_dtype, k, v, kv_dtype, key, value, positions, slots, tables, mbs, lens, S, Hq, Hkv, D, BS,
    #  NB, scale, prefix_blocks, psize, flags, ws, ws_bytes, stream)
    st = f(None, None, 0, None, None, 0, None, None, None, None, None, 8, None, 2, 32, 8, 128, 16, 10, 0.1, 2, 0, 0,
           None, 0, None)
    assert st == 2 and "bf16" in pkv.last_error()
    st = f(None, None, 1, None, None, 3, None, None, None, None, None, 8, None, 2, 32, 8, 128, 16, 10, 0.1, 2, 0, 0,
           None, 0, None)
    assert st == 2
    for pb in (0, 9):
        st = f(None, None, 1, None, None, 1, None, None, None, None, None, 8, None, 2, 32, 8, 128, 16, 10, 0.1, pb, 0,
               0, None, 0, None)
        assert st == 1 and "prefix_blocks" in pkv.last_error()
    st = f(None, None, 1, None, None, 1, 1, None, None, None, None, 8, None, 2, 32, 8, 128, 16, 10, 0.1, 2, 0, 0,
           None, 0, None)
    assert st == 1 and "key" in pkv.last_error()
    st = f(1, 1, 1, 1, 1, 1, None, None, None, None, 1, 8, 1, 2, 32, 8, 128, 16, 10, 0.1, 2, 0, 0, None, 0, None)
    assert st == 3 and "workspace" in pkv.last_error()
    st = f(None, None, 1, None, None, 1, None, None, None, None, None, 8, None, 2, 32, 8, 96, 16, 10, 0.1, 2, 0, 0,
           1 << 20, 1 << 20, None)
    assert st == 2 and "head_dim" in pkv.last_error()
    st = f(None, None, 1, None, None, 1, None, None, None, None, None, 8, None, 2, 32, 8, 128, 16, 10, 0.1, 2, 0, 4,
           1 << 20, 1 << 20, None)
    assert st == 1 and "flags" in pkv.last_error()
    # an empty batch is a no-op
    assert f(None, None, 1, None, None, 1, None, None, None, None, None, 8, None, 0, 32, 8, 128, 16, 10, 0.1, 2, 0, 0,
             None, 0, None) == 0

    # preconditions
    bt = torch.tensor([[3, 5, 7, 0], [3, 5, 9, 1], [3, 5, 2, 4]], dtype=torch.int32)
    lens = torch.tensor([50, 49, 64], dtype=torch.int32)
    pkv.validate_shared_prefix(bt, lens, 2)
    with pytest.raises(pkv.PkvError, match="differs"):
        pkv.validate_shared_prefix(bt, lens, 3)
    with pytest.raises(pkv.PkvError, match="shorter"):
        pkv.validate_shared_prefix(bt, torch.tensor([50, 31, 64], dtype=torch.int32), 2)
    with pytest.raises(pkv.PkvError):
        pkv.validate_shared_prefix(bt, lens, 5)

    # workspace: the prefix records, (acc[D], m, l, 2 unused) fp32 per (sequence, query head); the records of
    # sequences finished in one piece, (acc[G][D], m[16], l[16]) per (sequence, KV head); each 256-byte
    # aligned; then the decode's workspace for the tokens past the prefix, or its plan area (16 bytes per
    # sequence, 256-byte aligned) when no sequence can be cut
    S, Hq, Hkv, D = 128, 64, 8, 128
    align = lambda n: -(-n // 256) * 256
    pre = align(S * Hq * (D + 4) * 4) + align(S * Hkv * ((Hq // Hkv) * D + 32) * 4)
    for max_len, P in ((3100, 64), (1024, 64), (1100, 64), (5000, 1)):
        got = pkv.paged_attn_shared_prefix_workspace_bytes("bf16", S, Hq, Hkv, D, max_len, P)
        split = pkv.paged_attn_workspace_bytes("bf16", S, Hq, Hkv, D, max(max_len - 16 * P, 0))
        assert got == pre + (split if split else align(16 * S)), (max_len, P)
    assert pkv.paged_attn_shared_prefix_workspace_bytes("bf16", 0, Hq, Hkv, D, 3100, 64) == 0


# --------------------------------------------------------------------------
# host block reuse: prefix cache and H2O retention
# --------------------------------------------------------------------------

def test_prefix_cache_reproduces_page_example():
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "prefix_reuse_example.json")))
    pool = pkv.BlockPool(16)
    c = pkv.PrefixCache(pool, g["block_size"])
    assert c.match(g["first"]) == []
    first_blocks = [pool.alloc() for _ in range(3)]
    assert c.insert(g["first"], first_blocks) == 3
    hits = c.match(g["second"])
    assert len(hits) == g["second_reused"] and hits == first_blocks[:2]
    assert 3 - len(hits) == g["second_new_blocks"]
    # the lookup handed the caller a reference per block, the cache holds one
    assert [pool.refcount(b) for b in first_blocks] == [3, 3, 2]


def test_prefix_cache_matches_oracle_on_random_requests():
    """Differential test against the oracle's full-prefix-key dictionary:
    requests over a small vocabulary (many shared prefixes) look up, take
    new blocks for the rest, store their full blocks and finish."""
    rng = random.Random(9)
    bs = 4
    pool = pkv.BlockPool(4000)
    c = pkv.PrefixCache(pool, bs)
    o = oracle.reuse.PrefixCache(bs)
    for _ in range(300):
        n = rng.randint(0, 30)
        stem = [1, 2, 3, 4, 5, 6, 7, 8][: rng.randint(0, 8)]
        toks = stem + [rng.randint(0, 3) for _ in range(n)]
        got = c.match(toks)
        assert got == o.match(toks)
        need = -(-len(toks) // bs)
        blocks = got + [pool.alloc() for _ in range(need - len(got))]
        added = c.insert(toks, blocks)
        assert added == o.insert(toks, blocks)
        for b in blocks:                      # the request finishes
            pool.decref(b)
    assert len(c) == len(o.blocks)
    # every cached block is held by the cache only, so all can be evicted
    assert c.evict(10 ** 6) == len(o.blocks)
    assert len(c) == 0 and len(pool.free_list()) == pool.num_blocks


def test_prefix_cache_evicts_least_recently_used_leaf():
    pool = pkv.BlockPool(8)
    c = pkv.PrefixCache(pool, 2)
    a, b = [1, 2, 3, 4, 5, 6], [1, 2, 3, 4, 7, 8]
    ablk = [pool.alloc() for _ in range(3)]
    c.insert(a, ablk)
    hit = c.match(b)
    bblk = hit + [pool.alloc()]
    c.insert(b, bblk)
    for blk in ablk + bblk:
        pool.decref(blk)
    assert c.evict(1) == 1                    # a's last block: the older leaf
    ha, hb = c.match(a), c.match(b)
    assert ha == ablk[:2] and hb == bblk
    # blocks a running sequence holds are not evicted
    assert c.evict(10) == 0 and len(c) == 3
    for blk in ha + hb:
        pool.decref(blk)
    assert c.evict(10) == 3 and len(c) == 0
    assert len(pool.free_list()) == 8


def test_h2o_matches_page_and_oracle():
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "h2o_example.json")))
    assert pkv.h2o_retain(g["scores"], g["budget"], g["recent_count"]) == g["retained"]
    rng = random.Random(4)
    for _ in range(300):
        n = rng.randint(0, 40)
        scores = [rng.choice([0.0, 0.25, 1.0, 3.5]) for _ in range(n)]
        budget = rng.randint(0, n + 2)
        recent = rng.randint(0, budget + 1)
        assert pkv.h2o_retain(scores, budget, recent) == oracle.reuse.h2o_retain(scores, budget, recent)
    with pytest.raises(pkv.PkvError):
        pkv.h2o_retain([1.0, float("nan")], 1, 0)


def test_pool_sequence_operations_are_all_or_nothing():
    """pkv_pool_allocate_sequence / _fork / _release change nothing on an
    error: too few free blocks, a free or out-of-range block, a block listed
    more often than it is referenced."""
    p = pkv.BlockPool(5)
    a = p.allocate_sequence(40)                   # 3 blocks, the last partial
    assert a == [0, 1, 2] and p.free_list() == [3, 4]
    with pytest.raises(pkv.PkvError, match="needed"):
        p.allocate_sequence(48)                   # 3 more blocks, 2 free
    assert p.free_list() == [3, 4]
    f = p.fork(a)
    assert [p.refcount(b) for b in f] == [2, 2, 2]
    with pytest.raises(pkv.PkvError):
        p.fork([0, 3])                            # 3 is free
    assert [p.refcount(b) for b in (0, 3)] == [2, 0]
    with pytest.raises(pkv.PkvError):
        p.release([0, 0, 0])                      # 3 references asked, 2 held
    assert p.refcount(0) == 2
    p.release(f)
    p.release(a[::-1])                            # freed in table order
    assert p.free_list() == [3, 4, 2, 1, 0]
    assert p.allocate_sequence(0) == []
