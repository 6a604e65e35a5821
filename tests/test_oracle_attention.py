"""Pins the oracle's attention to brute force, a library routine and
invariants that hold for any correct paged decode."""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import attention, codecs, paging
from oracle_pipeline import OracleRun, to_raw
from workloads import draw_tensors, get_workload


def brute_force_decode(q, K, V, scale, Hq, Hkv):
    """Pure-Python loops in float64: one query row per head, one key per token."""
    L, _, D = K.shape
    out = [[0.0] * D for _ in range(Hq)]
    for h in range(Hq):
        kvh = h * Hkv // Hq
        scores = []
        for t in range(L):
            acc = 0.0
            for i in range(D):
                acc += float(q[h][i]) * float(K[t][kvh][i])
            scores.append(acc * scale)
        if not scores:
            continue
        mx = max(scores)
        ex = [np.exp(s - mx) for s in scores]
        tot = sum(ex)
        for i in range(D):
            out[h][i] = sum(ex[t] * float(V[t][kvh][i]) for t in range(L)) / tot
    return np.array(out)


def sdpa_reference(q, K, V, scale, Hq, Hkv):
    """torch's CPU scaled_dot_product_attention, GQA by repeating KV heads."""
    G = Hq // Hkv
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, None, :]              # [Hq,1,D]
    kt = torch.from_numpy(np.asarray(K, np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(np.asarray(V, np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(), scale=scale)
    return o[:, 0, :].numpy()


@pytest.fixture(scope="module")
def tiny():
    w = get_workload("tiny_fp32")
    t = draw_tensors(w, "cpu")
    return w, t, OracleRun(w, t)


def test_tiny_workload_shape(tiny):
    w, t, run = tiny
    assert w.seq_lens.tolist() == [40, 17, 64, 1]
    assert w.num_blocks == 32
    assert [len(x) for x in run.tables] == [3, 2, 5, 1]     # after the append
    assert run.lens.tolist() == [41, 18, 65, 2]


def test_brute_force_matches_vectorized(tiny):
    w, t, run = tiny
    q = to_raw(t["query"], "f32")
    out = run.decode(q)
    for s in range(w.S):
        K = paging.gather_sequence(run.k_cache, run.tables[s], run.lens[s], w.BS)
        V = paging.gather_sequence(run.v_cache, run.tables[s], run.lens[s], w.BS)
        ref = brute_force_decode(q[s], K, V, w.sm_scale, w.Hq, w.Hkv)
        assert np.abs(out[s] - ref).max() < 1e-6


def test_matches_sdpa_on_contiguous(tiny):
    """Paging changes addresses, not results: the paged decode equals plain
    attention over the logical sequence (library routine on CPU)."""
    w, t, run = tiny
    q = to_raw(t["query"], "f32")
    out = run.decode(q)
    for s in range(w.S):
        K = paging.gather_sequence(run.k_cache, run.tables[s], run.lens[s], w.BS)
        V = paging.gather_sequence(run.v_cache, run.tables[s], run.lens[s], w.BS)
        ref = sdpa_reference(q[s], K, V, w.sm_scale, w.Hq, w.Hkv)
        assert np.abs(out[s] - ref).max() < 1e-6


def test_written_rows_gather_back(tiny):
    """Every prompt token and every appended token reads back bit-exactly."""
    w, t, run = tiny
    key = to_raw(t["key"], "f32")
    seq_ids = t["seq_ids"].numpy()
    pos = t["positions"].numpy()
    for j in range(len(seq_ids)):
        s, p = int(seq_ids[j]), int(pos[j])
        got = paging.gather_sequence(run.k_cache, run.tables[s], p + 1, w.BS)[p]
        assert (got.view(np.uint32) == key[j].view(np.uint32)).all()
    nk = to_raw(t["new_key"], "f32")
    for s in range(w.S):
        got = paging.gather_sequence(run.k_cache, run.tables[s], run.lens[s], w.BS)[-1]
        assert (got.view(np.uint32) == nk[s].view(np.uint32)).all()
    # sequence 2 grew from 64 to 65 tokens: a fresh fifth block
    assert len(run.tables[2]) == 5


def test_all_60_placements_give_identical_output():
    """A 3-block sequence placed in every ordered choice of 3 of 5 physical
    blocks gives bit-identical output (summation follows logical order)."""
    rng = np.random.default_rng(7)
    Hq, Hkv, D, bs, L = 4, 2, 8, 16, 40
    K = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    outs = []
    for placement in itertools.permutations(range(5), 3):
        kc = np.full((5, bs, Hkv, D), np.nan, np.float32)
        vc = np.full((5, bs, Hkv, D), np.nan, np.float32)
        slots = [paging.slot_of(placement, t, bs) for t in range(L)]
        paging.reshape_and_cache(kc, K, slots, bs)
        paging.reshape_and_cache(vc, V, slots, bs)
        o = attention.paged_decode(q, "f32", kc, vc, "f32", np.array([placement]), [L], bs, 0.3)
        outs.append(o)
    assert len(outs) == 60
    for o in outs[1:]:
        assert (o.view(np.uint32) == outs[0].view(np.uint32)).all()
    ref = sdpa_reference(q[0], K, V, 0.3, Hq, Hkv)
    assert np.abs(outs[0][0] - ref).max() < 1e-6


def test_special_cases():
    rng = np.random.default_rng(3)
    D = 16
    K = rng.standard_normal((33, D))
    V = rng.standard_normal((33, D))
    q = rng.standard_normal(D)
    # one token: output is that token's value, exactly
    out, p = attention.softmax_attention(q, K[:1], V[:1], 0.25)
    assert (out == V[0]).all() and p.tolist() == [1.0]
    # constant values: output is the constant
    c = np.full((33, D), 0.75)
    out, p = attention.softmax_attention(q, K, c, 0.25)
    assert np.abs(out - 0.75).max() < 1e-15
    assert abs(p.sum() - 1.0) < 1e-15 and (p > 0).all()
    # zero query: uniform weights, output is the mean of the values
    out, p = attention.softmax_attention(np.zeros(D), K, V, 0.25)
    assert np.abs(out - V.mean(axis=0)).max() < 1e-14
    # one dominant score: output is (nearly) that token's value
    K2 = np.zeros((33, D)); K2[17] = 1.0
    out, _ = attention.softmax_attention(np.full(D, 100.0), K2, V, 1.0)
    assert np.abs(out - V[17]).max() < 1e-12
    # scores enter with their sign: a large negative score drops a token
    K3 = np.zeros((2, D)); K3[0] = -1.0
    out, p = attention.softmax_attention(np.full(D, 100.0), K3, V[:2], 1.0)
    assert p[1] > 0.999999 and np.abs(out - V[1]).max() < 1e-6
    # empty sequence: zeros
    out, p = attention.softmax_attention(q, K[:0], V[:0], 0.25)
    assert (out == 0).all() and p.size == 0


@pytest.mark.parametrize("L,sink,window,psize", [
    (40, 0, 0, 16), (1000, 0, 0, 512), (1000, 0, 0, 128), (5000, 4, 4092, 512),
    (9000, 4, 4092, 512), (4096, 4, 4092, 512), (1, 0, 0, 512),
])
def test_split_k_merge_equals_single_pass(L, sink, window, psize):
    rng = np.random.default_rng(L)
    D = 32
    K = rng.standard_normal((L, D)) * 2
    V = rng.standard_normal((L, D))
    q = rng.standard_normal(D)
    kept = attention.kept_positions(L, sink, window)
    ref, _ = attention.softmax_attention(q, K[kept], V[kept], 0.2)
    m, l, acc = attention.partition_partials(q, K[kept], V[kept], 0.2, kept, psize)
    assert m.size == -(-L // psize)
    if sink and (L - window) // psize >= 2:
        assert np.isneginf(m).any()          # partitions between sinks and window are empty
    out = attention.merge_partials(m, l, acc)
    assert np.abs(out - ref).max() < 1e-13


def test_streaming_mask_equals_attention_on_kept_subsequence():
    rng = np.random.default_rng(11)
    L, D, Hq, Hkv = 5000, 16, 4, 2
    K = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((Hq, D)).astype(np.float32)
    out = attention.decode_sequence(q, K, V, 0.25, sink=4, window=4092)
    keep = np.r_[0:4, L - 4092:L]
    ref = sdpa_reference(q, K[keep], V[keep], 0.25, Hq, Hkv)
    assert np.abs(out - ref).max() < 1e-6
    full = attention.decode_sequence(q, K[:4096], V[:4096], 0.25, sink=4, window=4092)
    assert (full == attention.decode_sequence(q, K[:4096], V[:4096], 0.25)).all()


def test_copy_on_write_step_on_shared_prefix():
    """Shrunk shared-prefix workload: the fork's shared partial block is copied
    exactly once, the source block is untouched by the write, and the other
    sequences keep their outputs."""
    w = get_workload("shared_prefix_b128", S=6, len_lo=20, len_hi=60, prefix_tokens=64, D=16, Hq=8, Hkv=2)
    t = draw_tensors(w, "cpu")
    before = OracleRun(w, t, do_step=False)
    run = OracleRun(w, t)
    assert len(run.cow) == 1
    src, dst = run.cow[0]
    # the copy carries the shared rows; the write went into the copy only
    off = int(before.lens[0]) % w.BS
    assert (run.k_cache[dst][:off].view(np.uint32) == run.cow_src_before[0][0][:off].view(np.uint32)).all() \
        if w.src_dtype == "f32" else (run.k_cache[dst][:off] == run.cow_src_before[0][0][:off]).all()
    # the old block keeps the shared rows, then receives the fork's own token
    assert (run.k_cache[src][:off] == run.cow_src_before[0][0][:off]).all()
    # both sequences now have distinct last blocks
    assert run.tables[0][-1] != run.tables[1][-1]
    assert run.tables[0][:-1] == run.tables[1][:-1]
    # every sequence but 0 and 1 shares the prefix blocks
    for s in range(2, w.S):
        assert run.tables[s][:4] == run.tables[0][:4]
    q = to_raw(t["query"], "bf16")
    out = run.decode(q)
    assert np.isfinite(out).all()


# --------------------------------------------------------------------------
# several query tokens per sequence
# --------------------------------------------------------------------------

def _paged_case(rng, S, L, Hq, Hkv, D, bs=16):
    nb = sum(-(-l // bs) for l in L)
    order = rng.permutation(nb)
    k = rng.standard_normal((nb, bs, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((nb, bs, Hkv, D)).astype(np.float32)
    tables, pos = [], 0
    for l in L:
        n = -(-l // bs)
        tables.append(list(order[pos:pos + n]) + [0])
        pos += n
    width = max(len(t) for t in tables)
    bt = np.array([t + [0] * (width - len(t)) for t in tables], dtype=np.int64)
    return k, v, bt


def test_multi_query_token_t_is_the_decode_of_its_prefix():
    """Token t of T new tokens gives exactly the one-token decode of the
    sequence cut after its own position; T = 1 is the decode."""
    rng = np.random.default_rng(41)
    S, Hq, Hkv, D, T = 3, 8, 2, 16, 4
    L = [37, 16, 70]
    k, v, bt = _paged_case(rng, S, L, Hq, Hkv, D)
    q = rng.standard_normal((S, T, Hq, D)).astype(np.float32)
    out = attention.multi_query_decode(q, "f32", k, v, "f32", bt, L, 16, 0.25)
    for t in range(T):
        cut = [l - T + t + 1 for l in L]
        ref = attention.paged_decode(q[:, t], "f32", k, v, "f32", bt, cut, 16, 0.25)
        assert np.array_equal(out[:, t], ref)
    one = attention.multi_query_decode(q[:, -1:], "f32", k, v, "f32", bt, L, 16, 0.25)
    assert np.array_equal(one[:, 0], attention.paged_decode(q[:, -1], "f32", k, v, "f32", bt, L, 16, 0.25))


def test_multi_query_against_scalar_loops():
    """Brute force: explicit loops over positions with the causal limit."""
    rng = np.random.default_rng(43)
    S, Hq, Hkv, D, T = 2, 4, 2, 8, 3
    L = [19, 5]
    k, v, bt = _paged_case(rng, S, L, Hq, Hkv, D)
    q = rng.standard_normal((S, T, Hq, D)).astype(np.float32)
    out = attention.multi_query_decode(q, "f32", k, v, "f32", bt, L, 16, 0.5)
    G = Hq // Hkv
    for s in range(S):
        for t in range(T):
            for h in range(Hq):
                n = L[s] - T + t + 1
                sc, vals = [], []
                for p in range(n):
                    blk, off = bt[s][p // 16], p % 16
                    sc.append(0.5 * sum(float(q[s, t, h, d]) * float(k[blk, off, h // G, d]) for d in range(D)))
                    vals.append([float(x) for x in v[blk, off, h // G]])
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                tot = sum(w)
                ref = [sum(w[i] * vals[i][d] for i in range(n)) / tot for d in range(D)]
                assert np.abs(out[s, t, h] - np.array(ref)).max() < 1e-5
