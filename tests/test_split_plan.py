"""Invariants of the decode's stream-K split, on random shapes (CPU).

The decode kernel plans its split on the device (build_block_list in
paged_attn.hip); this test restates that arithmetic in Python and checks,
over thousands of shapes far more varied than the GPU parity cases, what
the merge and the block lists rely on:

* every unit (partition holding a kept token) has exactly one owner;
* a sequence's units go to consecutive workgroups with none skipped (the
  merge reads slot 2w of every workgroup between the first and the last);
* the plan entry's last workgroup is the owner of the sequence's last unit;
* no workgroup's block list overflows, with the grid sized as the host
  sizes it (decode_slots in api.hip).

Two split rules are covered: units counted one by one, and, for full
attention with partitions of several blocks, units placed by their first
block (a workgroup takes a run of blocks and the units that start in it).
The GPU parity tests check the kernel itself against the oracle.
"""

import random

import pytest


def cdiv(a, b):
    return -(-a // b)


def grid_slots(S, hkv, num_partitions, psize, cus=256):
    """Workgroups along the sequence axis, as the host sizes the grid."""
    list_cap = 128 * min(hkv, 8)
    k = max(cdiv(8 * cus, hkv), S)
    bpu = max(psize // 16, 1)
    cap = (list_cap - bpu + 1) // bpu if 3 * bpu <= list_cap else list_cap // bpu
    if cap > 0:
        k = max(k, cdiv(S * num_partitions, cap))
    return k, list_cap


def plan(lens, psize, K, list_cap):
    """Owner workgroup of every (sequence, unit), blocks per workgroup and the
    last workgroup of each sequence, by the kernel's rules (full attention)."""
    bpp = psize // 16
    min_units = max(1, 128 // psize)
    weighted = bpp > 1 and 3 * bpp <= list_cap
    step = bpp if weighted else 1
    seqs, P = [], 0
    for L in lens:
        nb, n = cdiv(L, 16), cdiv(L, psize)
        seqs.append((P, n, nb))
        P += nb if weighted else n
    U = P
    if U == 0:
        return {}, [], {}
    if weighted:
        k_eff = max(1, min(K, min(U // (min_units * step), U // step)))
    else:
        Q = max(min_units, cdiv(U, K))
        k_eff = cdiv(U, Q)
    owner, blocks, last = {}, [0] * k_eff, {}
    for w in range(k_eff):
        u0, u1 = w * U // k_eff, (w + 1) * U // k_eff
        for s, (P, n, nb) in enumerate(seqs):
            if P >= u1:
                break
            i0 = min(n, cdiv(u0 - P, step) if u0 > P else 0)
            i1 = min(n, cdiv(u1 - P, step))
            for u in range(i0, i1):
                assert (s, u) not in owner
                owner[(s, u)] = w
                blocks[w] += min((u + 1) * bpp, nb) - u * bpp
            if i0 == 0 and i1 > 0:
                last[s] = ((P + (n - 1) * step + 1) * k_eff - 1) // U
    return owner, blocks, last


def check(lens, psize, hkv):
    mbs = max(cdiv(L, 16) for L in lens) + 1
    K, list_cap = grid_slots(len(lens), hkv, cdiv(mbs * 16, psize), psize)
    owner, blocks, last = plan(lens, psize, K, list_cap)
    for s, L in enumerate(lens):
        n = cdiv(L, psize)
        ws = [owner[(s, u)] for u in range(n)]          # every unit owned
        assert ws == sorted(ws)
        if n:
            assert set(range(ws[0], ws[-1] + 1)) <= set(ws), (s, ws)
            assert last[s] == ws[-1]
    assert len(owner) == sum(cdiv(L, psize) for L in lens)
    assert max(blocks, default=0) <= list_cap
    return blocks


def test_split_invariants_on_random_shapes():
    rng = random.Random(7)
    for _ in range(2000):
        S = rng.choice([1, 2, 4, 7, 64, 65, 130])
        psize = rng.choice([16, 32, 64, 128, 256, 512, 1024, 2048])
        hkv = rng.choice([1, 2, 8, 16])
        if psize // 16 > 128 * min(hkv, 8):
            continue                                    # rejected by the host
        big = 131073 if S <= 4 else 3000
        lens = [rng.choice([0, 1, 15, 16, 17, rng.randint(1, 6000), big]) for _ in range(S)]
        check(lens, psize, hkv)


def test_block_balanced_split_at_128k():
    """4 sequences of 131072 tokens plus the appended one, 512-token
    partitions, 8 KV heads: counted in blocks no workgroup takes more than
    129 blocks (counted in partitions, some took 5 partitions = 160)."""
    blocks = check([131073] * 4, 512, 8)
    assert len(blocks) == 256 and max(blocks) == 129


@pytest.mark.parametrize("psize", [16, 64, 512])
def test_one_sequence_many_workgroups(psize):
    check([20000], psize, 8)
