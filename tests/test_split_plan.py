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

from split_model import cdiv, grid_slots, plan


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


@pytest.mark.parametrize("T", [2, 3, 4])
@pytest.mark.parametrize("psize", [0, 64])
def test_tail_cut_generator_reaches_the_causal_tail(T, psize):
    """The multi-token parity cases' lengths put a workgroup boundary at a
    unit past position L - T of a cut sequence (a block holding fewer than T
    of its tokens) and include a sequence shorter than T."""
    from split_model import causal_tail_starts, tail_cut_lens
    for append in (True, False):
        prompt = tail_cut_lens(T, psize, 8, append=append)
        lens = [L + (1 if append else 0) for L in prompt]
        mbs = max(cdiv(L, 16) for L in lens) + 1
        cuts = causal_tail_starts(lens, psize, T, 8, mbs)
        assert any(t0 > 0 for _, t0 in cuts)
        assert min(lens) < T
        # the start is a true cut: inside the sequence, past token 0's limit
        for s, t0 in cuts:
            assert t0 == 0 or lens[s] - T < t0 < lens[s]
