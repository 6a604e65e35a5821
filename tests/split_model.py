"""CPU model of the decode's stream-K split (test helper).

The decode kernel plans its split on the device (build_block_list in
paged_attn.hip).  This module restates that arithmetic in Python so that
tests can check its invariants on many shapes and can pick lengths that put
a workgroup boundary where a parity case needs one.  It holds none of the
attention arithmetic.
"""


def cdiv(a, b):
    return -(-a // b)


def grid_slots(S, hkv, num_partitions, psize, cus=256):
    """Workgroups along the sequence axis, as the host sizes the grid, and
    the block-list capacity of one workgroup."""
    list_cap = 128 * min(hkv, 8)
    k = max(cdiv(8 * cus, hkv), S)
    bpu = max(psize // 16, 1)
    cap = (list_cap - bpu + 1) // bpu if 3 * bpu <= list_cap else list_cap // bpu
    if cap > 0:
        k = max(k, cdiv(S * num_partitions, cap))
    return k, list_cap


def plan(lens, psize, K, list_cap):
    """Owner workgroup of every (sequence, unit), blocks per workgroup and the
    last workgroup of each sequence, by the kernel's rules (full attention).
    A unit is a partition of ``psize`` tokens holding at least one token."""
    bpp = psize // 16
    min_units = max(1, 80 // psize)
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


def resolve_partition(psize, mbs):
    """The partition size the library uses for a 16-bit or code cache whose
    tables hold ``mbs`` entries (``psize`` 0 = the library's choice)."""
    if psize > 0:
        return psize
    max_len = mbs * 16
    return max_len if max_len <= 512 else 16


def segment_starts(lens, psize, hkv, mbs, cus=256):
    """(sequence, first token) of every segment the split makes: the first
    unit of each sequence and every unit whose owner differs from the
    previous unit's."""
    ps = resolve_partition(psize, mbs)
    K, list_cap = grid_slots(len(lens), hkv, cdiv(mbs * 16, ps), ps, cus)
    owner, _, _ = plan(lens, ps, K, list_cap)
    starts = []
    for s, L in enumerate(lens):
        for u in range(cdiv(L, ps)):
            if u == 0 or owner[(s, u)] != owner[(s, u - 1)]:
                starts.append((s, u * ps))
    return starts


def causal_tail_starts(lens, psize, T, hkv, mbs, cus=256):
    """Segments that begin past the first query token's causal limit: with T
    query tokens at positions L - T .. L - 1, token 0 sees positions up to
    L - T, so a segment starting at token t0 > L - T holds nothing that
    token sees (and, for L < T, some token sees nothing at all)."""
    return [(s, t0) for s, t0 in segment_starts(lens, psize, hkv, mbs, cus) if t0 > lens[s] - T]


def tail_cut_lens(T, psize, hkv, S=4, lo=520, hi=1400, append=True, cus=256, seed=0):
    """Prompt lengths for a multi-token parity case whose split starts a
    segment inside the causal tail: S - 1 lengths drawn from [lo, hi] (a
    seeded search) such that some workgroup's segment of a sequence begins
    at a unit past position L - T, then one empty prompt, whose decode
    length (1 after the append) is below T.  ``append``: the decode step
    appends one token, so decode lengths are prompt lengths + 1."""
    import random
    rng = random.Random(1000 * T + psize + 7 * seed)
    extra = 1 if append else 0
    for _ in range(20000):
        prompt = [rng.randint(lo, hi) for _ in range(S - 1)] + [0]
        lens = [L + extra for L in prompt]
        mbs = max(cdiv(L, 16) for L in lens) + 1
        cuts = causal_tail_starts(lens, psize, T, hkv, mbs, cus)
        if any(t0 > 0 for _, t0 in cuts):
            return prompt
    raise RuntimeError("no length draw puts a segment start in the causal tail")
