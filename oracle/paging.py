"""Block-paged KV addressing, slot write and block copy (oracle, test-only).

Layout.  "Chapter 18 - KV-Cache Optimization Strategies", section "How
PagedAttention Works" and its "Physical KV Block" figure: the cache is cut into
fixed blocks of ``block_size`` tokens, each block holding
``[block_size, n_kv_heads, d_k]`` keys and the same for values.  The whole
cache is therefore ``[num_blocks, block_size, n_kv_heads, d_k]`` for K and again
for V.

Addressing.  The same section and the block-table paragraph of Learning-AI
topic t13_4: a per-sequence table maps logical block ``t // block_size`` to a
physical block; token ``t`` sits at offset ``t % block_size`` inside it.  The
flat slot number of a token is ``physical_block * block_size + offset`` and a
slot identifies one row ``cache[slot // block_size, slot % block_size]``.

Writes.  New tokens are appended into the current block (Chapter 18, "How
PagedAttention Works"; t13_4 on appending entries as tokens are generated).
Copy-on-write duplicates a whole shared block when a sequence diverges
(t13_4, copy-on-write paragraph).

All functions work on raw storage arrays (any numpy dtype) and are bit copies.
"""

import numpy as np


def slot_of(table_row, t, block_size):
    """Flat slot of logical token ``t`` of a sequence with block table
    ``table_row``: ``table_row[t // block_size] * block_size + t % block_size``.
    """
    t = int(t)
    return int(table_row[t // block_size]) * block_size + t % block_size


def slot_mapping(block_tables, seq_ids, positions, block_size):
    """Slot of each token j, which is token ``positions[j]`` of sequence
    ``seq_ids[j]``.  Returns int64 slots."""
    bt = np.asarray(block_tables)
    out = np.empty(len(positions), dtype=np.int64)
    for j, (s, t) in enumerate(zip(seq_ids, positions)):
        out[j] = slot_of(bt[int(s)], int(t), block_size)
    return out


def reshape_and_cache(cache, rows, slots, block_size):
    """Write ``rows[j]`` (shape ``[n_kv_heads, d_k]``) into the cache row of
    slot ``slots[j]``; a negative slot means "skip this token".  In place,
    bitwise.  ``cache`` has shape ``[num_blocks, block_size, n_kv_heads, d_k]``.
    """
    for j, slot in enumerate(np.asarray(slots).tolist()):
        if slot < 0:
            continue
        cache[slot // block_size, slot % block_size] = rows[j]
    return cache


def copy_blocks(arrays, pairs):
    """Copy-on-write duplication: for each ``(src, dst)`` in ``pairs``, copy
    the whole physical block ``src`` (every slot, every head) to ``dst`` in
    each array of ``arrays`` (K cache, V cache, and per-block scales when the
    cache is quantised).  Pairs are applied in order.  In place, bitwise."""
    for src, dst in pairs:
        for a in arrays:
            a[int(dst)] = a[int(src)]
    return arrays


def gather_sequence(cache, table_row, length, block_size):
    """Rows of a sequence in logical order: element ``t`` is the cache row of
    token ``t``, for ``t < length``.  Shape ``[length, n_kv_heads, d_k]``.

    The blocks need not be adjacent; the table fixes their logical order
    ("KV Cache Engineering", section 10 "Paging": the attention code reads
    non-adjacent blocks in logical sequence order)."""
    idx = [slot_of(table_row, t, block_size) for t in range(int(length))]
    if not idx:
        return cache[:0, 0].copy()
    idx = np.asarray(idx, dtype=np.int64)
    return cache[idx // block_size, idx % block_size].copy()


def blocks_needed(length, block_size):
    """Number of blocks a sequence of ``length`` tokens occupies: every block
    is full except possibly the last."""
    return -(-int(length) // block_size)


def wasted_slots(length, block_size):
    """Unused slots of a sequence: only its last block can be partly empty
    (t13_4, block-table paragraph)."""
    return blocks_needed(length, block_size) * block_size - int(length)
