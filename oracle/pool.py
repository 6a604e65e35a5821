"""Free-block pool with reference counts and copy-on-write (oracle, test-only).

* "KV Cache Engineering for LLM Serving", section 10 "Paging": a shared pool of
  equal blocks; a request takes free blocks from the front of the free list
  and a finished request returns its blocks to the back of it (the page's
  example: A takes [0, 1, 2], B takes [3, 4], A's return leaves [5, 0, 1, 2],
  C then takes [5, 0]).
* "Chapter 18", section "How PagedAttention Works": new tokens fill the
  current block and a new block is taken when it is full.
* "Chapter 18", section "Prefix Caching", and Learning-AI topic t13_4,
  copy-on-write paragraph: shared blocks are referenced by several
  sequences; when a sequence writes into a shared block, that block is
  duplicated first and the sequence's table is repointed to the copy.
"""

from collections import deque


class PoolExhausted(MemoryError):
    """No free block is left."""


class BlockPool:
    """FIFO free list of physical block ids plus a reference count per block."""

    def __init__(self, num_blocks, initial_order=None):
        order = list(range(num_blocks)) if initial_order is None else [int(b) for b in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.free_list = deque(order)
        self.refcount = [0] * num_blocks

    # -- basic operations ---------------------------------------------------
    def alloc(self):
        """Take the block at the front of the free list (refcount becomes 1)."""
        if not self.free_list:
            raise PoolExhausted("block pool exhausted")
        b = self.free_list.popleft()
        self.refcount[b] = 1
        return b

    def incref(self, b):
        if self.refcount[b] <= 0:
            raise ValueError(f"incref of free block {b}")
        self.refcount[b] += 1

    def decref(self, b):
        """Drop one reference; a block whose count reaches 0 goes to the back
        of the free list."""
        if self.refcount[b] <= 0:
            raise ValueError(f"decref of free block {b}")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free_list.append(b)

    # -- sequence-level operations --------------------------------------------
    def allocate_sequence(self, length, block_size):
        """Blocks for a new sequence of ``length`` tokens, taken in order."""
        n = -(-int(length) // block_size)
        return [self.alloc() for _ in range(n)]

    def fork(self, table):
        """A new sequence sharing every block of ``table`` (refcounts + 1)."""
        for b in table:
            self.incref(b)
        return list(table)

    def release(self, table):
        """A finished sequence returns its blocks, in table order."""
        for b in table:
            self.decref(b)

    def append(self, table, length, block_size):
        """Reserve the slot of token ``length`` of a sequence.

        Mutates ``table`` and returns ``(slot, cow)``, where ``cow`` is None or
        the ``(src, dst)`` pair of a block that must be copied before the
        write.  A new block is taken exactly when ``length % block_size == 0``;
        otherwise, if the current last block is shared (refcount > 1), it is
        duplicated: a fresh block is taken, the old one loses a reference, and
        the table points at the copy.
        """
        cow = None
        if length % block_size == 0:
            if length // block_size != len(table):
                raise ValueError("table length does not match sequence length")
            table.append(self.alloc())
        else:
            i = length // block_size
            b = table[i]
            if self.refcount[b] > 1:
                nb = self.alloc()
                self.decref(b)
                table[i] = nb
                cow = (b, nb)
        slot = table[length // block_size] * block_size + length % block_size
        return slot, cow

    # -- statistics -------------------------------------------------------------
    def stats(self):
        used = sum(1 for r in self.refcount if r > 0)
        shared = sum(1 for r in self.refcount if r > 1)
        return {"free": len(self.free_list), "used": used, "shared": shared}
