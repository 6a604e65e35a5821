"""Prefix reuse and heavy-hitter retention (oracle, test-only).

"KV Cache Engineering for LLM Serving, clearly explained":

* section 11 "Prefix reuse": every completed prefix block is stored under a
  lookup key made of the whole token prefix up to the end of that block, so
  a block is reused only when everything before it matches too; a request
  reuses its leading blocks whose keys are already stored.
* section 9 "Eviction" (H2O): with a budget of positions, the latest
  ``recent`` positions are kept, and the remaining budget goes to the older
  positions with the largest accumulated attention scores (heavy hitters);
  equal scores keep the earlier position (a stable sort by score).

Plain Python: dictionaries and sorts, nothing clever.
"""


def prefix_keys(tokens, block_size):
    """Lookup keys of the full blocks of ``tokens``: the whole prefix up to
    the end of each block."""
    return [tuple(tokens[:end]) for end in range(block_size, len(tokens) + 1, block_size)]


class PrefixCache:
    """Full-prefix key -> physical block."""

    def __init__(self, block_size):
        self.block_size = block_size
        self.blocks = {}

    def match(self, tokens):
        """Blocks of the leading full blocks of ``tokens`` whose keys are
        stored, up to the first miss."""
        out = []
        for key in prefix_keys(tokens, self.block_size):
            if key not in self.blocks:
                break
            out.append(self.blocks[key])
        return out

    def insert(self, tokens, blocks):
        """Stores the keys of the full blocks of ``tokens`` with their blocks
        (``blocks[i]`` holds block i); a stored key keeps its block.
        Returns the number of keys added."""
        added = 0
        for i, key in enumerate(prefix_keys(tokens, self.block_size)):
            if i >= len(blocks):
                break
            if key not in self.blocks:
                self.blocks[key] = blocks[i]
                added += 1
        return added


def h2o_retain(scores, budget, recent_count):
    """Positions kept under a budget: the latest ``recent_count`` positions
    plus the ``budget - recent_count`` older positions with the largest
    scores (earlier position first among equal scores), in position order."""
    n = len(scores)
    if budget >= n:
        return list(range(n))
    recent_count = min(recent_count, budget)
    positions = list(range(n))
    recent = positions[n - recent_count:] if recent_count else []
    older = positions[:n - recent_count]
    heavy = sorted(older, key=lambda p: scores[p], reverse=True)[:budget - recent_count]
    return sorted(heavy + recent)
