"""Pins the prefix-reuse and heavy-hitter oracles to the pages' examples
("KV Cache Engineering for LLM Serving", sections 9 and 11) and to brute
force."""

import itertools
import json
import os
import random

from oracle import reuse

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    return json.load(open(os.path.join(GOLDEN, name)))


def test_prefix_reuse_example():
    g = golden("prefix_reuse_example.json")
    c = reuse.PrefixCache(g["block_size"])
    first_hits = c.match(g["first"])
    c.insert(g["first"], [100, 101, 102])
    second_hits = c.match(g["second"])
    n = len(reuse.prefix_keys(g["second"], g["block_size"]))
    assert len(first_hits) == g["first_reused"]
    assert len(second_hits) == g["second_reused"] and second_hits == [100, 101]
    assert n == g["blocks_per_request"]
    assert n - len(second_hits) == g["second_new_blocks"]


def test_full_prefix_keys_prevent_false_matches():
    """The same four tokens in the middle of two requests do not match when
    what precedes them differs."""
    c = reuse.PrefixCache(4)
    c.insert([1, 2, 3, 4, 5, 6, 7, 8], [0, 1])
    assert c.match([9, 9, 9, 9, 5, 6, 7, 8]) == []
    assert c.match([1, 2, 3, 4, 5, 6, 7, 9]) == [0]
    # a partial last block has no key
    assert c.match([1, 2, 3]) == []


def test_h2o_example():
    g = golden("h2o_example.json")
    kept = reuse.h2o_retain(g["scores"], g["budget"], g["recent_count"])
    assert kept == g["retained"]
    older = [p for p in kept if p not in g["recent"]]
    assert older == g["heavy_hitters"]


def test_h2o_against_brute_force():
    """The kept set maximises the summed score of the older positions among
    all sets that keep the recent ones, preferring earlier positions on
    ties (checked by enumerating every subset)."""
    rng = random.Random(3)
    for _ in range(200):
        n = rng.randint(1, 9)
        scores = [rng.choice([0.0, 0.5, 1.0, 2.0, 3.0]) for _ in range(n)]
        budget = rng.randint(0, n + 1)
        recent = rng.randint(0, budget)
        kept = reuse.h2o_retain(scores, budget, recent)
        if budget >= n:
            assert kept == list(range(n))
            continue
        r = min(recent, budget)
        must = list(range(n - r, n))
        best = None
        for combo in itertools.combinations(range(n - r), budget - r):
            key = (sum(scores[p] for p in combo), [-p for p in combo])
            if best is None or key > best[0]:
                best = (key, list(combo))
        assert kept == sorted(best[1] + must)
