"""Pins the Quest oracle ("KV Cache Engineering for LLM Serving", section 7
"Query-aware sparse reads") to the page's worked example, to the bound the
score stands for, and to full attention when nothing is skipped."""

import json
import os

import numpy as np
import pytest

from oracle import attention, quest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_values(x):
    """float32 values rounded to bf16 (nearest even), as float64."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def test_page_example():
    g = json.load(open(os.path.join(GOLDEN, "quest_example.json")))
    pages = np.array(g["pages"], dtype=np.float64)
    q = np.array(g["query"])
    scores = [quest.page_score(q, *quest.page_summary(p)) for p in pages]
    assert scores == g["page_scores"]
    sel = quest.select_pages(scores, g["pages_read"])
    assert sel == g["selected_pages"]
    per_page = pages.shape[1]
    assert len(sel) * per_page == g["entries_read"]
    assert pages.shape[0] * per_page == g["entries_stored"]


@pytest.mark.parametrize("seed", range(5))
def test_score_is_the_tight_bound_of_q_dot_k_over_the_page(seed):
    """Every key of the page scores at most the page score, and the corner of
    the page's box that the query points to scores exactly the page score."""
    rng = np.random.default_rng(seed)
    D = 64
    keys = bf16_values(rng.standard_normal((16, D)))
    q = bf16_values(rng.standard_normal(D) * 3)
    kmin, kmax = quest.page_summary(keys)
    s = quest.page_score(q, kmin, kmax)
    for k in keys:
        assert float(np.dot(q, k)) <= s + 1e-12
    corner = np.where(q >= 0, kmax, kmin)
    assert quest.page_score(q, corner, corner) == s
    # the summary is the box: every key lies inside it
    assert (keys >= kmin).all() and (keys <= kmax).all()
    assert (kmin == keys.min(axis=0)).all() and (kmax == keys.max(axis=0)).all()


def test_group_score_is_the_best_head():
    rng = np.random.default_rng(7)
    keys = rng.standard_normal((16, 8))
    qg = rng.standard_normal((4, 8))
    kmin, kmax = quest.page_summary(keys)
    per_head = [quest.page_score(q, kmin, kmax) for q in qg]
    assert quest.group_page_score(qg, kmin, kmax) == max(per_head)
    assert quest.group_page_score(qg[:1], kmin, kmax) == per_head[0]


def test_selection_order_and_ties():
    assert quest.select_pages([3.0, 1.0, 3.0, 3.0, 0.0], 2) == [0, 2]
    assert quest.select_pages([3.0, 1.0, 3.0, 3.0, 0.0], 4) == [0, 1, 2, 3]
    assert quest.select_pages([0.5, 2.0], 5) == [0, 1]
    assert quest.select_pages([-1.0, -2.0, -0.5], 1) == [2]


def test_partial_last_page_summarises_its_written_rows():
    rng = np.random.default_rng(3)
    L, D = 37, 8
    keys = rng.standard_normal((L, D))
    q = rng.standard_normal((2, D))
    scores = quest.sequence_page_scores(q, keys, L)
    assert len(scores) == 3
    last = quest.group_page_score(q, *quest.page_summary(keys[32:37]))
    assert scores[2] == last


def test_full_budget_is_full_attention():
    rng = np.random.default_rng(11)
    L, Hq, Hkv, D = 70, 8, 2, 16
    q = rng.standard_normal((Hq, D))
    K = rng.standard_normal((L, Hkv, D))
    V = rng.standard_normal((L, Hkv, D))
    out, chosen = quest.quest_decode(q, K, V, L, budget=5, sm_scale=0.25)
    assert chosen == [[0, 1, 2, 3, 4]] * Hkv
    ref = attention.decode_sequence(q, K, V, 0.25)
    assert np.abs(out - ref).max() < 1e-6


def test_budget_reads_only_the_best_page():
    """One page whose keys line up with every query head of the group and a
    constant value row c; the other pages score low.  With a budget of one
    page the output is exactly c."""
    rng = np.random.default_rng(5)
    L, Hq, Hkv, D = 64, 4, 1, 8
    q = np.abs(rng.standard_normal((Hq, D))) + 0.5
    K = -np.abs(rng.standard_normal((L, Hkv, D)))
    V = rng.standard_normal((L, Hkv, D))
    K[32:48] = np.abs(K[32:48]) + 4.0
    V[32:48] = 0.75
    out, chosen = quest.quest_decode(q, K, V, L, budget=1, sm_scale=0.3)
    assert chosen == [[2]]
    assert (out == np.float32(0.75)).all()
