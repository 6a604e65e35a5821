"""Query-aware page selection (Quest) - oracle, test-only.

"KV Cache Engineering for LLM Serving, clearly explained", section 7
"Query-aware sparse reads": the cache is cut into pages of neighbouring
token entries; each page also keeps the smallest and the largest value its
keys take in every key dimension.  For a new query, every page is scored
from that summary - per dimension the larger of query x minimum and query x
maximum, summed over the dimensions - and only the highest-scoring pages
are read; every entry stays stored.

Readings taken where the page is silent:

* A page is one physical block of the paged cache (16 tokens).  A partial
  last block summarises the rows written so far, nothing else.
* Summaries are exact: the minimum and maximum of the stored values.
* The score is the largest value q . k can take for a key inside the page's
  box, and the sum that forms it is taken exactly rounded (``math.fsum``).
* Grouped-query attention: the G query heads of a KV head read the same
  pages, so a page's score for that KV head is the largest of the G heads'
  scores (the best score any of them can reach inside the page).  Selection
  is per (sequence, KV head).
* ``budget`` pages are kept per (sequence, KV head); a sequence with no more
  pages than that keeps all of them.  Among equal scores the lower page
  (logical block) index is kept.  Kept pages are read in logical order.
* Attention then runs over every written token of the kept pages.
"""

import math

import numpy as np

from . import attention


def page_summary(keys):
    """(minimum, maximum) per key dimension over the rows of one page.

    ``keys``: [n, D] stored values of the page's written rows (n >= 1)."""
    k = np.asarray(keys, dtype=np.float64)
    return k.min(axis=0), k.max(axis=0)


def page_score(q, kmin, kmax):
    """Sum over dimensions of max(q_i * min_i, q_i * max_i), exactly rounded.

    Each product of two stored values (16-bit or fp32) is exact in float64."""
    q = np.asarray(q, dtype=np.float64)
    terms = np.maximum(q * np.asarray(kmin, dtype=np.float64), q * np.asarray(kmax, dtype=np.float64))
    return math.fsum(terms.tolist())


def group_page_score(q_group, kmin, kmax):
    """Score of a page for a KV head read by the query heads ``q_group`` [G, D]:
    the largest of their scores."""
    return max(page_score(q, kmin, kmax) for q in np.asarray(q_group))


def select_pages(scores, budget):
    """Indices of the ``budget`` highest scores in ascending order; on equal
    scores the lower index is kept; all indices when there are no more than
    ``budget``."""
    n = len(scores)
    if budget >= n:
        return list(range(n))
    order = sorted(range(n), key=lambda i: (-scores[i], i))
    return sorted(order[:budget])


def sequence_page_scores(q_group, keys, L, bs=16):
    """Scores of the pages of one sequence for one KV head.

    ``keys``: [L, D] that head's keys in logical order; page p holds tokens
    [p*bs, min((p+1)*bs, L))."""
    out = []
    for p in range((L + bs - 1) // bs):
        kmin, kmax = page_summary(keys[p * bs:min((p + 1) * bs, L)])
        out.append(group_page_score(q_group, kmin, kmax))
    return out


def quest_decode(q, K, V, L, budget, sm_scale, bs=16):
    """Decode of one sequence reading only its selected pages.

    ``q`` [Hq, D], ``K``/``V`` [L, Hkv, D] in logical order (float values).
    Returns (out [Hq, D] float32, selected pages per KV head)."""
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    Hkv = K.shape[1]
    out = np.zeros((Hq, D), dtype=np.float32)
    chosen = []
    for kvh in range(Hkv):
        heads = [h for h in range(Hq) if attention.kv_head_of(h, Hq, Hkv) == kvh]
        scores = sequence_page_scores(q[heads], K[:, kvh, :], L, bs)
        pages = select_pages(scores, budget)
        chosen.append(pages)
        toks = [t for p in pages for t in range(p * bs, min((p + 1) * bs, L))]
        if not toks:
            continue
        for h in heads:
            o, _ = attention.softmax_attention(q[h], K[toks, kvh], V[toks, kvh], sm_scale)
            out[h] = o.astype(np.float32)
    return out, chosen
