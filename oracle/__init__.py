"""CPU oracle for paged-KV decode attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the paged-KV decode path computes, written from the
pages' descriptions.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the HIP
library and its Python binding) never imports, links or calls anything here,
and nothing here imports the product path.

Sources (cited by page title and section):

* "Chapter 18 - KV-Cache Optimization Strategies" (Language Modelling - The
  Complete Guide): sections "How PagedAttention Works" (with the "Physical KV
  Block" figure), "Prefix Caching", "KV-Cache Quantization", "Token Eviction
  and Pruning" (StreamingLLM cache layout).
* "KV Cache Engineering for LLM Serving, clearly explained": "The cache
  formula", section 1 "GQA and MQA cache fewer heads", section 3 "Sliding
  windows", section 7 "Query-aware sparse reads", section 8 "Quantization",
  section 9 "Eviction", section 10 "Paging", section 11 "Prefix reuse".
* Learning-AI topic t13_4 (KV cache management): the cache-size formula
  paragraph, the block-table paragraph and its example, and the
  copy-on-write paragraph.

Modules:

* ``codecs``    - exact decoders of bf16 / fp16 / FP8-e4m3 / FP8-e5m2 /
                  packed INT4 storage, and the brute-force FP8
                  round-to-nearest-even encoders.
* ``paging``    - slot addressing, gather in logical order, the slot write
                  (reshape_and_cache) and whole-block copy (copy-on-write).
* ``attention`` - textbook softmax attention in float64 over the gathered
                  sequence, GQA head mapping, StreamingLLM keep-mask, and the
                  split-K partial/merge formulation.
* ``quant``     - the symmetric absmax quantiser (INT8, INT4, FP8-e4m3 and
                  FP8-e5m2 codes) with one scale per block tile or grouped
                  scales (K per channel, V per token), and the
                  requantisation of a growing block.
* ``pool``      - FIFO free-block pool with reference counts and
                  copy-on-write append.
* ``sizes``     - the KV cache-size formula.
* ``quest``     - query-aware page selection: per-page key minimum /
                  maximum, the page score, top-budget selection, and decode
                  over the selected pages.
* ``reuse``     - full-prefix block keys and their cache; H2O retention of
                  the recent positions plus the older heavy hitters.

Every function here is pinned by tests in ``tests/test_oracle_*.py`` against
values the pages print, closed forms, invariants, library routines
(``torch.nn.functional.scaled_dot_product_attention`` on CPU, torch's
``float8_e4m3fn`` and ``float8_e5m2`` casts) or brute force.  No function is "parity unpinned".
"""

from . import attention, codecs, paging, pool, quant, quest, reuse, sizes  # noqa: F401
