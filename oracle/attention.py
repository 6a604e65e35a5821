"""Textbook decode attention over a paged cache (oracle, test-only).

What is computed ("KV Cache Engineering for LLM Serving", section 1 "GQA and
MQA cache fewer heads"): the current token's query is compared with every
cached key; the comparisons give attention weights; the weights combine the
cached values.  Paging only changes where keys and values live, so the result
is exactly softmax attention over the sequence's tokens in logical order.

GQA (same section): query head ``h`` reads KV head ``h // (Hq // Hkv)``.

Several query tokens per sequence (``multi_query_decode``): each new token
sees the cache up to and including its own position.

StreamingLLM keep-mask ("Chapter 18 - KV-Cache Optimization Strategies",
section "Token Eviction and Pruning"): the first ``sink`` tokens plus the most
recent ``window`` tokens (4 + 4092 = 4096 entries in the page's layout).

Grouped scales (``paged_decode_grouped``): keys dequantised with one scale
per (block, KV head, channel), values with one per (block, KV head, token).

Arithmetic: every value is decoded exactly to float32 (``codecs.decode``,
``quant.dequantize``) and the attention itself runs in float64.  The result is
stored as float32.  A sequence of length 0 yields a zero output row.
"""

import numpy as np

from . import codecs, paging, quant


def kv_head_of(q_head, num_q_heads, num_kv_heads):
    """GQA head mapping: ``q_head // (num_q_heads // num_kv_heads)``."""
    return q_head // (num_q_heads // num_kv_heads)


def kept_positions(length, sink=0, window=0):
    """Logical positions that take part in attention.

    Full attention (``sink == window == 0``): all ``t < length``.
    StreamingLLM variant: ``t < sink`` or ``t >= length - window``.
    """
    length = int(length)
    t = np.arange(length, dtype=np.int64)
    if sink == 0 and window == 0:
        return t
    keep = (t < sink) | (t >= length - window)
    return t[keep]


def softmax_attention(q, K, V, sm_scale):
    """Single-query softmax attention in float64.

    ``q``: [D]; ``K``, ``V``: [T, D].  Returns (out [D], p [T]) where
    ``s_t = sm_scale * (q . K_t)``, ``p = exp(s - max s) / sum exp(s - max s)``
    and ``out = sum_t p_t V_t``.  T == 0 gives a zero output.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64), np.zeros(0, dtype=np.float64)
    s = float(sm_scale) * (K @ q)
    e = np.exp(s - s.max())
    p = e / e.sum()
    return p @ V, p


def decode_sequence(q_rows, K_seq, V_seq, sm_scale, sink=0, window=0):
    """Decode attention for one sequence.

    ``q_rows``: [Hq, D] decoded query; ``K_seq``/``V_seq``: [L, Hkv, D]
    decoded keys/values in logical order.  Returns float32 [Hq, D].
    """
    Hq, D = q_rows.shape
    L, Hkv, _ = K_seq.shape
    kept = kept_positions(L, sink, window)
    out = np.zeros((Hq, D), dtype=np.float64)
    for h in range(Hq):
        kvh = kv_head_of(h, Hq, Hkv)
        out[h], _ = softmax_attention(q_rows[h], K_seq[kept, kvh], V_seq[kept, kvh], sm_scale)
    return out.astype(np.float32)


def decoded_cache_rows(cache, table_row, length, block_size, dtype, scales=None):
    """Gather one sequence's raw rows in logical order and decode them to
    exact float32 values, applying the per-(block, kv-head) scale when the
    cache holds quantised codes.  Returns [L, Hkv, D] float32."""
    raw = paging.gather_sequence(cache, table_row, length, block_size)
    vals = codecs.decode(raw, dtype)
    if dtype in quant.CODE_DTYPES:
        if scales is None:
            raise ValueError("quantised cache needs scales")
        L = int(length)
        blocks = np.asarray([table_row[t // block_size] for t in range(L)], dtype=np.int64)
        sc = np.asarray(scales, dtype=np.float32)[blocks] if L else np.zeros((0, vals.shape[1]), np.float32)
        vals = quant.dequantize(vals, sc[:, :, None])
    return vals


def decoded_cache_rows_grouped(cache, table_row, length, block_size, dtype, group_scales, group):
    """One sequence's rows in logical order, dequantised with grouped scales
    (``quant.quantize_cache_blocks_grouped``): ``group_scales`` [NB, Hkv, D]
    for "channel", [NB, Hkv, BS] for "token".  Returns [L, Hkv, D] float32."""
    L = int(length)
    Hkv = cache.shape[2]
    out = []
    for lb in range((L + block_size - 1) // block_size):
        b = int(table_row[lb])
        vals = codecs.decode(cache[b], dtype)                        # [BS, Hkv, D]
        tile = np.stack([quant.dequantize_grouped(vals[:, h, :], group_scales[b, h], group)
                         for h in range(Hkv)], axis=1)
        out.append(tile[: min(block_size, L - lb * block_size)])
    D = vals.shape[-1] if out else cache.shape[3] * (2 if dtype == "i4" else 1)
    return np.concatenate(out) if out else np.zeros((0, Hkv, D), np.float32)


def paged_decode_grouped(query, q_dtype, k_cache, v_cache, kv_dtype, block_tables, seq_lens, block_size,
                         sm_scale, k_channel_scales, v_token_scales):
    """``paged_decode`` over a cache quantised with grouped scales: keys with
    one scale per (block, KV head, channel), values with one per (block, KV
    head, token).  Returns float32 [S, Hq, D]."""
    qv = codecs.decode(query, q_dtype)
    S, Hq, D = qv.shape
    out = np.zeros((S, Hq, D), dtype=np.float32)
    for s in range(S):
        L = int(seq_lens[s])
        K = decoded_cache_rows_grouped(k_cache, block_tables[s], L, block_size, kv_dtype, k_channel_scales,
                                       "channel")
        V = decoded_cache_rows_grouped(v_cache, block_tables[s], L, block_size, kv_dtype, v_token_scales,
                                       "token")
        out[s] = decode_sequence(qv[s], K, V, sm_scale)
    return out


def paged_decode(query, q_dtype, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                 block_size, sm_scale, k_scales=None, v_scales=None, sink=0, window=0,
                 seqs=None):
    """Paged decode attention for a batch (or the subset ``seqs``).

    ``query``: raw [S, Hq, D]; caches raw [NB, BS, Hkv, D]; ``block_tables``
    [S, MBS]; ``seq_lens`` [S].  Returns float32 [S, Hq, D] (rows of
    sequences not in ``seqs`` are left zero).
    """
    qv = codecs.decode(query, q_dtype)
    S, Hq, D = qv.shape
    out = np.zeros((S, Hq, D), dtype=np.float32)
    for s in (range(S) if seqs is None else seqs):
        L = int(seq_lens[s])
        K = decoded_cache_rows(k_cache, block_tables[s], L, block_size, kv_dtype, k_scales)
        V = decoded_cache_rows(v_cache, block_tables[s], L, block_size, kv_dtype, v_scales)
        out[s] = decode_sequence(qv[s], K, V, sm_scale, sink, window)
    return out


def multi_query_decode(query, q_dtype, k_cache, v_cache, kv_dtype, block_tables, seq_lens, block_size,
                       sm_scale, k_scales=None, v_scales=None):
    """Several new tokens per sequence attending to the paged cache (a
    speculative-decode check or a short chunk of prefill; the pages stop at
    one token per step, this is the plain causal reading).

    ``query``: raw [S, T, Hq, D]; ``seq_lens[s]`` counts the T new tokens,
    whose keys and values are already in the cache at positions
    L - T .. L - 1.  Token t sees the positions 0 .. L - T + t.  Returns
    float32 [S, T, Hq, D]."""
    qv = codecs.decode(query, q_dtype)
    S, T, Hq, D = qv.shape
    out = np.zeros((S, T, Hq, D), dtype=np.float32)
    for s in range(S):
        L = int(seq_lens[s])
        K = decoded_cache_rows(k_cache, block_tables[s], L, block_size, kv_dtype, k_scales)
        V = decoded_cache_rows(v_cache, block_tables[s], L, block_size, kv_dtype, v_scales)
        for t in range(T):
            n = L - T + t + 1
            if n <= 0:
                continue
            out[s, t] = decode_sequence(qv[s, t], K[:n], V[:n], sm_scale)
    return out


# ---------------------------------------------------------------------------
# split-K formulation: per-partition partials and their log-sum-exp merge
# ---------------------------------------------------------------------------

def partition_partials(q, K, V, sm_scale, positions, partition_size):
    """Per-partition partial softmax state for one (sequence, query head).

    Tokens are grouped by ``t // partition_size`` (partition boundaries are
    multiples of ``partition_size`` from t = 0).  For partition p over the kept
    positions ``positions`` that fall in it: ``m_p = max s_t``,
    ``l_p = sum exp(s_t - m_p)``, ``acc_p = sum exp(s_t - m_p) V_t``.  An empty
    partition has m = -inf, l = 0, acc = 0.  ``K``/``V`` are [T, D] rows for
    ``positions``.  Returns (m [P], l [P], acc [P, D]) in float64, with P the
    number of partitions covering the positions' range.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    n_part = int(positions.max()) // partition_size + 1 if positions.size else 0
    m = np.full(n_part, -np.inf)
    l = np.zeros(n_part)
    acc = np.zeros((n_part, V.shape[1]))
    s = float(sm_scale) * (K @ q)
    for p in range(n_part):
        sel = (positions // partition_size) == p
        if not sel.any():
            continue
        m[p] = s[sel].max()
        e = np.exp(s[sel] - m[p])
        l[p] = e.sum()
        acc[p] = e @ V[sel]
    return m, l, acc


def merge_partials(m, l, acc):
    """Log-sum-exp merge: ``M = max m_p``; ``out = sum_p e^(m_p - M) acc_p /
    sum_p e^(m_p - M) l_p``.  Empty partitions (m = -inf) contribute nothing;
    if every partition is empty the output is zero."""
    m = np.asarray(m, dtype=np.float64)
    if m.size == 0 or not np.isfinite(m).any():
        return np.zeros(np.asarray(acc).shape[-1])
    M = m[np.isfinite(m)].max()
    w = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m - M, 0.0)), 0.0)
    return (w @ np.asarray(acc, dtype=np.float64)) / (w @ np.asarray(l, dtype=np.float64))
