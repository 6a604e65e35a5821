"""KV cache-size formula (oracle, test-only).

Learning-AI topic t13_4, cache-size paragraph, and "KV Cache Engineering for
LLM Serving", section "The cache formula": the raw cache of one sequence is
2 (keys and values) x layers x heads x head dimension x tokens x bytes per
element.  The head count that matters is the number of KV heads: GQA shrinks
exactly this term (section 1: 64 query heads with 8 KV heads give 40 GB
instead of 320 GB at 128K tokens).
"""


def kv_cache_bytes(num_layers, num_kv_heads, head_dim, num_tokens, bytes_per_element):
    """Bytes of K plus V for one sequence."""
    return 2 * num_layers * num_kv_heads * head_dim * num_tokens * bytes_per_element


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, bytes_per_element):
    return kv_cache_bytes(num_layers, num_kv_heads, head_dim, 1, bytes_per_element)


def block_bytes(block_size, num_kv_heads, head_dim, bytes_per_element):
    """One physical block of one layer, K and V ("Chapter 18", "Physical KV
    Block" figure: 2 x 16 x 8 x 128 x 2 B = 64 KB)."""
    return 2 * block_size * num_kv_heads * head_dim * bytes_per_element


def tokens_in_pool(pool_bytes, bytes_per_token):
    """Whole tokens that fit in a fixed pool ("KV Cache Engineering", section
    10: an 8 GB pool at 320 KB or 160 KB per token)."""
    return pool_bytes // bytes_per_token
