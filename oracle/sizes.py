"""KV-cache size arithmetic.

[ch7] 7.1 「KV cache 的数学」 and 「KV cache 显存估算」: the K and V of one token take
2 x layers x KV heads x head_dim x bytes-per-element; a cache of n tokens takes n times that.
"""


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """Bytes of K plus V for one token over all layers ([ch7] 7.1 core formula)."""
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


def kv_cache_bytes(num_layers: int, num_kv_heads: int, head_dim: int, num_tokens: int,
                   dtype_bytes: int) -> int:
    """Bytes of K plus V for `num_tokens` tokens ([ch7] 7.1 「KV cache 显存估算」)."""
    return kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype_bytes) * num_tokens
