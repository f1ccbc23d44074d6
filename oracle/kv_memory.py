"""KV-cache size model (test infrastructure only; see package docstring).

[KVC] section "O gargalo de memória do KV Cache em contextos longos" gives the
size of a cache per sequence batch as a product: a factor 2 (keys and values),
the number of layers that hold a cache, the KV heads, the head dimension, the
number of cached positions, the bytes per element and the batch size.
[KVL] section "01 · Conceito" states the same model with its variables (two for K
plus V, L cached layers, T positions, H_kv heads, D, B bytes per element) and
works the Qwen-like example that the tests pin.
"""


def kv_cache_bytes(n_layers: int, n_kv_heads: int, head_dim: int, seq_len: int,
                   bytes_per_elem: int, batch: int = 1) -> int:
    """Bytes held by the K and V caches of ``n_layers`` attention layers."""
    return 2 * n_layers * n_kv_heads * head_dim * seq_len * bytes_per_elem * batch
