"""KV-cache size closed forms [P3 §1.5], in the GQA form [P1 §04].

TEST INFRASTRUCTURE ONLY (see the package docstring).

[P3 §1.5] gives the bytes of KV cache per token as
2 (K and V) x layers x (heads x head_dim) x bytes per element, and the total
for a batch as batch x sequence length x that. Only the KV heads are cached,
so under GQA the head count in that product is the number of KV heads: P1 §04
notes that Llama-3-8B's 8 KV heads for 32 query heads shrink the cache to a
quarter. With ``num_kv_heads == num_heads`` (MHA) the two readings agree.
"""


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       elem_bytes: int) -> int:
    """Bytes of cached K plus V for one token over all layers."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def total_kv_bytes(batch: int, seq_len: int, num_layers: int, num_kv_heads: int,
                   head_dim: int, elem_bytes: int) -> int:
    """Bytes of KV cache for ``batch`` sequences of ``seq_len`` tokens."""
    return batch * seq_len * kv_bytes_per_token(num_layers, num_kv_heads, head_dim,
                                                elem_bytes)


def paged_cache_bytes(num_blocks: int, block_size: int, num_kv_heads: int,
                      head_dim: int, elem_bytes: int, num_layers: int = 1) -> int:
    """Bytes of a paged pool ``[layers, 2, num_blocks, block_size, Hkv, D]`` [P1 §02]."""
    return num_layers * 2 * num_blocks * block_size * num_kv_heads * head_dim * elem_bytes
