"""Cache-size and paging arithmetic, as the pages state it.

[TAI] section "The KV cache" and [IR] section "The memory equation":
    KV bytes per token = 2 (K and V) x L x n_kv_heads x d_head x bytes
    cache bytes        = 2 x L x H_kv x d_head x S x B x b
[TAI] section "Paged attention": waste is at most one partly filled block
per sequence. [IR] section "PagedAttention: why fragmentation was eating most
of the rest": a naive allocator reserves max_seq_len per request.
[IR] section "Prefix caching: the biggest single lever most teams have":
a cached prefix removes its share of prefill work.
"""
from __future__ import annotations

BLOCK = 16


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, d_head: int, bytes_per_elem: float) -> float:
    return 2 * n_layers * n_kv_heads * d_head * bytes_per_elem


def cache_bytes(n_layers: int, n_kv_heads: int, d_head: int, seq_len: int, batch: int, bytes_per_elem: float) -> float:
    return 2 * n_layers * n_kv_heads * d_head * seq_len * batch * bytes_per_elem


def blocks_needed(n_tokens: int, block_size: int = BLOCK) -> int:
    return -(-int(n_tokens) // block_size)


def paged_waste_slots(n_tokens: int, block_size: int = BLOCK) -> int:
    """Unused slots in a sequence's last block."""
    return blocks_needed(n_tokens, block_size) * block_size - int(n_tokens)


def paged_cache_bytes(n_layers: int, n_kv_heads: int, d_head: int, n_tokens: int, kv_bits: int,
                      block_size: int = BLOCK) -> int:
    """Bytes a paged cache holds for one sequence of n_tokens: whole blocks
    of K and V, plus one fp16 scale per (block, KV head) for K and for V when
    the cache is quantized (kv_bits < 16)."""
    nb = blocks_needed(n_tokens, block_size)
    per_tile = block_size * d_head * kv_bits // 8 + (2 if kv_bits < 16 else 0)
    return 2 * n_layers * nb * n_kv_heads * per_tile


def naive_untouched_fraction(max_seq_len: int, used_tokens: int) -> float:
    """Share of a max_seq_len reservation that a request never touches."""
    return 1.0 - used_tokens / max_seq_len


def prefix_prefill_saving(prefix_tokens: int, query_tokens: int) -> float:
    """Share of prefill work removed when the prefix is served from cache."""
    return prefix_tokens / (prefix_tokens + query_tokens)
