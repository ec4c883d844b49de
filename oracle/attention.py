"""Textbook attention over a paged KV cache (float64, CPU).

[TAI] section "Paged attention": the cache is kept in fixed-size blocks
(16 tokens) reached through a per-sequence block table, and the attention
kernel follows that table. [IR] section "PagedAttention: why fragmentation was
eating most of the rest": the table maps logical positions to physical blocks.
So logical token t of sequence s lives in slot
    table[s][t // 16] * 16 + t % 16
of the pool; gathering those slots in t order gives the contiguous K/V a
non-paged cache would hold.

Attention itself ([JE], the figure of attention as a soft query-key-value
lookup; [IR] section "What it is": the cache holds K and V of every previous
token) is read as standard scaled dot-product softmax attention with scale
1/sqrt(d_head): o = softmax(q K^T / sqrt(d)) V. GQA ([IR] "What it is" and the
table in "The memory equation"): query head h uses KV head h // G with
G = n_heads / n_kv_heads (contiguous groups).

Decode ([TAI] "The KV cache"): the new token's K/V are appended before the
step, so the single query attends to all context_lens[s] tokens; no mask.
Prefill chunk ([JE] "Chunked prefill"; [TAI] "Scheduling prefill and decode"):
the same attention split into pieces; query i of a chunk of q_len tokens sits
at absolute position ctx - q_len + i and attends to keys 0..position
(inclusive).

Sliding window ([IR] "The memory equation" lists sliding-window attention
among the ways to shrink the cache, with no formula; [TAI] "The KV cache"
names sliding-window layers): read as the query at position p attending only
the last W tokens, keys p - W + 1 .. p, so W = 1 is the token itself and
W >= p + 1 is full attention. The same rule holds for the decode's single
query and for every row of a prefill chunk.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Decode an input encoding to float64 exactly: 'f32' float32 values, or
    'bf16' uint16 bit patterns (the upper half of a float32)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def gather(pool: np.ndarray, table_row: np.ndarray, n: int, block_size: int = BLOCK) -> np.ndarray:
    """Contiguous copy of logical tokens 0..n-1 of one sequence."""
    t = np.arange(int(n))
    phys = np.asarray(table_row)[t // block_size].astype(np.int64)
    return pool[phys * block_size + t % block_size]


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(K q * scale) V for one query vector; max-subtracted (exactly
    the same value as the unshifted formula)."""
    z = (K @ q) * scale
    z = z - z.max()
    p = np.exp(z)
    p = p / p.sum()
    return p @ V


def paged_decode(q, k_pool, v_pool, block_tables, context_lens, *, n_kv: int,
                 block_size: int = BLOCK, scale: float | None = None, seqs=None,
                 window: int | None = None) -> np.ndarray:
    """Decode attention for every sequence (or the listed `seqs`).

    q [S, H, D] float64; k_pool/v_pool [num_blocks*block_size, n_kv, D]
    float64; returns float64 [S, H, D] (rows of unlisted sequences are NaN).
    A sequence with context length 0 gets a zero output row. With a window W
    the query (the last token, position n - 1) attends tokens max(0, n - W)
    .. n - 1 only.
    """
    q = np.asarray(q, dtype=np.float64)
    S, H, D = q.shape
    G = H // n_kv
    assert G * n_kv == H
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    out = np.full((S, H, D), np.nan)
    for s in (range(S) if seqs is None else seqs):
        n = int(context_lens[s])
        if n <= 0:
            out[s] = 0.0
            continue
        K = gather(k_pool, block_tables[s], n, block_size)  # [n, n_kv, D]
        V = gather(v_pool, block_tables[s], n, block_size)
        if window is not None:
            first = max(0, n - int(window))
            K, V = K[first:], V[first:]
        for h in range(H):
            kvh = h // G
            out[s, h] = softmax_attention(q[s, h], K[:, kvh, :], V[:, kvh, :], scale)
    return out


def paged_prefill(q, cu_q_lens, k_pool, v_pool, block_tables, context_lens, *, n_kv: int,
                  block_size: int = BLOCK, scale: float | None = None, rows=None,
                  window: int | None = None) -> np.ndarray:
    """Causal attention of a chunk of query tokens per sequence.

    q [total_q, H, D]; chunk of sequence s is rows cu[s]..cu[s+1]-1; returns
    float64 [total_q, H, D] (rows not listed in `rows` are NaN). With a
    sliding window W the row at position p attends keys max(0, p - W + 1) .. p
    (the decode's window, read for every row of the chunk).
    """
    q = np.asarray(q, dtype=np.float64)
    T, H, D = q.shape
    G = H // n_kv
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    out = np.full((T, H, D), np.nan)
    want = None if rows is None else np.asarray(sorted(set(int(r) for r in rows)), dtype=np.int64)
    for s in range(len(context_lens)):
        n = int(context_lens[s])
        lo, hi = int(cu_q_lens[s]), int(cu_q_lens[s + 1])
        qlen = hi - lo
        if qlen == 0:
            continue
        r = np.arange(lo, hi) if want is None else want[(want >= lo) & (want < hi)]
        if r.size == 0:
            continue
        pos = n - qlen + (r - lo)                      # absolute position of each row
        K = gather(k_pool, block_tables[s], n, block_size)
        V = gather(v_pool, block_tables[s], n, block_size)
        visible = np.arange(n)[None, :] <= pos[:, None]  # key t visible to row iff t <= pos
        if window is not None:
            visible &= np.arange(n)[None, :] > pos[:, None] - int(window)  # ... and t >= pos - W + 1
        for h in range(H):
            kvh = h // G
            # one softmax_attention per row, written as one matrix product
            z = (q[r, h, :] @ K[:, kvh, :].T) * scale
            z = np.where(visible, z, -np.inf)
            z = z - z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p = p / p.sum(axis=1, keepdims=True)
            out[r, h] = p @ V[:, kvh, :]
    return out
