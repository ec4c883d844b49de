"""Appending new tokens' keys and values to a paged KV cache (CPU).

TEST INFRASTRUCTURE ONLY, like the rest of this package: nothing in the
library imports or calls it.

[TAI] section "The KV cache": each step computes K and V only for the new
token and appends them to the cache; a prefill chunk appends its tokens the
same way. [IR] section "PagedAttention: why fragmentation was eating most of
the rest": the block table maps logical positions to physical blocks, so the
token at position t of sequence s goes to slot

    block_tables[s][t // 16] * 16 + t % 16.

The new tokens of sequence s are its last n_s positions, ctx_s - n_s ..
ctx_s - 1, where ctx_s is its length after the append.

Quantized pools ([JE] section "KV-cache quantization": each key/value is an
integer sharing one scale with its group, one (block, KV head) tile here).
The pages do not say how a block that fills one token at a time keeps its
scale. Reading: at every moment a block's codes and scale are those that
quantize_tiles gives for the tokens written into it so far, the slots not
yet written counting as 0. So each write into a block recomputes its scale
(and every code of the block), and once the block holds 16 tokens it is
exactly the block kv_quantize would produce from its bf16 tokens.
"""
from __future__ import annotations

import numpy as np

from .quantize import quantize_tiles, quantize_tiles_fp8

BLOCK = 16


def new_token_slots(block_tables, context_lens, cu_new, block_size: int = BLOCK) -> np.ndarray:
    """Slot of every new token, in the order of the new-token rows: rows
    cu_new[s] .. cu_new[s+1]-1 are sequence s's positions
    context_lens[s] - n_s .. context_lens[s] - 1 (n_s = cu_new[s+1] - cu_new[s])."""
    cu = np.asarray(cu_new, dtype=np.int64)
    out = np.empty(int(cu[-1]), dtype=np.int64)
    for s in range(len(cu) - 1):
        n = int(cu[s + 1] - cu[s])
        if n == 0:
            continue
        ctx = int(context_lens[s])
        pos = np.arange(ctx - n, ctx, dtype=np.int64)
        out[cu[s]:cu[s + 1]] = np.asarray(block_tables[s], dtype=np.int64)[pos // block_size] * block_size \
            + pos % block_size
    return out


def append(pool_slots: np.ndarray, written: np.ndarray, new_rows: np.ndarray, slots: np.ndarray):
    """The pool (slot form [num_blocks*16, n_kv, d]) and its written-slot mask
    after writing new_rows[i] into slots[i]; inputs are not modified."""
    pool = pool_slots.copy()
    w = written.copy()
    pool[slots] = new_rows
    w[slots] = True
    return pool, w


def quantized_state(values_slots: np.ndarray, written: np.ndarray, bits) -> tuple:
    """Codes and scales of every block of a quantized pool whose written slots
    hold values_slots (float32 slot form) and whose other slots count as 0.
    bits: 8, 4 or 'fp8'."""
    x = np.where(written[:, None, None], np.asarray(values_slots, dtype=np.float32), np.float32(0))
    if bits == "fp8":
        return quantize_tiles_fp8(x)
    return quantize_tiles(x, bits)
