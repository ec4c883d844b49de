"""Paged-KV-cache attention for AMD Instinct MI355X (gfx950).

The compute lives in libpagedattn.so (hand-written HIP, C ABI declared in
include/paged_attn.h); `binding` is its thin ctypes wrapper.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    PagedAttnError,
    alloc_pool,
    alloc_scales,
    decode,
    kv_write,
    prefill_chunk,
    quantize,
)
