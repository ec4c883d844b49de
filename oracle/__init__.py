"""CPU oracle for paged decode attention, chunked prefill and KV quantization.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports, links or calls this
package; only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may. It is deliberately plain and slow:
each sequence is gathered through its block table into contiguous K/V, then
textbook softmax attention runs in float64 with BLAS matrix products. It
shares no code with the HIP path and knows nothing of the library's device
memory layout: pools are given in slot form ``pool[block * 16 + offset, kv_head, :]``.

Sources (three web pages on KV caching; cited by title and section):
  [TAI] "KV cache, continuous batching and paged attention"
        (techaiinterview.com, inference & serving)
  [IR]  "KV cache, GQA, paging and continuous batching"
        (interview reference, 05-ai-llm)
  [JE]  jovanaeducation.com inference guide a2-inf-2 (sections "PagedAttention:
        virtual memory for the cache", "Prefix caching", "Chunked prefill",
        "KV-cache quantization")

Pinning status (what each function is checked against lives in tests/):
  attention.paged_decode   pinned: pure-Python brute force, closed forms,
                           MHA/GQA/MQA reductions, permutation and sharing
                           invariants, retrieval probes.
  attention.paged_prefill  pinned: brute force, last-row == decode, split
                           invariance, causal probe.
  quantize.quantize_tiles  pinned: independent pure-Python brute force
                           (struct-based float32/float16 rounding), invariants.
  quantize.*fp8, e4m3_*    pinned: the format's defining values, brute-force
                           nearest search over all codes, ties, saturation,
                           invariants of the quantized tiles.
  formulas.*               pinned: the pages' printed worked values.
  cache_write.*            pinned: pure-Python brute force of the slot rule,
                           appends in steps == one append, the brute-force
                           quantizer on zero-filled partly written tiles.
  The softmax scale 1/sqrt(d_head) is a reading (the pages lose the formula);
  it is fixed by convention, not by a printed value.
"""
from .attention import as_f64, paged_decode, paged_prefill, softmax_attention, gather  # noqa: F401
from .quantize import quantize_tiles, dequantize, QMAX  # noqa: F401
from .quantize import (E4M3_MAX, e4m3_value, e4m3_round, quantize_tiles_fp8,  # noqa: F401
                       dequantize_fp8)
from . import formulas  # noqa: F401
from . import cache_write  # noqa: F401
from . import brute  # noqa: F401
