"""Seeded synthetic inputs for paged decode attention and chunked prefill.

This package is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds random draws, block-table construction, permutations and
storage-format conversion of inputs (float32 -> bfloat16 bit patterns) only:
none of the attention or quantization arithmetic lives here.
"""
from .gen import (  # noqa: F401
    DecodeCase,
    PrefillCase,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_decode_case,
    make_config_case,
    make_clustered_prefix_case,
    make_mixed_case,
    make_prefill_case,
    make_probe_case,
    make_prefill_probe_case,
    make_prefix_probe_case,
    permute_pool,
    poison_unused,
    private_twin,
    privatize,
    used_slot_mask,
)
from .configs import CONFIGS, config_seed  # noqa: F401
