"""The five synthetic workloads the library is measured and checked on.

Shapes follow the pages' own worked examples:
  * 70B-class layer (64 query heads, 8 KV heads, head dim 128) -- "KV cache,
    GQA, paging and continuous batching", section "The memory equation".
  * 16-token blocks -- "KV cache, continuous batching and paged attention",
    section "Paged attention".
  * 4,000-token shared system prompt -- "KV cache, GQA, paging and continuous
    batching", section "Prefix caching: the biggest single lever most teams
    have".
  * chunks of 512-2,048 tokens -- "KV cache, continuous batching and paged
    attention", section "Scheduling prefill and decode".
There is no public dataset behind these workloads; every value is a seeded
N(0, 1) draw.
"""

BLOCK_SIZE = 16

CONFIGS = {
    1: dict(
        name="tiny_fp32",
        workload="tiny fp32 paged decode: 4 q heads / 2 kv heads, d 64, ctx {5,17,33,40}, 32-block pool",
        n_heads=4, n_kv=2, d=64, dtype="f32",
        ctx=[5, 17, 33, 40], pool_blocks=32,
    ),
    2: dict(
        name="llama3_8b_bf16",
        workload="Llama-3-8B-shaped bf16 decode layer: 32 q / 8 kv heads, d 128, 64 seqs, ctx U[512,4096], pool 1.1x need",
        n_heads=32, n_kv=8, d=128, dtype="bf16",
        num_seqs=64, ctx_lo=512, ctx_hi=4096, pool_factor=1.1,
    ),
    3: dict(
        name="prefix_shared_70b_bf16",
        workload="70B-class bf16 decode layer with a shared 4000-token prefix: 64 q / 8 kv heads, d 128, 256 seqs, private tails U[200,500]",
        n_heads=64, n_kv=8, d=128, dtype="bf16",
        num_seqs=256, prefix_tokens=4000, tail_lo=200, tail_hi=500,
    ),
    4: dict(
        name="quant_kv_70b",
        workload="70B-class decode layer with int8 / int4 KV: 64 q / 8 kv heads, d 128, 128 seqs x 8000 tokens",
        n_heads=64, n_kv=8, d=128, dtype="bf16",
        num_seqs=128, ctx_fixed=8000, kv_bits=(8, 4),
    ),
    5: dict(
        name="mixed_chunked_prefill_bf16",
        workload="mixed step: one 2048-token causal chunk over 6000 cached tokens + 64 decode seqs, lognormal median 2048 clipped [128,16384]; 32 q / 8 kv heads, d 128",
        n_heads=32, n_kv=8, d=128, dtype="bf16",
        chunk_tokens=2048, cached_tokens=6000,
        decode_seqs=64, decode_median=2048, decode_sigma=1.0, decode_lo=128, decode_hi=16384,
    ),
}


def config_seed(index: int) -> int:
    """Seed of workload `index` (1..5)."""
    return 4290 + int(index)
