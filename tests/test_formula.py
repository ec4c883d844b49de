"""Oracle cache-size and paging arithmetic against the pages' printed values."""
import json
import math
import os

import numpy as np
import pytest

from oracle import formulas as F
from synth import make_config_case

GOLD = os.path.join(os.path.dirname(__file__), "golden")
GIB = 1 << 30


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_bytes_per_token_worked_values():
    g = _load("kv_cache_worked_values.json")
    for row in g["per_token"]:
        got = F.kv_bytes_per_token(row["layers"], row["kv_heads"], row["d_head"], row["bytes"])
        assert got == row["bytes_per_token"], row
    mha, gqa, mqa = (r["bytes_per_token"] for r in g["per_token"])
    assert mha == 2.5 * (1 << 20)
    assert gqa == 320 * 1024 and mqa == 40 * 1024
    assert mha // gqa == g["gqa_capacity_multiplier"]


def test_cache_bytes_equation_matches_per_token_form():
    # cache bytes = 2 L H_kv d S B b, linear in every factor
    for L, h, d, S, B, b in [(80, 8, 128, 8192, 1, 2), (32, 8, 128, 4096, 64, 2), (1, 1, 64, 5, 3, 4)]:
        assert F.cache_bytes(L, h, d, S, B, b) == F.kv_bytes_per_token(L, h, d, b) * S * B


def test_per_sequence_gib_at_8k():
    g = _load("kv_cache_worked_values.json")
    n = g["per_sequence_8k_tokens"]
    gib = {r["scheme"]: F.cache_bytes(r["layers"], r["kv_heads"], r["d_head"], n, 1, r["bytes"]) / GIB
           for r in g["per_token"]}
    assert gib["MHA"] == g["per_sequence_gib"]["MHA"]
    assert gib["GQA"] == g["per_sequence_gib"]["GQA"]
    assert gib["MQA"] == g["per_sequence_gib"]["MQA_exact"]
    assert round(gib["MQA"], 1) == g["per_sequence_gib"]["MQA_printed"]
    # the page's concurrency: 180 / printed per-sequence figure
    for k, printed in (("MHA", 20), ("GQA", 2.5), ("MQA", 0.3)):
        assert math.floor(g["free_for_cache_gb"] / printed + 1e-9) == g["concurrent_sequences"][k]


def test_deployment_sizing():
    g = _load("deployment_sizing.json")
    per_tok = F.kv_bytes_per_token(80, 8, 128, 2)
    assert per_tok == g["kib_per_token"] * 1024
    gib = F.cache_bytes(80, 8, 128, g["context_tokens_reading"], 1, 2) / GIB
    assert gib == g["gib_per_sequence"]
    assert round(gib, 2) == g["gib_per_sequence_printed"]
    per_node = g["available_gb"] / g["gib_per_sequence_printed"]
    assert abs(per_node - g["sequences_per_node_printed"]) < 1
    # fp8 halves the cache (1 byte per element)
    assert F.kv_bytes_per_token(80, 8, 128, 1) * 2 == per_tok
    assert abs(2 * per_node - g["fp8_sequences_per_node_printed"]) < 2
    # 70B GQA with ~450 GB of cache: ~340 at 4k (4096: 335; 4000: 343), ~10 at 128k
    at4k = g["kv_budget_gb_8x80"] * 1e9 / (per_tok * 4096)
    at4000 = g["kv_budget_gb_8x80"] * 1e9 / (per_tok * 4000)
    at128k = g["kv_budget_gb_8x80"] * 1e9 / (per_tok * 131072)
    assert at4k < g["seqs_at_4k_printed"] < at4000
    assert math.floor(at128k) == g["seqs_at_128k_printed"]


def test_block_table_diagram_waste():
    g = _load("block_table_diagram.json")
    bs = g["block_size"]
    used = set()
    for name, s in g["sequences"].items():
        assert F.blocks_needed(s["n_tokens"], bs) == len(s["table"])
        assert F.paged_waste_slots(s["n_tokens"], bs) == s["waste_slots"]
        used |= set(s["table"])
    assert not used & set(g["free_blocks"])
    partly = [s["table"][-1] for s in g["sequences"].values() if F.paged_waste_slots(s["n_tokens"], bs)]
    assert partly == g["partly_filled_blocks"]


def test_naive_reservation_and_prefix_saving():
    g = _load("paging_and_prefix_worked.json")
    frac = F.naive_untouched_fraction(g["naive"]["max_seq_len"], g["naive"]["avg_tokens"])
    assert round(100 * frac) == g["naive"]["untouched_percent_printed"]
    sav = F.prefix_prefill_saving(g["prefix"]["prefix_tokens"], g["prefix"]["query_tokens"])
    assert round(100 * sav) == g["prefix"]["saving_percent_printed"]


@pytest.mark.parametrize("n", list(range(1, 70)) + [4000, 4096, 8000, 8048, 16384])
def test_waste_bound(n):
    g = _load("paging_and_prefix_worked.json")
    w = F.paged_waste_slots(n)
    assert 0 <= w <= g["max_waste_slots_per_sequence"]
    assert (w == 0) == (n % 16 == 0)


def test_quantized_footprint_ratio():
    g = _load("paging_and_prefix_worked.json")
    for bits, ratio in g["quant_footprint_ratio"].items():
        b = int(bits)
        codes = F.paged_cache_bytes(80, 8, 128, 8000, b) - 2 * 80 * 500 * 8 * 2  # minus the scales
        full = F.paged_cache_bytes(80, 8, 128, 8000, 16)
        assert codes / full == ratio
    # scale overhead: one fp16 per (block, head) for K and V = 2 bytes per 16 tokens per head
    assert F.paged_cache_bytes(1, 8, 128, 16, 8) == 2 * 8 * (16 * 128 + 2)


def test_workload_pools_match_formula():
    # every workload 1 sequence occupies whole blocks; waste per sequence matches
    c = make_config_case(1)
    assert [F.paged_waste_slots(n) for n in c.context_lens] == [11, 15, 15, 8]
    assert c.k_slots.nbytes == c.num_blocks * 16 * F.kv_bytes_per_token(1, 2, 64, 4) / 2
    assert int((c.block_tables >= 0).sum()) == sum(F.blocks_needed(n) for n in c.context_lens) == 9


@pytest.mark.parametrize("bits,n_tokens,n_kv,d", [(8, 8000, 8, 128), (4, 8000, 8, 128), (8, 17, 2, 64), (4, 1, 4, 64)])
def test_cache_bytes_counted_from_the_stored_arrays(bits, n_tokens, n_kv, d):
    """paged_cache_bytes against a count of what a quantized cache stores for
    one sequence of one layer: the code tiles of its whole blocks, built with
    the tests' own statement of the pool layout, and one fp16 scale per
    (block, KV head), for K and for V."""
    from tests.layout_ref import pack_pool
    nb = -(-n_tokens // 16)
    codes = np.zeros((nb * 16, n_kv, d), dtype=np.int8)
    stored = 0
    for kind in ("k", "v"):
        stored += pack_pool(codes, kind, bits).nbytes
        stored += np.zeros((nb, n_kv), dtype=np.float16).nbytes
    assert F.paged_cache_bytes(1, n_kv, d, n_tokens, bits) == stored
