"""Pins of the cache-append oracle (oracle/cache_write.py): slot numbers
against a pure-Python brute force of the block-table rule, appends in steps
against one append, and the quantized state of partly written blocks against
the brute-force quantizer on zero-filled tiles."""
import numpy as np
import pytest

from oracle import brute
from oracle import cache_write as W
from synth import make_decode_case
from synth.gen import bf16_bits_to_f32


def _brute_slots(tables, ctx, cu):
    out = []
    for s in range(len(ctx)):
        n = int(cu[s + 1]) - int(cu[s])
        for i in range(n):
            t = int(ctx[s]) - n + i
            out.append(int(tables[s][t // 16]) * 16 + t % 16)
    return out


@pytest.mark.parametrize("seed", range(4))
def test_new_token_slots_vs_brute_force(seed):
    g = np.random.default_rng(700 + seed)
    ctx = g.integers(1, 90, size=5)
    n_new = [int(g.integers(0, c + 1)) for c in ctx]
    c = make_decode_case(4, 2, 8, "f32", ctx, 710 + seed, pool_factor=1.5)
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int64)
    got = W.new_token_slots(c.block_tables, c.context_lens, cu)
    assert got.tolist() == _brute_slots(c.block_tables.tolist(), ctx.tolist(), cu.tolist())
    assert len(set(got.tolist())) == len(got)  # no two tokens share a slot


def _grow(c, steps):
    """Write the case's own slot values into an empty pool in the given
    appends: steps is a list of (lengths after the append) per sequence."""
    pool = np.zeros_like(c.k_slots)
    written = np.zeros(c.k_slots.shape[0], dtype=bool)
    prev = np.zeros(c.num_seqs, dtype=np.int64)
    for after in steps:
        after = np.asarray(after, dtype=np.int64)
        n = after - prev
        cu = np.concatenate([[0], np.cumsum(n)])
        slots = W.new_token_slots(c.block_tables, after, cu)
        pool, written = W.append(pool, written, c.k_slots[slots], slots)
        prev = after
    return pool, written


def test_appends_in_steps_equal_one_append():
    """A prompt chunk then single-token decode steps crossing block
    boundaries leave the same pool as writing every token at once."""
    c = make_decode_case(4, 2, 8, "f32", [40, 17, 33], 720, pool_factor=1.5)
    full = c.context_lens.astype(np.int64)
    steps = [[30, 5, 16]] + [[min(30 + k, 40), min(5 + k, 17), min(16 + k, 33)] for k in range(1, 18)]
    assert steps[-1] == full.tolist()
    a, wa = _grow(c, steps)
    b, wb = _grow(c, [full])
    assert np.array_equal(wa, wb) and np.array_equal(a, b)
    # exactly the slots the sequences read are written, and hold the case's values
    from synth import used_slot_mask
    assert np.array_equal(wa, used_slot_mask(c))
    assert np.array_equal(a[wa], c.k_slots[wa])


@pytest.mark.parametrize("bits", [8, 4, "fp8"])
def test_quantized_state_of_partly_written_blocks(bits):
    """Blocks with 1, 7, 15 and 16 written slots: codes and scale equal the
    brute-force quantizer's on the tile with unwritten slots set to 0;
    unwritten slots hold code 0; whatever the unwritten slots of the pool
    hold does not matter."""
    c = make_decode_case(4, 2, 8, "bf16", [1, 7, 15, 16], 730, pool_blocks=4)
    vals = bf16_bits_to_f32(c.k_slots)
    written = np.zeros(vals.shape[0], dtype=bool)
    for s, n in enumerate([1, 7, 15, 16]):
        b = int(c.block_tables[s, 0])
        written[b * 16:b * 16 + n] = True
    codes, scales = W.quantized_state(vals, written, bits)
    garbage = np.where(written[:, None, None], vals, np.float32(1e4))
    codes2, scales2 = W.quantized_state(garbage, written, bits)
    assert np.array_equal(codes, codes2) and np.array_equal(scales.view(np.uint16), scales2.view(np.uint16))
    q = brute.quantize_tile_fp8 if bits == "fp8" else (lambda v: brute.quantize_tile(v, bits))
    for b in range(4):
        for h in range(2):
            tile = np.where(written[b * 16:(b + 1) * 16, None], vals[b * 16:(b + 1) * 16, h, :], 0.0)
            bc, bs = q([float(v) for v in tile.ravel()])
            assert float(scales[b, h]) == bs
            assert codes[b * 16:(b + 1) * 16, h, :].ravel().tolist() == bc
            unw = ~written[b * 16:(b + 1) * 16]
            assert (codes[b * 16:(b + 1) * 16][unw] == 0).all()


def test_full_block_state_is_the_whole_block_quantized():
    """Once a block holds 16 tokens, its state is the quantization of its 16
    tokens, whatever order they were written in."""
    from oracle import quantize_tiles
    c = make_decode_case(4, 2, 8, "bf16", [16], 731, pool_blocks=1)
    vals = bf16_bits_to_f32(c.k_slots)
    codes, scales = W.quantized_state(vals, np.ones(16, dtype=bool), 8)
    rc, rs = quantize_tiles(vals, 8)
    assert np.array_equal(codes, rc) and np.array_equal(scales.view(np.uint16), rs.view(np.uint16))
