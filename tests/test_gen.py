"""The seeded workloads have the structure the pages describe."""
import numpy as np
import pytest

from synth import (CONFIGS, make_config_case, make_mixed_case, permute_pool, private_twin, used_slot_mask)
from synth.gen import bf16_bits_to_f32, f32_to_bf16_bits


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 65504.0], dtype=np.float32)
    b = f32_to_bf16_bits(x)
    back = bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 65536.0]


def test_determinism():
    a = make_config_case(2, num_seqs=3)
    b = make_config_case(2, num_seqs=3)
    assert np.array_equal(a.k_slots, b.k_slots) and np.array_equal(a.block_tables, b.block_tables)


def _check_tables(c):
    nb = -(-c.context_lens.astype(np.int64) // 16)
    for s in range(c.num_seqs):
        row = c.block_tables[s]
        assert (row[:nb[s]] >= 0).all() and (row[:nb[s]] < c.num_blocks).all()
        assert (row[nb[s]:] == -1).all()
        waste = nb[s] * 16 - c.context_lens[s]
        assert 0 <= waste <= 15


def test_workload1():
    c = make_config_case(1)
    assert c.context_lens.tolist() == [5, 17, 33, 40]
    assert c.num_blocks == 32 and c.q.dtype == np.float32
    _check_tables(c)
    ids = c.block_tables[c.block_tables >= 0]
    assert len(np.unique(ids)) == 9


def test_workload2_distribution():
    c = make_config_case(2)
    cfg = CONFIGS[2]
    assert c.num_seqs == 64
    assert c.context_lens.min() >= 512 and c.context_lens.max() <= 4096
    need = int((-(-c.context_lens.astype(np.int64) // 16)).sum())
    assert c.num_blocks == int(np.ceil(1.1 * need))
    _check_tables(c)
    ids = c.block_tables[c.block_tables >= 0]
    assert len(np.unique(ids)) == len(ids) == need
    assert c.k_slots.shape == (c.num_blocks * 16, 8, 128) and c.k_slots.dtype == np.uint16
    # N(0,1) bf16 draws
    vals = bf16_bits_to_f32(c.k_slots[:200000].ravel())
    assert abs(vals.mean()) < 0.01 and abs(vals.std() - 1) < 0.01


def test_workload3_sharing_structure():
    c = make_config_case(3, num_seqs=32)
    assert c.shared_prefix_blocks == 250
    assert (c.block_tables[:, :250] == c.block_tables[0, :250]).all()
    tails = c.context_lens - 4000
    assert tails.min() >= 200 and tails.max() <= 500
    _check_tables(c)
    priv = np.concatenate([c.block_tables[s, 250:(-(-int(c.context_lens[s]) // 16))] for s in range(32)])
    assert len(np.unique(priv)) == len(priv)
    assert not set(priv) & set(c.block_tables[0, :250])
    t = private_twin(c)
    _check_tables(t)
    assert np.array_equal(used_slot_mask(t).sum(), c.context_lens.sum())


def test_workload4_and_5_shapes():
    c = make_config_case(4, num_seqs=2)
    assert c.context_lens.tolist() == [8000, 8000] and c.max_blocks_per_seq == 500
    pre, dec = make_mixed_case()
    assert pre.context_lens.tolist() == [8048] and pre.max_q_len == 2048
    assert dec.num_seqs == 64
    assert dec.context_lens.min() >= 128 and dec.context_lens.max() <= 16384
    assert 1200 < np.median(dec.context_lens) < 3200


def test_permutation_is_bijection():
    c = make_config_case(2, num_seqs=4)
    p = permute_pool(c, 1)
    pi = p.extra["perm"]
    assert sorted(pi.tolist()) == list(range(c.num_blocks))
    m = c.block_tables >= 0
    assert np.array_equal(p.block_tables[m], pi[c.block_tables[m]])
    b = int(c.block_tables[0, 0])
    assert np.array_equal(p.k_slots[pi[b] * 16:(pi[b] + 1) * 16], c.k_slots[b * 16:(b + 1) * 16])


def test_clustered_prefix_structure():
    from synth import make_clustered_prefix_case
    clusters = [(5, [100, 70, 33]), (2, [40, 16]), (0, [17])]
    c = make_clustered_prefix_case(8, 2, 64, "f32", clusters, 11)
    t = c.block_tables
    # members of a cluster point their first min(nblk, P) entries at the same blocks
    assert (t[0, :5] == t[1, :5]).all() and (t[2, :3] == t[0, :3]).all()
    assert (t[3, :2] == t[4, :1].tolist() + [t[3, 1]]).all() and t[3, 0] == t[4, 0]
    used = []
    for s in range(c.num_seqs):
        used += t[s, :-(-int(c.context_lens[s]) // 16)].tolist()
    # every referenced block exists; only shared prefix blocks are referenced twice
    assert min(used) >= 0 and max(used) < c.num_blocks
    from collections import Counter
    multi = {b for b, n in Counter(used).items() if n > 1}
    assert multi == set(t[0, :5].tolist()) | {int(t[3, 0])}


def test_privatize_references_each_block_once():
    from synth import make_clustered_prefix_case, privatize
    import oracle
    c = make_clustered_prefix_case(8, 2, 64, "f32", [(4, [80, 64, 50]), (0, [9])], 12)
    p = privatize(c)
    used = []
    for s in range(p.num_seqs):
        used += p.block_tables[s, :-(-int(p.context_lens[s]) // 16)].tolist()
    assert len(used) == len(set(used))
    f = lambda x: oracle.as_f64(x, "f32")
    a = oracle.paged_decode(f(c.q), f(c.k_slots), f(c.v_slots), c.block_tables, c.context_lens, n_kv=2)
    b = oracle.paged_decode(f(p.q), f(p.k_slots), f(p.v_slots), p.block_tables, p.context_lens, n_kv=2)
    assert np.array_equal(a, b)
