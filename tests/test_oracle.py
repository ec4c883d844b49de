"""Pins of the attention oracle: brute force, closed forms, library reductions
and the paging invariants the pages state."""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from synth import (make_config_case, make_decode_case, make_mixed_case, make_prefill_case,
                   make_prefill_probe_case, make_prefix_probe_case, make_probe_case, permute_pool, poison_unused,
                   private_twin)
from synth.gen import bf16_bits_to_f32


def f64(case, x):
    return oracle.as_f64(x, case.dtype)


def run_decode(case, seqs=None):
    return oracle.paged_decode(f64(case, case.q), f64(case, case.k_slots), f64(case, case.v_slots),
                               case.block_tables, case.context_lens, n_kv=case.n_kv, seqs=seqs)


def run_prefill(case, rows=None):
    return oracle.paged_prefill(f64(case, case.q), case.cu_q_lens, f64(case, case.k_slots), f64(case, case.v_slots),
                                case.block_tables, case.context_lens, n_kv=case.n_kv, rows=rows)


def test_as_f64_bf16_exact():
    x = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], dtype=np.uint16)
    got = oracle.as_f64(x, "bf16")
    assert got[0] == 1.0 and got[1] == -1.0
    assert got[2] == 3.140625
    assert got[3] == 2.0 ** -133  # bf16 denormal
    assert got[4] == (2 - 2 ** -7) * 2.0 ** 127


def test_oracle_vs_brute_force_workload1():
    c = make_config_case(1)
    out = run_decode(c)
    q, k, v = f64(c, c.q), f64(c, c.k_slots), f64(c, c.v_slots)
    for s in range(c.num_seqs):
        ref = brute.decode_attention(q[s].tolist(), k.tolist(), v.tolist(), c.block_tables[s].tolist(),
                                     int(c.context_lens[s]), c.n_kv)
        np.testing.assert_allclose(out[s], np.array(ref), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_oracle_vs_brute_force_random_tiny(seed):
    g = np.random.default_rng(seed)
    n_kv = int(g.choice([1, 2, 3]))
    G = int(g.choice([1, 2, 4]))
    d = int(g.choice([4, 8, 16]))
    ctx = g.integers(1, 50, size=int(g.integers(1, 4)))
    dtype = "bf16" if seed % 2 else "f32"
    c = make_decode_case(n_kv * G, n_kv, d, dtype, ctx, 100 + seed, pool_factor=1.5)
    out = run_decode(c)
    q, k, v = f64(c, c.q), f64(c, c.k_slots), f64(c, c.v_slots)
    for s in range(c.num_seqs):
        ref = brute.decode_attention(q[s].tolist(), k.tolist(), v.tolist(), c.block_tables[s].tolist(),
                                     int(c.context_lens[s]), n_kv)
        np.testing.assert_allclose(out[s], np.array(ref), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_window_vs_brute_force_random_tiny(seed):
    """Sliding window W: keys n - W .. n - 1 only (brute force, windows from 1
    to past the context)."""
    g = np.random.default_rng(50 + seed)
    n_kv, G, d = int(g.choice([1, 2])), int(g.choice([1, 2, 4])), int(g.choice([4, 8]))
    ctx = g.integers(1, 60, size=3)
    c = make_decode_case(n_kv * G, n_kv, d, "bf16" if seed % 2 else "f32", ctx, 150 + seed, pool_factor=1.5)
    q, k, v = f64(c, c.q), f64(c, c.k_slots), f64(c, c.v_slots)
    for w in (1, 2, 15, 16, 17, 33, 70):
        out = oracle.paged_decode(q, k, v, c.block_tables, c.context_lens, n_kv=n_kv, window=w)
        for s in range(c.num_seqs):
            ref = brute.decode_attention(q[s].tolist(), k.tolist(), v.tolist(), c.block_tables[s].tolist(),
                                         int(c.context_lens[s]), n_kv, window=w)
            np.testing.assert_allclose(out[s], np.array(ref), rtol=0, atol=1e-12)


def test_window_one_is_last_value():
    """A window of one token: the softmax has one term, so the output is
    exactly that token's V."""
    c = make_decode_case(8, 2, 32, "bf16", [1, 17, 40, 100], 9, pool_factor=1.2)
    q, k, v = f64(c, c.q), f64(c, c.k_slots), f64(c, c.v_slots)
    out = oracle.paged_decode(q, k, v, c.block_tables, c.context_lens, n_kv=2, window=1)
    for s in range(c.num_seqs):
        t = int(c.context_lens[s]) - 1
        slot = c.block_tables[s, t // 16] * 16 + t % 16
        for h in range(8):
            assert np.array_equal(out[s, h], v[slot, h // 4])


def test_window_equals_truncated_context():
    """Decode with window W equals full decode of a sequence that holds only
    its last W tokens (copied into fresh blocks, starting at slot 0), and a
    window covering the context changes nothing."""
    c = make_decode_case(8, 4, 16, "f32", [5, 31, 64, 77], 10, pool_factor=1.3)
    q, k, v = f64(c, c.q), f64(c, c.k_slots), f64(c, c.v_slots)
    full = run_decode(c)
    for w in (3, 16, 20, 64, 200):
        got = oracle.paged_decode(q, k, v, c.block_tables, c.context_lens, n_kv=4, window=w)
        for s in range(c.num_seqs):
            n = int(c.context_lens[s])
            if w >= n:
                assert np.array_equal(got[s], full[s])
            m = min(w, n)
            toks = np.arange(n - m, n)
            slots = c.block_tables[s, toks // 16].astype(np.int64) * 16 + toks % 16
            nb = -(-m // 16)
            table = np.arange(nb, dtype=np.int32)[None, :]
            kk = np.zeros((nb * 16,) + k.shape[1:])
            vv = np.zeros_like(kk)
            kk[:m], vv[:m] = k[slots], v[slots]
            ref = oracle.paged_decode(q[s:s + 1], kk, vv, table, np.array([m]), n_kv=4)
            np.testing.assert_allclose(got[s], ref[0], rtol=0, atol=1e-14)


def test_closed_form_single_token():
    c = make_decode_case(8, 2, 32, "f32", [1, 1, 1], 7)
    out = run_decode(c)
    v = f64(c, c.v_slots)
    for s in range(3):
        slot = c.block_tables[s, 0] * 16
        for h in range(8):
            assert np.array_equal(out[s, h], v[slot, h // 4])


def test_closed_form_zero_query_is_mean():
    c = make_decode_case(4, 2, 16, "f32", [7, 33, 100], 8)
    c.q[:] = 0
    out = run_decode(c)
    v = f64(c, c.v_slots)
    for s in range(c.num_seqs):
        V = oracle.gather(v, c.block_tables[s], int(c.context_lens[s]))
        for h in range(4):
            np.testing.assert_allclose(out[s, h], V[:, h // 2].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_closed_form_constant_values():
    c = make_decode_case(4, 4, 16, "f32", [9, 40], 9)
    c.v_slots[:] = np.arange(16, dtype=np.float32)[None, None, :] * 0.5 - 3.0
    out = run_decode(c)
    np.testing.assert_allclose(out, np.broadcast_to(np.arange(16) * 0.5 - 3.0, out.shape), rtol=0, atol=1e-13)


def _sdpa(q, K, V):
    """torch's scaled_dot_product_attention (CPU, float64) on one sequence:
    q [H, D], K/V [n, H, D] (already one KV head per query head)."""
    qt = torch.from_numpy(q)[:, None, :]             # [H, 1, D]
    kt = torch.from_numpy(K).permute(1, 0, 2).contiguous()  # [H, n, D]
    vt = torch.from_numpy(V).permute(1, 0, 2).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0, :].numpy()


@pytest.mark.parametrize("n_heads,n_kv", [(8, 8), (8, 1), (8, 2), (32, 8)])
def test_reduces_to_library_attention(n_heads, n_kv):
    """MHA (G=1), MQA (n_kv=1) and GQA all reduce to textbook single-head
    attention with each query head's KV head repeated G times (contiguous
    groups), as computed by torch's SDPA."""
    c = make_decode_case(n_heads, n_kv, 64, "bf16", [1, 16, 17, 300], 11)
    out = run_decode(c)
    q, k, v = f64(c, c.q), f64(c, c.k_slots), f64(c, c.v_slots)
    G = n_heads // n_kv
    for s in range(c.num_seqs):
        K = oracle.gather(k, c.block_tables[s], int(c.context_lens[s]))
        V = oracle.gather(v, c.block_tables[s], int(c.context_lens[s]))
        Kr = np.repeat(K, G, axis=1)   # repeat_interleave: head h uses kv head h // G
        Vr = np.repeat(V, G, axis=1)
        np.testing.assert_allclose(out[s], _sdpa(q[s], Kr, Vr), rtol=1e-12, atol=1e-13)


def test_gqa_equals_mha_with_repeated_heads():
    c = make_decode_case(8, 2, 32, "f32", [20, 45], 12)
    out = run_decode(c)
    k = np.repeat(c.k_slots, 4, axis=1)
    v = np.repeat(c.v_slots, 4, axis=1)
    mha = oracle.paged_decode(f64(c, c.q), f64(c, k), f64(c, v), c.block_tables, c.context_lens, n_kv=8)
    assert np.array_equal(out, mha)


def test_wrong_head_mapping_is_detected():
    """A plausible slip (kv head = h % n_kv instead of h // G) changes the
    result: the pins above are sensitive to the grouping."""
    c = make_decode_case(8, 2, 32, "f32", [20, 45], 12)
    out = run_decode(c)
    k = c.k_slots[:, np.arange(8) % 2]
    v = c.v_slots[:, np.arange(8) % 2]
    wrong = oracle.paged_decode(f64(c, c.q), f64(c, k), f64(c, v), c.block_tables, c.context_lens, n_kv=8)
    assert not np.allclose(out, wrong)


def test_permutation_invariance():
    c = make_config_case(2, num_seqs=6)
    p = permute_pool(c, 5)
    assert not np.array_equal(p.block_tables, c.block_tables)
    assert np.array_equal(run_decode(c), run_decode(p))


def test_shared_equals_private():
    c = make_config_case(3, num_seqs=4)
    assert c.shared_prefix_blocks == 250
    assert (c.block_tables[:, :250] == c.block_tables[0, :250]).all()
    t = private_twin(c)
    assert len(np.unique(t.block_tables[:, :250])) == 4 * 250
    assert np.array_equal(run_decode(c), run_decode(t))


def test_unused_slots_do_not_matter():
    c = make_config_case(2, num_seqs=5)
    ref = run_decode(c)
    for kind in ("nan", "big"):
        p = poison_unused(c, kind)
        assert np.array_equal(run_decode(p), ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_retrieval_probe(dtype):
    c = make_probe_case(16, 4, 128, dtype, [5, 16, 17, 200, 999], 13)
    out = run_decode(c)
    v = f64(c, c.v_slots)
    for s in range(c.num_seqs):
        t = int(c.extra["tstar"][s])
        slot = c.block_tables[s, t // 16] * 16 + t % 16
        for h in range(16):
            np.testing.assert_allclose(out[s, h], v[slot, h // 4], rtol=0, atol=1e-40)


def test_retrieval_probe_negative_control():
    """Corrupting one block-table entry (the magnet's block) must fail the probe."""
    c = make_probe_case(4, 2, 64, "f32", [40, 40], 14)
    t = int(c.extra["tstar"][0])
    j = t // 16
    good = run_decode(c)
    bad_tables = c.block_tables.copy()
    bad_tables[0, j] = c.block_tables[1, j]
    bad = oracle.paged_decode(f64(c, c.q), f64(c, c.k_slots), f64(c, c.v_slots), bad_tables, c.context_lens, n_kv=2)
    assert not np.array_equal(good[0], bad[0])


@pytest.mark.parametrize("dtype,shared_pos", [("bf16", 0), ("bf16", 200), ("f32", 255)])
def test_prefix_retrieval_probe(dtype, shared_pos):
    """Shared-prefix probe: a sequence with a tail magnet returns V there,
    the others V at the shared magnet (up to float64 weights below 1e-60 on
    the other keys, which float32 flushes to 0); brute force agrees."""
    tails = [1, 5, 16, 17, 40, 3]
    c = make_prefix_probe_case(16, 4, 64, dtype, 256, tails, 19, shared_pos=shared_pos,
                               tail_magnet=[1, 0, 1, 0, 1, 1])
    out = run_decode(c)
    v = f64(c, c.v_slots)
    for s in range(c.num_seqs):
        t = int(c.extra["tstar"][s])
        assert (t == shared_pos) != bool([1, 0, 1, 0, 1, 1][s])
        slot = c.block_tables[s, t // 16] * 16 + t % 16
        for h in range(16):
            np.testing.assert_allclose(out[s, h], v[slot, h // 4], rtol=0, atol=1e-40, err_msg=f"{s} {h}")
    # every sequence points its first 16 blocks at the same physical blocks
    assert (c.block_tables[:, :16] == c.block_tables[0, :16]).all()
    q, k, vv = f64(c, c.q), f64(c, c.k_slots).tolist(), v.tolist()
    for s in (0, 1):
        ref = brute.decode_attention(q[s].tolist(), k, vv, c.block_tables[s].tolist(), int(c.context_lens[s]), 4)
        np.testing.assert_allclose(out[s], np.array(ref), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_windowed_prefill_vs_brute_force(seed):
    """Windowed chunk rows: row at position p attends keys p - W + 1 .. p
    (brute force, windows from one token to past the context)."""
    g = np.random.default_rng(90 + seed)
    n_kv, G, d = int(g.choice([1, 2])), int(g.choice([1, 2, 4])), int(g.choice([4, 8]))
    ctx = g.integers(1, 50, size=3)
    qlens = [int(g.integers(0, c + 1)) for c in ctx]
    c = make_prefill_case(n_kv * G, n_kv, d, "bf16" if seed % 2 else "f32", ctx, qlens, 190 + seed)
    q, k, v = f64(c, c.q), f64(c, c.k_slots), f64(c, c.v_slots)
    for w in (1, 2, 15, 16, 17, 60):
        out = oracle.paged_prefill(q, c.cu_q_lens, k, v, c.block_tables, c.context_lens, n_kv=n_kv, window=w)
        for s in range(c.num_seqs):
            lo, hi = int(c.cu_q_lens[s]), int(c.cu_q_lens[s + 1])
            if hi == lo:
                continue
            ref = brute.prefill_attention(q[lo:hi].tolist(), k.tolist(), v.tolist(), c.block_tables[s].tolist(),
                                          int(c.context_lens[s]), n_kv, window=w)
            np.testing.assert_allclose(out[lo:hi], np.array(ref), rtol=0, atol=1e-12)


def test_windowed_prefill_special_cases():
    """W = 1: each row returns its own V exactly; W past every position: the
    unwindowed chunk; the last row equals the windowed decode of the whole
    context."""
    c = make_prefill_case(8, 2, 16, "bf16", [40, 17, 100], [40, 5, 33], 195)
    q, k, v = f64(c, c.q), f64(c, c.k_slots), f64(c, c.v_slots)
    one = oracle.paged_prefill(q, c.cu_q_lens, k, v, c.block_tables, c.context_lens, n_kv=2, window=1)
    for s in range(c.num_seqs):
        lo, hi = int(c.cu_q_lens[s]), int(c.cu_q_lens[s + 1])
        n = int(c.context_lens[s])
        for i in range(hi - lo):
            p = n - (hi - lo) + i
            slot = c.block_tables[s, p // 16] * 16 + p % 16
            for h in range(8):
                assert np.array_equal(one[lo + i, h], v[slot, h // 4])
    full = run_prefill(c)
    wide = oracle.paged_prefill(q, c.cu_q_lens, k, v, c.block_tables, c.context_lens, n_kv=2, window=1000)
    assert np.array_equal(full, wide)
    w = 23
    win = oracle.paged_prefill(q, c.cu_q_lens, k, v, c.block_tables, c.context_lens, n_kv=2, window=w)
    last_rows = np.asarray(c.cu_q_lens[1:]) - 1
    dec = oracle.paged_decode(q[last_rows], k, v, c.block_tables, c.context_lens, n_kv=2, window=w)
    np.testing.assert_allclose(win[last_rows], dec, rtol=0, atol=1e-14)


@pytest.mark.parametrize("window", [1, 5, 64, 65, 300])
def test_windowed_prefill_first_key_probe(window):
    """The causal probe with its queries negated: scores fall strictly with
    position, so each windowed row returns V at max(0, p - W + 1), the first
    key its window shows (float64 weights of the others below 1e-60)."""
    c = make_prefill_probe_case(8, 2, 128, "f32", [300, 64, 17], [100, 64, 3], 196)
    c.q = -c.q
    out = oracle.paged_prefill(f64(c, c.q), c.cu_q_lens, f64(c, c.k_slots), f64(c, c.v_slots), c.block_tables,
                               c.context_lens, n_kv=2, window=window)
    v = f64(c, c.v_slots)
    for s in range(c.num_seqs):
        lo, hi = int(c.cu_q_lens[s]), int(c.cu_q_lens[s + 1])
        n = int(c.context_lens[s])
        for i in range(hi - lo):
            p = max(0, n - (hi - lo) + i - window + 1)
            sl = c.block_tables[s, p // 16] * 16 + p % 16
            for h in range(8):
                np.testing.assert_allclose(out[lo + i, h], v[sl, h // 4], rtol=0, atol=1e-40)


def test_prefill_vs_brute_force():
    c = make_prefill_case(4, 2, 8, "f32", [5, 33, 20], [5, 7, 1], 15)
    out = run_prefill(c)
    q, k, v = f64(c, c.q), f64(c, c.k_slots), f64(c, c.v_slots)
    for s in range(c.num_seqs):
        lo, hi = int(c.cu_q_lens[s]), int(c.cu_q_lens[s + 1])
        ref = brute.prefill_attention(q[lo:hi].tolist(), k.tolist(), v.tolist(), c.block_tables[s].tolist(),
                                      int(c.context_lens[s]), c.n_kv)
        np.testing.assert_allclose(out[lo:hi], np.array(ref), rtol=0, atol=1e-12)


def test_prefill_last_row_and_q1_equal_decode():
    c = make_prefill_case(8, 2, 32, "bf16", [100, 37], [30, 1], 16)
    out = run_prefill(c)
    lastrows = c.cu_q_lens[1:] - 1
    dec = oracle.paged_decode(f64(c, c.q[lastrows]), f64(c, c.k_slots), f64(c, c.v_slots), c.block_tables,
                              c.context_lens, n_kv=c.n_kv)
    np.testing.assert_allclose(out[lastrows], dec, rtol=1e-13, atol=1e-14)


def test_prefill_split_invariance():
    """Two half chunks == one chunk: the chunk is the same attention split up."""
    c = make_prefill_case(4, 2, 16, "f32", [64], [40], 17)
    whole = run_prefill(c)
    # first 20 queries as a chunk of a 44-token context, the rest as a chunk of 64
    first = oracle.paged_prefill(f64(c, c.q[:20]), np.array([0, 20]), f64(c, c.k_slots), f64(c, c.v_slots),
                                 c.block_tables, np.array([44]), n_kv=2)
    second = oracle.paged_prefill(f64(c, c.q[20:]), np.array([0, 20]), f64(c, c.k_slots), f64(c, c.v_slots),
                                  c.block_tables, np.array([64]), n_kv=2)
    np.testing.assert_allclose(np.concatenate([first, second]), whole, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_causal_probe(dtype):
    c = make_prefill_probe_case(8, 2, 128, dtype, [300, 64, 17], [100, 64, 3], 18)
    out = run_prefill(c)
    v = f64(c, c.v_slots)
    for s in range(c.num_seqs):
        lo, hi = int(c.cu_q_lens[s]), int(c.cu_q_lens[s + 1])
        n = int(c.context_lens[s])
        for i in range(hi - lo):
            p = n - (hi - lo) + i
            slot = c.block_tables[s, p // 16] * 16 + p % 16
            for h in range(8):
                np.testing.assert_allclose(out[lo + i, h], v[slot, h // 4], rtol=0, atol=1e-30)


def test_prefill_probe_detects_noncausal():
    """Planting an off-by-one in the causal limit (oracle side, CPU) fails the probe."""
    c = make_prefill_probe_case(2, 1, 64, "f32", [40], [10], 19)
    good = run_prefill(c)
    q, k, v = f64(c, c.q), f64(c, c.k_slots), f64(c, c.v_slots)
    K = oracle.gather(k, c.block_tables[0], 40)
    V = oracle.gather(v, c.block_tables[0], 40)
    row = 3
    pos = 30 + row
    # a non-causal row that also sees key pos+1
    leaky = oracle.softmax_attention(q[row, 0], K[:pos + 2, 0], V[:pos + 2, 0], 1 / 8)
    assert not np.allclose(leaky, good[row, 0])


def test_mixed_case_structure():
    pre, dec = make_mixed_case(decode_seqs=8, chunk_tokens=64, cached_tokens=96)
    assert pre.context_lens[0] == 160 and pre.max_q_len == 64
    assert dec.num_seqs == 8
    used = np.concatenate([pre.block_tables[pre.block_tables >= 0], dec.block_tables[dec.block_tables >= 0]])
    assert len(np.unique(used)) == len(used) == pre.num_blocks
