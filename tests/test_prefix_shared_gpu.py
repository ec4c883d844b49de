"""GPU checks of the 70B-class prefix-shared decode at its full shape: 256
sequences, 64 query / 8 KV heads, d_head 128, a shared 4000-token prefix
(250 physical blocks) and private tails of U[200, 500] tokens. At 2048
query rows per KV head this batch takes the prefix pass (one MFMA
contraction over each tile's common run of blocks, merged with the decode of
the blocks after it), so these tests pin block-table exactness on that path:
exact retrieval probes with magnets inside the prefix pass's run, in the
part of the shared run it leaves to the decode, and in the private tails; a
corrupted shared-run entry that must fail the probe; bit-identical output
under any relabelling of physical blocks; and the whole batch against the
oracle."""
import numpy as np
import pytest
import torch

import oracle
from synth import config_seed, make_config_case, make_prefix_probe_case, permute_pool, private_twin
from tests.gpu_util import assert_close, dev_to_f64, gpu_decode, oracle_decode

pytestmark = pytest.mark.gpu

PREFIX = 4000
S, H, KV, D = 256, 64, 8, 128


def _tails():
    """The private tail lengths of the prefix-shared workload (its own draw)."""
    kids = np.random.SeedSequence(config_seed(3)).spawn(5)
    return np.random.Generator(np.random.PCG64(kids[0])).integers(200, 500, size=S, endpoint=True)


def _expect_probe(c, got):
    v = c.v_slots  # bf16 bit patterns
    bad = []
    for s in range(c.num_seqs):
        t = int(c.extra["tstar"][s])
        slot = int(c.block_tables[s, t // 16]) * 16 + t % 16
        want = v[slot]  # [n_kv, d]
        for h in range(c.n_heads):
            if not np.array_equal(got[s, h], want[h // (c.n_heads // c.n_kv)]):
                bad.append((s, h))
    return bad


@pytest.fixture(scope="module")
def workload3():
    return make_config_case(3)


def test_workload3_full_batch(lib, workload3):
    """Every one of the 256 sequences against the oracle, in the launch
    configuration the benchmark times."""
    c = workload3
    assert c.num_seqs * c.group >= 512 and c.shared_prefix_blocks == 250
    got = dev_to_f64(gpu_decode(c))
    assert_close(got, oracle_decode(c), "bf16", "workload3 all sequences")


# Positions of the shared magnet: the first prefix token; the last token of
# the second of the prefix pass's four key ranges (its 248-block run is cut
# into stage ranges ending at tokens 960, 1984, 2944 and 3968); the first and
# last tokens of the two shared blocks past the run, which the decode reads.
@pytest.mark.parametrize("shared_pos", [0, 1983, 3968, 3999])
def test_workload3_prefix_probe_exact(lib, shared_pos):
    """Odd sequences carry a magnet in their private tail, even ones see
    only the shared magnet; every output row must equal V at its magnet bit
    for bit."""
    c = make_prefix_probe_case(H, KV, D, "bf16", PREFIX, _tails(), 610 + shared_pos, shared_pos=shared_pos,
                               tail_magnet=[s % 2 for s in range(S)])
    got = gpu_decode(c).cpu().view(torch.int16).numpy().view(np.uint16)
    bad = _expect_probe(c, got)
    assert not bad, f"{len(bad)} rows differ, first {bad[:4]}"


def test_workload3_prefix_probe_negative_control(lib):
    """Sequence 64 (a tile's first member) and sequence 130 (mid-tile) have
    the shared magnet's block replaced by an in-range block without a
    magnet: both must miss the magnet, both tiles' common runs shrink, the
    GPU still matches the oracle on the corrupted tables, and every other
    sequence still returns its magnet exactly."""
    shared_pos = 2500
    c = make_prefix_probe_case(H, KV, D, "bf16", PREFIX, _tails(), 620, shared_pos=shared_pos,
                               tail_magnet=[s % 2 for s in range(S)])
    j = shared_pos // 16
    victims = (64, 130)
    # a private tail block of sequence 0 (no magnet there: sequence 0 has none)
    donor = int(c.block_tables[0, 250])
    good_slot = int(c.block_tables[0, j]) * 16 + shared_pos % 16
    for s in victims:
        assert c.extra["tstar"][s] == shared_pos
        c.block_tables[s, j] = donor
    got16 = gpu_decode(c).cpu()
    got = got16.view(torch.int16).numpy().view(np.uint16)
    for s in victims:
        for h in range(H):
            assert not np.array_equal(got[s, h], c.v_slots[good_slot, h // 8])
    bad = [x for x in _expect_probe(c, got) if x[0] not in victims]
    assert not bad, f"{len(bad)} rows differ, first {bad[:4]}"
    ref = oracle_decode(c, seqs=list(victims) + [0, 1, 65, 131])
    rows = list(victims) + [0, 1, 65, 131]
    assert_close(dev_to_f64(got16)[rows], ref[rows], "bf16", "corrupted shared block")


def test_workload3_permutation_bitexact(lib, workload3):
    """Relabelling physical blocks by a random bijection (tables remapped)
    keeps which blocks are shared, so the prefix pass finds the same runs:
    output bit-identical."""
    a = gpu_decode(workload3).cpu()
    b = gpu_decode(permute_pool(workload3, 11)).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_workload3_shared_vs_private(lib, workload3):
    """Private copies of the shared prefix go through the per-sequence decode
    (no common run), the shared blocks through the prefix pass, whose
    floating-point sums run in another order: the two agree with each other
    and with the oracle to the bf16 tolerance (the share of bit-identical
    elements and the largest difference are printed)."""
    c = workload3
    a = gpu_decode(c).cpu()
    b = gpu_decode(private_twin(c)).cpu()
    fa, fb = dev_to_f64(a), dev_to_f64(b)
    ref = oracle_decode(c)
    assert_close(fa, ref, "bf16", "shared")
    assert_close(fb, ref, "bf16", "private")
    assert_close(fa, fb, "bf16", "shared vs private")
    # distance in bf16 units in the last place (ordered bit patterns)
    ia = a.view(torch.int16).numpy().astype(np.int32)
    ib = b.view(torch.int16).numpy().astype(np.int32)
    oa = np.where(ia < 0, -(ia & 0x7FFF), ia)
    ob = np.where(ib < 0, -(ib & 0x7FFF), ib)
    ulp = np.abs(oa - ob)
    print(f"shared vs private: {float((ulp == 0).mean()):.4f} of elements bit-identical, "
          f"{float((ulp <= 1).mean()):.4f} within one bf16 ulp, max abs difference {np.abs(fa - fb).max():.3e}")
