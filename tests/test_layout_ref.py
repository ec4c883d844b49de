"""The tests' NumPy statement of the device pool layout agrees with the
header's formula at hand-computed offsets, and round-trips."""
import numpy as np
import pytest

from tests.layout_ref import elem_index, pack_pool, unpack_pool


def test_hand_computed_offsets():
    # bf16 K, d 128: x = 8, (t=3, i=9) -> ((1*16)+3)*8 + 1 = 153
    assert elem_index("k", 128, 16)[3, 9] == 153
    # V: (t=3, i=9) -> 9*16 + 3
    assert elem_index("v", 128, 16)[3, 9] == 147
    # int4 K, d 64: x = 32, (t=5, i=40) -> ((1*16)+5)*32 + 8 = 680
    assert elem_index("k", 64, 4)[5, 40] == 680
    # fp32 K: x = 4, (t=15, i=127) -> ((31*16)+15)*4 + 3
    assert elem_index("k", 128, 32)[15, 127] == (31 * 16 + 15) * 4 + 3
    # int8 K: x = 16, (t=0, i=17) -> (16 + 0)*16 + 1
    assert elem_index("k", 128, 8)[0, 17] == 257
    # int4 V, d 128 (8 dim blocks): (t=9, i=37) -> (((5*2 + 1) * 8) + 2) * 8 + 1
    assert elem_index("v", 128, 4)[9, 37] == 721
    # int4 V, d 64 (4 dim blocks): (t=7, i=63) -> (((15*2 + 0) * 4) + 3) * 8 + 7
    assert elem_index("v", 64, 4)[7, 63] == 991


@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("bits,d", [(32, 64), (16, 128), (8, 128), (4, 64), (4, 128)])
def test_index_is_a_permutation_and_roundtrips(kind, bits, d):
    idx = elem_index(kind, d, bits)
    assert sorted(idx.ravel().tolist()) == list(range(16 * d))
    g = np.random.default_rng(bits + d)
    if bits == 32:
        slots = g.standard_normal((3 * 16, 2, d)).astype(np.float32)
    elif bits == 16:
        slots = g.integers(0, 1 << 16, size=(3 * 16, 2, d)).astype(np.uint16)
    else:
        q = 127 if bits == 8 else 7
        slots = g.integers(-q, q + 1, size=(3 * 16, 2, d)).astype(np.int8)
    img = pack_pool(slots, kind, bits)
    assert img.shape == (3, 2, 16 * d * bits // 8)
    back = unpack_pool(img, kind, bits, d)
    if bits == 32:
        back = back.view(np.float32)
    assert np.array_equal(back, slots)


def test_int4_nibble_order():
    slots = np.zeros((16, 1, 64), dtype=np.int8)
    slots[0, 0, 0] = 3      # element 0 -> low nibble of byte 0
    slots[0, 0, 1] = -2     # element 1 -> high nibble of byte 0
    img = pack_pool(slots, "k", 4)
    assert img[0, 0, 0] == (3 | (0xE << 4))
    # V int4: (t=1, i=0) is element 1 -> high nibble of byte 0
    v = np.zeros((16, 1, 64), dtype=np.int8)
    v[1, 0, 0] = 5
    assert pack_pool(v, "v", 4)[0, 0, 0] == 5 << 4
