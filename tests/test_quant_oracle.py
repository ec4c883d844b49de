"""Pins of the quantization oracle: an independent pure-Python brute force
(struct-based float32/float16 rounding, Python's round-half-even) and the
properties symmetric b-bit quantization must have."""
import numpy as np
import pytest

import oracle
from oracle import brute
from synth.gen import bf16_bits_to_f32, f32_to_bf16_bits


def _tiles(seed, nb=3, n_kv=2, d=16, scale=1.0):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((nb * 16, n_kv, d)) * scale).astype(np.float32)
    return bf16_bits_to_f32(f32_to_bf16_bits(x))  # bf16-representable, as the cache source is


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("seed,scale", [(0, 1.0), (1, 1e-3), (2, 300.0), (3, 1e-6)])
def test_quantize_vs_brute_force(bits, seed, scale):
    x = _tiles(seed, scale=scale)
    codes, scales = oracle.quantize_tiles(x, bits)
    nb, n_kv = scales.shape
    for b in range(nb):
        for h in range(n_kv):
            tile = x[b * 16:(b + 1) * 16, h, :]
            bc, bs = brute.quantize_tile([float(v) for v in tile.ravel()], bits)
            assert float(scales[b, h]) == bs
            assert codes[b * 16:(b + 1) * 16, h, :].ravel().tolist() == bc


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_properties(bits):
    qmax = oracle.QMAX[bits]
    x = _tiles(5, nb=8, n_kv=4, d=64)
    codes, scales = oracle.quantize_tiles(x, bits)
    assert codes.dtype == np.int8
    assert codes.min() >= -qmax and codes.max() <= qmax
    # the element of largest magnitude maps to +-qmax
    nb = scales.shape[0]
    t = x.reshape(nb, 16, 4, 64)
    c = codes.reshape(nb, 16, 4, 64)
    for b in range(nb):
        for h in range(4):
            i = np.unravel_index(np.argmax(np.abs(t[b, :, h, :])), (16, 64))
            assert abs(int(c[b, i[0], h, i[1]])) == qmax
    # odd symmetry
    codes_neg, scales_neg = oracle.quantize_tiles(-x, bits)
    assert np.array_equal(scales_neg, scales) and np.array_equal(codes_neg, -codes)
    # reconstruction error at most half a step (plus the fp16 rounding of s)
    deq = oracle.dequantize(codes, scales)
    s = np.repeat(scales.astype(np.float64), 16, axis=0)[:, :, None]
    err = np.abs(deq - x.astype(np.float64))
    assert (err <= s / 2 * (1 + 1e-6) + np.abs(x) * 2 ** -10).all()
    # footprint: 8 bits halve and 4 bits quarter 16-bit storage (codes only)
    assert bits / 16 == {8: 0.5, 4: 0.25}[bits]


def test_quantize_round_half_even_ties():
    """Values landing exactly on k + 1/2 steps round to even codes."""
    # amax = 127 -> s32 = 1.0 -> fp16 1.0, so codes are rint(x)
    x = np.zeros((16, 1, 8), dtype=np.float32)
    x[0, 0, :] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5]
    codes, scales = oracle.quantize_tiles(x, 8)
    assert float(scales[0, 0]) == 1.0
    assert codes[0, 0, :].tolist() == [127, 0, 2, 2, 0, -2, -2, 126]


def test_quantize_zero_and_overflow_tiles():
    x = np.zeros((32, 1, 8), dtype=np.float32)
    x[16:, 0, 0] = 3.0e6          # amax/7 > 65504: fp16 scale overflows
    codes, scales = oracle.quantize_tiles(x, 4)
    assert scales[0, 0] == 0 and (codes[:16] == 0).all()
    assert np.isinf(scales[1, 0]) and (codes[16:] == 0).all()
    bc, bs = brute.quantize_tile([float(v) for v in x[16:, 0, :].ravel()], 4)
    assert bs == float("inf") and set(bc) == {0}


def test_dequantize_exact():
    codes = np.arange(-127, 129, dtype=np.int64)[:256].clip(-127, 127).astype(np.int8).reshape(16, 1, 16)
    scales = np.array([[0.0078125]], dtype=np.float16)
    deq = oracle.dequantize(codes, scales)
    assert np.array_equal(deq, codes.astype(np.float64) * 0.0078125)


# --- fp8 (OCP e4m3) -----------------------------------------------------------

def test_e4m3_defining_values():
    """Values fixed by the e4m3 format's definition (sign, 4-bit exponent of
    bias 7, 3-bit mantissa, subnormals at exponent 0, 0x7F/0xFF NaN)."""
    v = oracle.e4m3_value
    assert v(0x00) == 0.0 and v(0x80) == 0.0 and np.signbit(v(0x80))
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9
    assert v(0x08) == 2.0 ** -6                    # smallest normal
    assert v(0x38) == 1.0 and v(0x39) == 1.125 and v(0x3F) == 1.875
    assert v(0x40) == 2.0 and v(0x7E) == 448.0     # largest finite
    assert v(0xB8) == -1.0 and v(0xFE) == -448.0
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    pos = v(np.arange(127))
    assert (np.diff(pos) > 0).all()
    assert np.array_equal(v(np.arange(127) | 0x80), -pos)
    table = dict(brute.e4m3_table())
    assert all(table[c] == pos[c] for c in range(127))


def test_e4m3_round_ties_and_saturation():
    r = np.array([1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -9, 3 * 2.0 ** -10, 464.0, 1e6, -1000.0,
                  -0.0, -1e-9, 0.0, 448.0, 440.0, 432.0, 416.0], np.float32)
    want = [0x38, 0x3A, 0x00, 0x02, 0x02, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00, 0x7E, 0x7E, 0x7E, 0x7D]
    assert oracle.e4m3_round(r).tolist() == want


def test_e4m3_round_vs_brute_force():
    g = np.random.default_rng(8)
    r = np.concatenate([g.standard_normal(600) * 10, g.standard_normal(300) * 0.01,
                        g.uniform(-500, 500, 300)]).astype(np.float32)
    got = oracle.e4m3_round(r)
    table = brute.e4m3_table()
    for x, c in zip(r.tolist(), got.tolist()):
        a = min(abs(x), 448.0)
        best = min(table, key=lambda cv: (abs(cv[1] - a), cv[0] % 2))
        assert c == (best[0] | (0x80 if x < 0 or (x == 0 and np.signbit(x)) else 0)), x


@pytest.mark.parametrize("seed,scale", [(0, 1.0), (1, 1e-3), (2, 300.0), (3, 1e-6)])
def test_quantize_fp8_vs_brute_force(seed, scale):
    x = _tiles(seed, scale=scale)
    codes, scales = oracle.quantize_tiles_fp8(x)
    assert codes.dtype == np.uint8
    nb, n_kv = scales.shape
    for b in range(nb):
        for h in range(n_kv):
            tile = x[b * 16:(b + 1) * 16, h, :]
            bc, bs = brute.quantize_tile_fp8([float(v) for v in tile.ravel()])
            assert float(scales[b, h]) == bs
            assert codes[b * 16:(b + 1) * 16, h, :].ravel().tolist() == bc


def test_quantize_fp8_properties():
    x = _tiles(6, nb=8, n_kv=4, d=64)
    codes, scales = oracle.quantize_tiles_fp8(x)
    deq = oracle.dequantize_fp8(codes, scales)
    assert not np.isnan(deq).any() and not ((codes & 0x7F) == 0x7F).any()
    s = scales.astype(np.float64)[:, None, :, None]
    t = x.reshape(8, 16, 4, 64).astype(np.float64)
    c = codes.reshape(8, 16, 4, 64)
    # the element of largest magnitude of each group maps to +-448
    for b in range(8):
        for h in range(4):
            i = np.unravel_index(np.argmax(np.abs(t[b, :, h, :])), (16, 64))
            assert c[b, i[0], h, i[1]] & 0x7F == 0x7E
    # odd symmetry and a half-spacing error bound (3 mantissa bits)
    neg, _ = oracle.quantize_tiles_fp8(-x)
    assert np.array_equal(neg, codes ^ 0x80)
    err = np.abs(deq.reshape(t.shape) - t)
    bound = np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10 * s)
    assert (err <= bound * (1 + 1e-12)).all()
    # footprint: one byte per element, as int8 (half of bf16)
    assert codes.nbytes == x.size


def test_quantize_fp8_degenerate_scales():
    x = np.zeros((32, 1, 8), np.float32)
    x[16:, 0, 0] = 3.0e7                             # amax / 448 > 65504: fp16 scale overflows
    x[16:, 0, 1] = -1.0
    codes, scales = oracle.quantize_tiles_fp8(x)
    assert scales[0, 0] == 0 and np.isinf(scales[1, 0])
    assert (codes == 0).all()
