"""Symmetric b-bit KV quantization with one scale per (block, KV head).

[JE] section "KV-cache quantization": keys and values are kept in 8 or 4 bits
instead of 16, each stored as an integer that shares one scale s with its
group. The printed formula is lost; this is the plain symmetric,
zero-point-free reading:

  group   = one (physical block, KV head) tile: 16 slots x d_head values,
            separately for K and for V
  amax    = max |x| over the group               (float32)
  s32     = amax / qmax                          (float32, IEEE division)
  s       = float16(s32)                         (round to nearest even)
  code    = clip(rint(x / float32(s)), -qmax, qmax)   (float32 division,
            rint = round half to even); all codes are 0 when s == 0
  value   = code * s                             (dequantized)
  qmax    = 127 for 8 bits, 7 for 4 bits (symmetric: -128 and -8 are never
            produced)

The codes divide by the *stored* fp16 scale so that dequantization code*s is
consistent with the stored data. Inputs are finite float32 (decoded bf16).
A scale that overflows fp16 (amax > 65504 * qmax) is stored as +inf and its
codes are all 0.
"""
from __future__ import annotations

import numpy as np

QMAX = {8: 127, 4: 7}
BLOCK = 16


def quantize_tiles(x: np.ndarray, bits: int, block_size: int = BLOCK):
    """x: float32 [num_blocks*block_size, n_kv, d] (slot form).

    Returns (codes int8 [same shape], scales float16 [num_blocks, n_kv]).
    """
    qmax = QMAX[bits]
    x = np.asarray(x, dtype=np.float32)
    ns, n_kv, d = x.shape
    nb = ns // block_size
    t = x.reshape(nb, block_size, n_kv, d)
    amax = np.abs(t).max(axis=(1, 3))                       # float32 [nb, n_kv]
    s32 = (amax / np.float32(qmax)).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    sf = s16.astype(np.float32)[:, None, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (t / sf).astype(np.float32)
    c = np.clip(np.rint(r), -qmax, qmax)
    c = np.where(sf == 0, 0.0, c)
    c = np.where(np.isfinite(r), c, 0.0)
    return c.astype(np.int8).reshape(ns, n_kv, d), s16


def dequantize(codes: np.ndarray, scales: np.ndarray, block_size: int = BLOCK) -> np.ndarray:
    """Exact float64 values code * s of slot-form codes with [num_blocks, n_kv]
    fp16 scales."""
    codes = np.asarray(codes)
    ns, n_kv, d = codes.shape
    nb = ns // block_size
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    v = codes.reshape(nb, block_size, n_kv, d).astype(np.float64) * s[:, None, :, None]
    return v.reshape(ns, n_kv, d)


# ---------------------------------------------------------------------------
# fp8 (OCP e4m3) variant. The pages name fp8 as the usual KV-cache
# quantization knob ([TAI] "The KV cache": quantizing the cache to fp8;
# [IR] "The debate": fp8 KV) without a formula. Reading: the same group and
# scale as above with qmax replaced by the largest finite e4m3 value (448),
# and the code being the e4m3 value nearest x / s instead of an integer:
#
#   s     = float16(float32(amax) / 448)           (as above)
#   code  = e4m3 value nearest float32(x / s), ties to the even code,
#           magnitudes beyond 448 saturating to 448, the sign of x kept
#           (a negative x that rounds to zero is -0, code 0x80); all codes
#           are 0x00 when s is 0 or not finite
#   value = e4m3(code) * s
#
# e4m3 (OCP 8-bit floating point, E4M3): bit 7 sign, bits 6..3 exponent
# (bias 7), bits 2..0 mantissa; exponent 0 holds the subnormals m * 2^-9;
# no infinities; 0x7F and 0xFF are NaN (never produced by the rounding).
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Exact float64 value of e4m3 code(s) (0..255)."""
    c = np.asarray(code).astype(np.int64)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    v = np.where(c & 0x80, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


_E4M3_POS = e4m3_value(np.arange(127))  # codes 0..126: 0 .. 448, increasing


def e4m3_round(r) -> np.ndarray:
    """e4m3 code (uint8) of the value nearest each float32 r, ties to the even
    code, |r| > 448 saturating to 448, sign bit from r."""
    r = np.asarray(r, dtype=np.float32)
    a = np.minimum(np.abs(r).astype(np.float64), E4M3_MAX)
    hi = np.minimum(np.searchsorted(_E4M3_POS, a, side="left"), 126)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    return (code | np.where(np.signbit(r), 0x80, 0)).astype(np.uint8)


def quantize_tiles_fp8(x: np.ndarray, block_size: int = BLOCK):
    """x: float32 [num_blocks*block_size, n_kv, d] (slot form).

    Returns (codes uint8 e4m3 [same shape], scales float16 [num_blocks, n_kv]).
    """
    x = np.asarray(x, dtype=np.float32)
    ns, n_kv, d = x.shape
    nb = ns // block_size
    t = x.reshape(nb, block_size, n_kv, d)
    amax = np.abs(t).max(axis=(1, 3))
    s32 = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    sf = s16.astype(np.float32)[:, None, :, None]
    usable = (sf > 0) & np.isfinite(sf)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(usable, t / np.where(usable, sf, np.float32(1)), np.float32(0)).astype(np.float32)
    c = np.where(usable, e4m3_round(r), np.uint8(0)).astype(np.uint8)
    return c.reshape(ns, n_kv, d), s16


def dequantize_fp8(codes: np.ndarray, scales: np.ndarray, block_size: int = BLOCK) -> np.ndarray:
    """Exact float64 values e4m3(code) * s of slot-form e4m3 codes with
    [num_blocks, n_kv] fp16 scales."""
    codes = np.asarray(codes, dtype=np.uint8)
    ns, n_kv, d = codes.shape
    nb = ns // block_size
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    v = e4m3_value(codes).reshape(nb, block_size, n_kv, d) * s[:, None, :, None]
    return v.reshape(ns, n_kv, d)
