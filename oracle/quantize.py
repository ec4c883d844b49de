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
