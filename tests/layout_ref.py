"""NumPy statement of the device pool layout that include/paged_attn.h
documents, used by the tests to build device pools byte by byte and to read
them back. Written from the header's formula, independently of the kernels:

  tile (block b, KV head h) at ((b * n_kv) + h) * tile_bytes,
  tile_bytes = 16 * d * bits / 8; inside a tile element (slot t, dim i) is
  element number
      K: ((i // x) * 16 + t) * x + i % x,   x = 128 // bits
      V: i * 16 + t   (int4: (((i % 16) * 2 + t // 8) * (d // 16) + i // 16) * 8 + t % 8)
  packed at `bits` each, little-endian; int4 pairs put the even element in
  the low nibble.
"""
import numpy as np


def elem_index(kind: str, d: int, bits: int) -> np.ndarray:
    """[16, d] array: element number of (slot t, dim i) inside a tile."""
    t = np.arange(16)[:, None]
    i = np.arange(d)[None, :]
    if kind == "k":
        x = 128 // bits
        return ((i // x) * 16 + t) * x + i % x
    if bits == 4:
        return (((i % 16) * 2 + t // 8) * (d // 16) + i // 16) * 8 + t % 8
    return i * 16 + t + 0 * t


def _np_dtype(bits):
    return {32: np.uint32, 16: np.uint16, 8: np.uint8}[bits]


def pack_pool(slots: np.ndarray, kind: str, bits: int) -> np.ndarray:
    """slots [NB*16, n_kv, d] (float32 / bf16 bits uint16 / int8 codes)
    -> uint8 [NB, n_kv, tile_bytes] device image."""
    ns, n_kv, d = slots.shape
    nb = ns // 16
    tiles = np.ascontiguousarray(slots.reshape(nb, 16, n_kv, d).transpose(0, 2, 1, 3))  # [nb, n_kv, 16, d]
    idx = elem_index(kind, d, bits)
    if bits == 4:
        codes = tiles.astype(np.int8).view(np.uint8) & 0xF
        flat = np.zeros((nb, n_kv, 16 * d), dtype=np.uint8)
        flat[:, :, idx] = codes
        return (flat[:, :, 0::2] | (flat[:, :, 1::2] << 4)).astype(np.uint8)
    raw = tiles.view(_np_dtype(bits)) if tiles.dtype.itemsize * 8 == bits else tiles.astype(_np_dtype(bits))
    flat = np.zeros((nb, n_kv, 16 * d), dtype=_np_dtype(bits))
    flat[:, :, idx] = raw
    return flat.view(np.uint8).reshape(nb, n_kv, -1)


def unpack_pool(img: np.ndarray, kind: str, bits: int, d: int) -> np.ndarray:
    """uint8 [NB, n_kv, tile_bytes] -> slots [NB*16, n_kv, d] (int8 codes for
    bits <= 8, raw uint16 / uint32 patterns otherwise)."""
    nb, n_kv, _ = img.shape
    idx = elem_index(kind, d, bits)
    if bits == 4:
        lo = (img & 0xF).astype(np.int16)
        hi = (img >> 4).astype(np.int16)
        flat = np.empty((nb, n_kv, 16 * d), dtype=np.int16)
        flat[:, :, 0::2] = lo
        flat[:, :, 1::2] = hi
        flat = np.where(flat >= 8, flat - 16, flat).astype(np.int8)
    elif bits == 8:
        flat = img.view(np.int8)
    else:
        flat = np.ascontiguousarray(img).view(_np_dtype(bits)).reshape(nb, n_kv, 16 * d)
    tiles = flat[:, :, idx]  # [nb, n_kv, 16, d]
    return np.ascontiguousarray(tiles.transpose(0, 2, 1, 3)).reshape(nb * 16, n_kv, d)
