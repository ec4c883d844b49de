"""Pure-Python brute force (tiny inputs only): used to pin the NumPy oracle.

No NumPy arithmetic here: plain loops, math.exp, float (IEEE double) and the
struct module for float32/float16 rounding, so a slip in the vectorised
oracle (a transposed operand, a wrong head mapping, a dropped term) shows up
as a disagreement.
"""
from __future__ import annotations

import math
import struct


def _f32(x: float) -> float:
    """Round a double to the nearest float32 (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _f16(x: float) -> float:
    """Round to the nearest float16 (ties to even); overflow -> inf."""
    try:
        return struct.unpack("<e", struct.pack("<e", x))[0]
    except OverflowError:
        return math.copysign(math.inf, x)


def decode_attention(q, k_pool, v_pool, table, n_ctx, n_kv, block_size=16, window=None):
    """q: nested lists [H][D]; pools: nested lists [slot][n_kv][D].
    Returns [H][D] with scale 1/sqrt(D), kv head = h // (H / n_kv). With a
    window W only the tokens t with n_ctx - W <= t < n_ctx are attended."""
    H = len(q)
    D = len(q[0])
    G = H // n_kv
    first = 0 if window is None else max(0, n_ctx - window)
    out = []
    for h in range(H):
        kvh = h // G
        scores = []
        for t in range(first, n_ctx):
            slot = table[t // block_size] * block_size + t % block_size
            dot = 0.0
            for i in range(D):
                dot += q[h][i] * k_pool[slot][kvh][i]
            scores.append(dot / math.sqrt(D))
        m = max(scores)
        w = [math.exp(z - m) for z in scores]
        tot = sum(w)
        row = [0.0] * D
        for t in range(first, n_ctx):
            slot = table[t // block_size] * block_size + t % block_size
            for i in range(D):
                row[i] += w[t - first] / tot * v_pool[slot][kvh][i]
        out.append(row)
    return out


def prefill_attention(qrows, k_pool, v_pool, table, n_ctx, n_kv, block_size=16, window=None):
    """qrows: [q_len][H][D], the last q_len tokens of a context of n_ctx.
    Row i attends keys 0..n_ctx-q_len+i (with a window W, only the last W of
    them)."""
    q_len = len(qrows)
    out = []
    for i in range(q_len):
        pos = n_ctx - q_len + i
        out.append(decode_attention(qrows[i], k_pool, v_pool, table, pos + 1, n_kv, block_size, window=window))
    return out


def quantize_tile(values, bits):
    """values: flat list of float32 numbers of one (block, KV head) group.
    Returns (codes list of ints, scale as a Python float holding the fp16)."""
    qmax = {8: 127, 4: 7}[bits]
    amax = 0.0
    for x in values:
        amax = max(amax, abs(x))
    s32 = _f32(amax / qmax)          # fl32(fl64(a/b)) == fl32(a/b) for float32 a, b
    s = _f16(s32)
    codes = []
    for x in values:
        if s == 0.0 or math.isinf(s):
            codes.append(0)
            continue
        r = _f32(x / s)
        c = round(r)                  # Python round(): half to even
        codes.append(max(-qmax, min(qmax, c)))
    return codes, s


def e4m3_table():
    """(code, value) of the 127 non-negative finite OCP e4m3 codes, built with
    math.ldexp from the bit fields: exponent field e (bias 7), mantissa m;
    e == 0 gives the subnormal m / 8 * 2^-6."""
    out = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        v = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
        out.append((code, v))
    return out


def quantize_tile_fp8(values):
    """values: flat list of float32 numbers of one group. Returns (list of
    e4m3 codes, fp16 scale as a Python float): s = fp16(fp32(amax / 448));
    each code is the non-negative e4m3 value nearest |x / s| (searched over
    every code, ties to the even code, beyond 448 saturating), with the sign
    bit of x / s; all 0x00 when s is 0 or infinite."""
    table = e4m3_table()
    amax = 0.0
    for x in values:
        amax = max(amax, abs(x))
    s = _f16(_f32(amax / 448.0))
    codes = []
    for x in values:
        if s == 0.0 or math.isinf(s):
            codes.append(0)
            continue
        r = _f32(x / s)
        a = min(abs(r), 448.0)
        best, best_d = None, None
        for code, v in table:
            d = abs(v - a)
            if best is None or d < best_d or (d == best_d and code % 2 == 0):
                best, best_d = code, d
        codes.append(best | (0x80 if math.copysign(1.0, r) < 0 else 0))
    return codes, s
