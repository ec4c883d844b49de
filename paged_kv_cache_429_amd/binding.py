"""ctypes binding of libpagedattn.so (include/paged_attn.h).

Argument marshalling only: every step of decode, prefill, quantization and
cache writes runs in the library's HIP kernels. PyTorch supplies device
memory and the current stream. There is no fallback: if the library is not
built, or a tensor is not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_OK = 0
PA_F32, PA_BF16 = 0, 1
PA_KIND_K, PA_KIND_V = 0, 1
PA_KV_FP8 = 264  # kv_bits code of OCP fp8 e4m3 pools
BLOCK_SIZE = 16

# every function declared in include/paged_attn.h and include/pa_block_manager.h
EXPORTS = (
    "pa_error_string", "pa_tile_bytes", "pa_kv_bytes_per_token", "pa_kv_cache_bytes",
    "paged_attn_decode_workspace_size", "paged_attn_decode", "paged_attn_decode_window", "paged_attn_prefill_chunk",
    "paged_attn_decode_noalloc", "paged_attn_prefill_chunk_window",
    "kv_quantize", "paged_kv_write", "paged_kv_append", "pa_copy_blocks", "pa_hbm_read_probe", "pa_take_block_id_error",
    "pa_bm_create", "pa_bm_destroy", "pa_bm_num_free", "pa_bm_ref_count", "pa_bm_add", "pa_bm_append",
    "pa_bm_fork", "pa_bm_release", "pa_bm_num_tokens", "pa_bm_table",
    "pa_sched_create", "pa_sched_destroy", "pa_sched_submit", "pa_sched_num_live", "pa_sched_step",
    "pa_sched_record", "pa_sched_finish",
)

_lib = None
_lock = threading.Lock()


class PagedAttnError(RuntimeError):
    pass


def _declare(lib):
    i, sz, vp, u64, i64 = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64
    lib.pa_error_string.restype = ctypes.c_char_p
    lib.pa_error_string.argtypes = [i]
    lib.pa_tile_bytes.restype = sz
    lib.pa_tile_bytes.argtypes = [i, i]
    lib.pa_kv_bytes_per_token.restype = u64
    lib.pa_kv_bytes_per_token.argtypes = [i, i, i, i]
    lib.pa_kv_cache_bytes.restype = u64
    lib.pa_kv_cache_bytes.argtypes = [i, i, i, i, i64]
    lib.paged_attn_decode_workspace_size.restype = sz
    lib.paged_attn_decode_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.paged_attn_decode.restype = i
    lib.paged_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, i, i, i, i, i, i, i, i, i, vp, vp, sz, i, vp]
    lib.paged_attn_decode_window.restype = i
    lib.paged_attn_decode_window.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, i, i, i, i, i, i, i, i, i, vp, vp, sz, i, i,
                                             vp]
    lib.paged_attn_decode_noalloc.restype = i
    lib.paged_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, i, i, i, i, i, i, i, i, i, vp, i, vp]
    lib.paged_attn_prefill_chunk.restype = i
    lib.paged_attn_prefill_chunk.argtypes = [vp, vp, i, i, vp, vp, vp, vp, vp, i, vp, i, i, i, i, i, i, i, i, i,
                                             vp, vp]
    lib.paged_attn_prefill_chunk_window.restype = i
    lib.paged_attn_prefill_chunk_window.argtypes = [vp, vp, i, i, vp, vp, vp, vp, vp, i, vp, i, i, i, i, i, i, i,
                                                    i, i, vp, i, vp]
    lib.kv_quantize.restype = i
    lib.kv_quantize.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.paged_kv_write.restype = i
    lib.paged_kv_write.argtypes = [vp, vp, vp, i, vp, vp, i, i, i, i, i, vp]
    lib.paged_kv_append.restype = i
    lib.paged_kv_append.argtypes = [vp, vp, vp, i, i, vp, i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.pa_copy_blocks.restype = i
    lib.pa_copy_blocks.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.pa_hbm_read_probe.restype = i
    lib.pa_hbm_read_probe.argtypes = [vp, i64, i, vp, i64, vp, i, vp]
    lib.pa_take_block_id_error.restype = i
    lib.pa_take_block_id_error.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_int32)]
    # host block manager and scheduler (opaque handles)
    lib.pa_bm_create.restype = vp
    lib.pa_bm_create.argtypes = [i, i]
    lib.pa_bm_destroy.restype = None
    lib.pa_bm_destroy.argtypes = [vp]
    lib.pa_bm_num_free.restype = i
    lib.pa_bm_num_free.argtypes = [vp]
    lib.pa_bm_ref_count.restype = i
    lib.pa_bm_ref_count.argtypes = [vp, i]
    lib.pa_bm_add.restype = i
    lib.pa_bm_add.argtypes = [vp, i64, vp, i, vp]
    lib.pa_bm_append.restype = i
    lib.pa_bm_append.argtypes = [vp, i64, vp, vp]
    lib.pa_bm_fork.restype = i
    lib.pa_bm_fork.argtypes = [vp, i64, i64]
    lib.pa_bm_release.restype = i
    lib.pa_bm_release.argtypes = [vp, i64]
    lib.pa_bm_num_tokens.restype = i
    lib.pa_bm_num_tokens.argtypes = [vp, i64]
    lib.pa_bm_table.restype = i
    lib.pa_bm_table.argtypes = [vp, i64, vp, i]
    lib.pa_sched_create.restype = vp
    lib.pa_sched_create.argtypes = [vp]
    lib.pa_sched_destroy.restype = None
    lib.pa_sched_destroy.argtypes = [vp]
    lib.pa_sched_submit.restype = i
    lib.pa_sched_submit.argtypes = [vp, i64, vp, i]
    lib.pa_sched_num_live.restype = i
    lib.pa_sched_num_live.argtypes = [vp]
    lib.pa_sched_step.restype = i
    lib.pa_sched_step.argtypes = [vp, i, vp, vp, vp, vp, vp, vp, vp]
    lib.pa_sched_record.restype = i
    lib.pa_sched_record.argtypes = [vp, i64, i64]
    lib.pa_sched_finish.restype = i
    lib.pa_sched_finish.argtypes = [vp, i64]


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise PagedAttnError(f"{LIB_PATH} is missing: build it with "
                                         "`python -m paged_kv_cache_429_amd.build`")
                h = ctypes.CDLL(LIB_PATH)
                _declare(h)
                _lib = h
    return _lib


def _check(name, status):
    if status != PA_OK:
        msg = lib().pa_error_string(status).decode()
        raise PagedAttnError(f"{name} failed: {msg} ({status})")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise PagedAttnError("tensors must be on a GPU")
        if not t.is_contiguous():
            raise PagedAttnError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise PagedAttnError("tensors must be on one device")
    return dev


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(dt):
    if dt == torch.float32:
        return PA_F32
    if dt == torch.bfloat16:
        return PA_BF16
    raise PagedAttnError(f"unsupported query dtype {dt}")


def tile_bytes(d_head: int, kv_bits: int) -> int:
    return int(lib().pa_tile_bytes(d_head, kv_bits))


def kv_bytes_per_token(n_layers, n_kv_heads, d_head, kv_bits) -> int:
    return int(lib().pa_kv_bytes_per_token(n_layers, n_kv_heads, d_head, kv_bits))


def kv_cache_bytes(n_layers, n_kv_heads, d_head, kv_bits, n_tokens) -> int:
    return int(lib().pa_kv_cache_bytes(n_layers, n_kv_heads, d_head, kv_bits, n_tokens))


def alloc_pool(num_blocks, n_kv_heads, d_head, kv_bits, device="cuda"):
    """Uninitialised pool in the library's tile layout (raw bytes)."""
    return torch.empty((num_blocks, n_kv_heads, tile_bytes(d_head, kv_bits)), dtype=torch.uint8, device=device)


def alloc_scales(num_blocks, n_kv_heads, device="cuda"):
    return torch.empty((num_blocks, n_kv_heads), dtype=torch.float16, device=device)


def _num_blocks(pool, n_kv, d, kv_bits):
    per = n_kv * tile_bytes(d, kv_bits)
    nbytes = pool.numel() * pool.element_size()
    if per == 0 or nbytes % per:
        raise PagedAttnError("pool size is not a whole number of blocks")
    return nbytes // per


_ws = {}


def decode_workspace(num_seqs, n_heads, n_kv_heads, d_head, max_context_len, partition_blocks=0,
                     device=None, stream=None):
    """A workspace large enough for the call, cached per (device, stream).
    It needs no initialisation (its arrival words are tagged with each
    call's epoch). It is allocated from the pool of the stream that uses it,
    so a buffer it replaces is reused only by work ordered after the calls
    on that stream."""
    n = int(lib().paged_attn_decode_workspace_size(num_seqs, n_heads, n_kv_heads, d_head, max_context_len,
                                                   partition_blocks))
    if n == 0:
        return None
    device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    s = stream if stream is not None else torch.cuda.current_stream(device)
    key = (device.index, s.cuda_stream)
    buf = _ws.get(key)
    if buf is None or buf.numel() < n:
        with torch.cuda.stream(s):
            buf = torch.empty(max(n, 4 << 20), dtype=torch.uint8, device=device)
        _ws[key] = buf
    return buf


def decode(q, k_pool, v_pool, block_tables, context_lens, *, n_kv_heads, max_context_len, kv_bits=None,
           k_scales=None, v_scales=None, out=None, workspace=None, partition_blocks=0, stream=None, window=None):
    """paged_attn_decode, or paged_attn_decode_window when a window (tokens,
    >= 1) is given. q [S, H, D] (float32 or bfloat16); block_tables
    [S, max_blocks] int32; context_lens [S] int32; returns out [S, H, D]."""
    dev = _gpu(q, k_pool, v_pool, block_tables, context_lens, k_scales, v_scales, out, workspace)
    S, H, D = q.shape
    dt = _dtype_code(q.dtype)
    if kv_bits is None:
        kv_bits = 32 if dt == PA_F32 else 16
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise PagedAttnError("block_tables and context_lens must be int32")
    nb = _num_blocks(k_pool, n_kv_heads, D, kv_bits)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = decode_workspace(S, H, n_kv_heads, D, max_context_len, partition_blocks, dev, stream)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_p(q), _p(k_pool), _p(v_pool), _p(k_scales), _p(v_scales), _p(block_tables), block_tables.shape[1],
            _p(context_lens), int(max_context_len), S, nb, BLOCK_SIZE, H, n_kv_heads, D, dt, kv_bits,
            _p(out), _p(workspace), wbytes, int(partition_blocks))
    if window is None:
        _check("paged_attn_decode", lib().paged_attn_decode(*args, _stream(stream, dev)))
    else:
        _check("paged_attn_decode_window",
               lib().paged_attn_decode_window(*args, int(window), _stream(stream, dev)))
    return out


def prefill_chunk(q, cu_q_lens, k_pool, v_pool, block_tables, context_lens, *, n_kv_heads, max_q_len,
                  max_context_len, kv_bits=None, k_scales=None, v_scales=None, out=None, stream=None, window=None):
    """paged_attn_prefill_chunk, or paged_attn_prefill_chunk_window when a
    window (tokens, >= 1) is given. q [total_q, H, D]; cu_q_lens [S+1] int32."""
    dev = _gpu(q, cu_q_lens, k_pool, v_pool, block_tables, context_lens, k_scales, v_scales, out)
    T, H, D = q.shape
    dt = _dtype_code(q.dtype)
    if kv_bits is None:
        kv_bits = 32 if dt == PA_F32 else 16
    nb = _num_blocks(k_pool, n_kv_heads, D, kv_bits)
    if out is None:
        out = torch.empty_like(q)
    S = context_lens.shape[0]
    args = (_p(q), _p(cu_q_lens), T, int(max_q_len), _p(k_pool), _p(v_pool), _p(k_scales), _p(v_scales),
            _p(block_tables), block_tables.shape[1], _p(context_lens), int(max_context_len), S, nb, BLOCK_SIZE,
            H, n_kv_heads, D, dt, kv_bits, _p(out))
    if window is None:
        _check("paged_attn_prefill_chunk", lib().paged_attn_prefill_chunk(*args, _stream(stream, dev)))
    else:
        _check("paged_attn_prefill_chunk_window",
               lib().paged_attn_prefill_chunk_window(*args, int(window), _stream(stream, dev)))
    return out


def quantize(src_pool, *, bits, kind, n_kv_heads, d_head, codes=None, scales=None, block_ids=None, stream=None):
    """kv_quantize of a bf16 pool; returns (codes pool, fp16 scales)."""
    dev = _gpu(src_pool, codes, scales, block_ids)
    nb = _num_blocks(src_pool, n_kv_heads, d_head, 16)
    if codes is None:
        codes = alloc_pool(nb, n_kv_heads, d_head, bits, dev)
    if scales is None:
        scales = alloc_scales(nb, n_kv_heads, dev)
    n_ids = 0 if block_ids is None else block_ids.numel()
    st = lib().kv_quantize(_p(src_pool), _p(codes), _p(scales), _p(block_ids), n_ids, nb, n_kv_heads, BLOCK_SIZE,
                           d_head, bits, kind, _stream(stream, dev))
    _check("kv_quantize", st)
    return codes, scales


def kv_write(k_src, v_src, slot_mapping, k_pool, v_pool, *, n_kv_heads, stream=None):
    """paged_kv_write: k_src/v_src [T, n_kv, D] float32 or bfloat16; slot_mapping [T] int64."""
    src = k_src if k_src is not None else v_src
    dev = _gpu(k_src, v_src, slot_mapping, k_pool, v_pool)
    T, _, D = src.shape
    dt = _dtype_code(src.dtype)
    if slot_mapping.dtype != torch.int64:
        raise PagedAttnError("slot_mapping must be int64")
    kv_bits = 32 if dt == PA_F32 else 16
    nb = _num_blocks(k_pool if k_pool is not None else v_pool, n_kv_heads, D, kv_bits)
    st = lib().paged_kv_write(_p(k_src), _p(v_src), _p(slot_mapping), T, _p(k_pool), _p(v_pool), nb, BLOCK_SIZE,
                              n_kv_heads, D, dt, _stream(stream, dev))
    _check("paged_kv_write", st)


def kv_append(k_new, v_new, cu_new, block_tables, context_lens, k_pool, v_pool, *, n_kv_heads, max_new,
              kv_bits=None, k_scales=None, v_scales=None, k_stage=None, v_stage=None, stream=None):
    """paged_kv_append: k_new/v_new [T, n_kv, D] float32 or bfloat16 (either
    may be None); cu_new [S+1] int32; context_lens [S] int32 (lengths after
    the append). Quantized pools need their scales and bf16 staging tiles
    [S, n_kv, 16, D]."""
    src = k_new if k_new is not None else v_new
    dev = _gpu(k_new, v_new, cu_new, block_tables, context_lens, k_pool, v_pool, k_scales, v_scales, k_stage,
               v_stage)
    T, _, D = src.shape
    dt = _dtype_code(src.dtype)
    if kv_bits is None:
        kv_bits = 32 if dt == PA_F32 else 16
    for t, name in ((cu_new, "cu_new"), (block_tables, "block_tables"), (context_lens, "context_lens")):
        if t.dtype != torch.int32:
            raise PagedAttnError(f"{name} must be int32")
    nb = _num_blocks(k_pool if k_pool is not None else v_pool, n_kv_heads, D, kv_bits)
    S = context_lens.shape[0]
    st = lib().paged_kv_append(_p(k_new), _p(v_new), _p(cu_new), T, int(max_new), _p(block_tables),
                               block_tables.shape[1], _p(context_lens), _p(k_pool), _p(v_pool), _p(k_scales),
                               _p(v_scales), _p(k_stage), _p(v_stage), S, nb, BLOCK_SIZE, n_kv_heads, D, dt, kv_bits,
                               _stream(stream, dev))
    _check("paged_kv_append", st)


def copy_blocks(pairs, k_pool, v_pool, *, n_kv_heads, d_head, kv_bits, k_scales=None, v_scales=None, stream=None):
    """pa_copy_blocks: pairs int32 [n, 2] (source, destination) on the pools' device."""
    dev = _gpu(pairs, k_pool, v_pool, k_scales, v_scales)
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2 or not pairs.is_contiguous():
        raise PagedAttnError("pairs must be a contiguous int32 [n, 2] tensor")
    nb = _num_blocks(k_pool if k_pool is not None else v_pool, n_kv_heads, d_head, kv_bits)
    st = lib().pa_copy_blocks(_p(k_pool), _p(v_pool), _p(k_scales), _p(v_scales), _p(pairs), int(pairs.shape[0]),
                              nb, n_kv_heads, d_head, kv_bits, _stream(stream, dev))
    _check("pa_copy_blocks", st)


def take_block_id_error():
    """pa_take_block_id_error: None, or (table index, block id) of the first
    out-of-range block-table entry a kernel met since the last take."""
    idx, bid = ctypes.c_int64(-1), ctypes.c_int32(0)
    r = lib().pa_take_block_id_error(ctypes.byref(idx), ctypes.byref(bid))
    _check("pa_take_block_id_error", min(r, 0))
    return (idx.value, bid.value) if r == 1 else None


def hbm_read_probe(buf, tile_bytes, *, order=None, grid=2048, xor_out=None, stream=None):
    """pa_hbm_read_probe over a uint8 device buffer cut into tiles of
    tile_bytes; returns the per-workgroup XOR words (int32 [grid])."""
    dev = _gpu(buf, order, xor_out)
    if order is not None and order.dtype != torch.int32:
        raise PagedAttnError("order must be int32")
    if xor_out is None:
        xor_out = torch.empty(grid, dtype=torch.int32, device=dev)
    st = lib().pa_hbm_read_probe(_p(buf), buf.numel(), tile_bytes, _p(order), 0 if order is None else order.numel(),
                                 _p(xor_out), grid, _stream(stream, dev))
    _check("pa_hbm_read_probe", st)
    return xor_out


class BlockManager:
    """The library's host block manager (include/pa_block_manager.h)."""

    def __init__(self, num_blocks: int, prefix_cache: bool = True):
        self._h = lib().pa_bm_create(int(num_blocks), int(bool(prefix_cache)))
        if not self._h:
            raise PagedAttnError("pa_bm_create failed")

    def close(self):
        if self._h:
            lib().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def num_free(self) -> int:
        return lib().pa_bm_num_free(self._h)

    def ref_count(self, block: int) -> int:
        return lib().pa_bm_ref_count(self._h, int(block))

    def add(self, seq: int, tokens) -> int:
        arr = (ctypes.c_int64 * len(tokens))(*[int(t) for t in tokens])
        cached = ctypes.c_int(0)
        _check("pa_bm_add", lib().pa_bm_add(self._h, int(seq), arr, len(tokens), ctypes.byref(cached)))
        return cached.value

    def append(self, seq: int):
        src, dst = ctypes.c_int32(-1), ctypes.c_int32(-1)
        _check("pa_bm_append", lib().pa_bm_append(self._h, int(seq), ctypes.byref(src), ctypes.byref(dst)))
        return None if src.value < 0 else (src.value, dst.value)

    def fork(self, parent: int, child: int) -> None:
        _check("pa_bm_fork", lib().pa_bm_fork(self._h, int(parent), int(child)))

    def release(self, seq: int) -> None:
        _check("pa_bm_release", lib().pa_bm_release(self._h, int(seq)))

    def num_tokens(self, seq: int) -> int:
        n = lib().pa_bm_num_tokens(self._h, int(seq))
        _check("pa_bm_num_tokens", min(n, 0))
        return n

    def table(self, seq: int):
        n = lib().pa_bm_table(self._h, int(seq), None, 0)
        _check("pa_bm_table", min(n, 0))
        row = (ctypes.c_int32 * max(n, 1))()
        lib().pa_bm_table(self._h, int(seq), row, n)
        return list(row[:n])


class Scheduler:
    """The library's scheduler step over a BlockManager."""

    def __init__(self, bm: BlockManager):
        self.bm = bm
        self._h = lib().pa_sched_create(bm.handle)
        if not self._h:
            raise PagedAttnError("pa_sched_create failed")

    def close(self):
        if self._h:
            lib().pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def submit(self, seq: int, prompt) -> None:
        arr = (ctypes.c_int64 * len(prompt))(*[int(t) for t in prompt])
        _check("pa_sched_submit", lib().pa_sched_submit(self._h, int(seq), arr, len(prompt)))

    def step(self):
        """(running, preempted, cow pairs, stalled count)."""
        cap = max(1, lib().pa_sched_num_live(self._h))
        run, pre = (ctypes.c_int64 * cap)(), (ctypes.c_int64 * cap)()
        cow = (ctypes.c_int32 * (2 * cap))()
        nr, npre, nc, ns = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check("pa_sched_step", lib().pa_sched_step(self._h, cap, run, ctypes.byref(nr), pre, ctypes.byref(npre),
                                                    cow, ctypes.byref(nc), ctypes.byref(ns)))
        pairs = [(cow[2 * i], cow[2 * i + 1]) for i in range(nc.value)]
        return list(run[:nr.value]), list(pre[:npre.value]), pairs, ns.value

    def record(self, seq: int, token: int) -> None:
        _check("pa_sched_record", lib().pa_sched_record(self._h, int(seq), int(token)))

    def finish(self, seq: int) -> None:
        _check("pa_sched_finish", lib().pa_sched_finish(self._h, int(seq)))
