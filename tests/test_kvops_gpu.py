"""GPU: cache writes and quantization are bit-exact; quantized decode matches
the oracle on exactly dequantized codes."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_429_amd import binding as B
from synth import make_config_case, make_decode_case, make_probe_case
from synth.gen import bf16_bits_to_f32
from tests.gpu_util import assert_close, dev_to_f64, gpu_decode, np_to_dev, oracle_decode, upload_pools
from tests.layout_ref import pack_pool, unpack_pool

pytestmark = pytest.mark.gpu


def _img(t):
    return t.cpu().numpy().view(np.uint8)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_kv_write_layout_bitexact(lib, dtype, d):
    c = make_decode_case(8, 4, d, dtype, [37, 16, 5], 400, pool_factor=2.0)
    kp, vp = upload_pools(c)
    bits = 32 if dtype == "f32" else 16
    assert np.array_equal(_img(kp), pack_pool(c.k_slots, "k", bits))
    assert np.array_equal(_img(vp), pack_pool(c.v_slots, "v", bits))


def test_kv_write_partial_and_skipped_slots(lib):
    c = make_decode_case(8, 2, 128, "bf16", [40], 401, pool_factor=2.0)
    kp, vp = upload_pools(c)
    before_k, before_v = _img(kp).copy(), _img(vp).copy()
    g = np.random.default_rng(0)
    slots = np.array([3, -1, 17, c.num_blocks * 16 + 5, 40], dtype=np.int64)
    newk = g.integers(0, 1 << 15, size=(5, 2, 128)).astype(np.uint16)
    newv = g.integers(0, 1 << 15, size=(5, 2, 128)).astype(np.uint16)
    B.kv_write(np_to_dev(newk, "bf16"), np_to_dev(newv, "bf16"), torch.from_numpy(slots).cuda(), kp, vp,
               n_kv_heads=2)
    torch.cuda.synchronize()
    ks, vs = c.k_slots.copy(), c.v_slots.copy()
    for i, sl in enumerate(slots):
        if 0 <= sl < c.num_blocks * 16:
            ks[sl], vs[sl] = newk[i], newv[i]
    assert np.array_equal(_img(kp), pack_pool(ks, "k", 16))
    assert np.array_equal(_img(vp), pack_pool(vs, "v", 16))
    assert not np.array_equal(_img(kp), before_k)


def _mixed_slot_mapping(num_blocks, seed):
    """A slot list mixing whole blocks written in order (some starting just
    before a multiple of 64 source rows, so that the block's tokens span two
    groups of 64), a block with one slot out of place, a block written in
    reverse, a partly written block, scattered single slots, and skipped
    (negative, out-of-range) entries. Every slot appears at most once."""
    g = np.random.default_rng(seed)
    blocks = iter(g.permutation(num_blocks).tolist())
    out = []

    def block_run(n=16):  # the first n slots of a fresh block, in order
        b = next(blocks)
        return [b * 16 + j for j in range(n)]

    def pad_to(n):  # single slots, every other slot of fresh blocks, until len(out) == n
        while len(out) < n:
            out.extend(block_run()[::2][: n - len(out)])
    out += block_run()                      # run at row 0
    pad_to(49)
    out += block_run()                      # run at rows 49..64
    out += [-1, num_blocks * 16 + 3]        # skipped
    pad_to(127)
    out += block_run()                      # head at row 127, the last row of a group of 64
    run = block_run()
    run[7] = next(blocks) * 16 + 2          # one slot out of place: no run
    out += run
    out += block_run()[::-1]                # reversed
    out += block_run(10)                    # partly written block
    for _ in range(5):
        out += block_run()                  # plain runs
    out.append(next(blocks) * 16 + 5)       # a last single slot
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_kv_write_runs_and_scattered_slots(lib, dtype, d):
    """Whole-block runs (written as tiles) and tokens written one by one in
    the same call land exactly where the slot list says; every other byte of
    the pools is untouched."""
    c = make_decode_case(8, 2, d, dtype, [40], 403 + d, pool_blocks=64)
    kp, vp = upload_pools(c)
    slots = _mixed_slot_mapping(c.num_blocks, 404 + d)
    n = len(slots)
    g = np.random.default_rng(405 + d)
    if dtype == "f32":
        newk = g.standard_normal((n, 2, d)).astype(np.float32)
        newv = g.standard_normal((n, 2, d)).astype(np.float32)
    else:
        newk = g.integers(0, 1 << 15, size=(n, 2, d)).astype(np.uint16)
        newv = g.integers(0, 1 << 15, size=(n, 2, d)).astype(np.uint16)
    B.kv_write(np_to_dev(newk, dtype), np_to_dev(newv, dtype), torch.from_numpy(slots).cuda(), kp, vp, n_kv_heads=2)
    torch.cuda.synchronize()
    ks, vs = c.k_slots.copy(), c.v_slots.copy()
    for i, sl in enumerate(slots):
        if 0 <= sl < c.num_blocks * 16:
            ks[sl], vs[sl] = newk[i], newv[i]
    bits = 32 if dtype == "f32" else 16
    assert np.array_equal(_img(kp), pack_pool(ks, "k", bits))
    assert np.array_equal(_img(vp), pack_pool(vs, "v", bits))


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("d", [64, 128])
def test_quantize_bitexact(lib, bits, kind, d):
    c = make_decode_case(8, 4, d, "bf16", [300, 77], 402 + d + bits, pool_factor=1.5)
    kp, vp = upload_pools(c)
    src = kp if kind == "k" else vp
    slots = c.k_slots if kind == "k" else c.v_slots
    codes, scales = B.quantize(src, bits=bits, kind=0 if kind == "k" else 1, n_kv_heads=4, d_head=d)
    torch.cuda.synchronize()
    ref_codes, ref_scales = oracle.quantize_tiles(bf16_bits_to_f32(slots), bits)
    got_scales = scales.cpu().numpy()
    assert np.array_equal(got_scales.view(np.uint16), ref_scales.view(np.uint16))
    got_codes = unpack_pool(_img(codes), kind, bits, d)
    assert np.array_equal(got_codes, ref_codes)
    assert np.array_equal(_img(codes), pack_pool(ref_codes, kind, bits))


def _tie_tiles(bits, d, n_kv=2, seed=406):
    """bf16 slot-form tiles whose quotients x / s land exactly on half-integers
    and one bf16 step either side: each tile's largest magnitude is qmax / 8,
    so its fp16 scale is exactly 1/8, and x = (k + 1/2) / 8 is a tie."""
    qmax = 127 if bits == 8 else 7
    g = np.random.default_rng(seed)
    nb = 6
    x = np.zeros((nb * 16, n_kv, d), dtype=np.float32)
    ties = (np.arange(-qmax, qmax) + 0.5) / 8.0
    for b in range(nb):
        for h in range(n_kv):
            vals = g.choice(ties, size=16 * d)
            step = b % 3  # 0: exact ties; 1: one bf16 step up; 2: one step down
            bits16 = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
            bits16 = bits16 + (0 if step == 0 else (1 if step == 1 else -1)) * np.sign(vals).astype(np.int64)
            vals = (bits16.astype(np.uint32) << 16).view(np.float32)
            vals[0] = qmax / 8.0 * (1 if b % 2 else -1)  # the tile's largest magnitude
            x[b * 16:(b + 1) * 16, h, :] = vals.reshape(16, d)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("kind", ["k", "v"])
def test_quantize_ties_bitexact(lib, bits, kind):
    """Quotients exactly on half-integers round to even, and one bf16 step
    either side to the nearest integer, as the oracle's float32 division."""
    d = 128
    slots = _tie_tiles(bits, d)
    src = np_to_dev(np.ascontiguousarray(pack_pool(slots, kind, 16).view(np.uint16)), "bf16")
    codes, scales = B.quantize(src, bits=bits, kind=0 if kind == "k" else 1, n_kv_heads=2, d_head=d)
    torch.cuda.synchronize()
    ref_codes, ref_scales = oracle.quantize_tiles(bf16_bits_to_f32(slots), bits)
    assert (ref_scales.astype(np.float32) == 0.125).all()
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), ref_scales.view(np.uint16))
    assert np.array_equal(unpack_pool(_img(codes), kind, bits, d), ref_codes)


def _fp8_tie_tiles(d, n_kv=2, seed=407):
    """bf16 slot-form tiles whose quotients x / s land on e4m3 rounding
    boundaries and one bf16 step either side: each tile's largest magnitude
    is 56, so its fp16 scale is exactly 56 / 448 = 1/8; the boundaries are the
    midpoints (1 + (2j+1)/16) 2^e between normal codes and (k + 1/2) / 512
    between subnormal ones."""
    g = np.random.default_rng(seed)
    mids = [(1 + (2 * j + 1) / 16) * 2.0 ** e for e in range(-6, 8) for j in range(8)]
    mids += [(k + 0.5) / 512 for k in range(8)]
    mids = np.array([m for m in mids if m < 448], dtype=np.float64) / 8.0
    nb = 6
    x = np.zeros((nb * 16, n_kv, d), dtype=np.float32)
    for b in range(nb):
        for h in range(n_kv):
            vals = (g.choice(mids, size=16 * d) * g.choice([-1.0, 1.0], size=16 * d)).astype(np.float32)
            step = b % 3  # 0: on the boundary; 1: one bf16 step out; 2: one step in
            bits16 = (vals.view(np.uint32) >> 16).astype(np.int64) + (0 if step == 0 else (1 if step == 1 else -1))
            vals = (bits16.astype(np.uint32) << 16).view(np.float32)
            vals[0] = 56.0 * (1 if b % 2 else -1)  # the tile's largest magnitude
            x[b * 16:(b + 1) * 16, h, :] = vals.reshape(16, d)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("kind", ["k", "v"])
def test_quantize_fp8_boundaries_bitexact(lib, kind):
    """e4m3 codes of quotients on rounding boundaries (ties to even) and one
    bf16 step either side match the oracle's, subnormal range included."""
    d = 128
    slots = _fp8_tie_tiles(d)
    src = np_to_dev(np.ascontiguousarray(pack_pool(slots, kind, 16).view(np.uint16)), "bf16")
    codes, scales = B.quantize(src, bits=B.PA_KV_FP8, kind=0 if kind == "k" else 1, n_kv_heads=2, d_head=d)
    torch.cuda.synchronize()
    ref_codes, ref_scales = oracle.quantize_tiles_fp8(bf16_bits_to_f32(slots))
    assert (ref_scales.astype(np.float32) == 0.125).all()
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), ref_scales.view(np.uint16))
    assert np.array_equal(unpack_pool(_img(codes), kind, 8, d), ref_codes.view(np.int8))


def test_quantize_block_subset_and_special_tiles(lib):
    c = make_decode_case(4, 2, 64, "bf16", [64], 403, pool_factor=3.0)
    # tile of zeros and a tile whose fp16 scale overflows
    c.k_slots[0:16] = 0
    c.k_slots[16:32, 0, 0] = np.uint16(0x4A80)   # 4194304.0: amax/7 > 65504
    kp, vp = upload_pools(c)
    ids = torch.tensor([0, 1, 3, 99999, -1], dtype=torch.int32, device="cuda")
    nb = c.num_blocks
    codes = B.alloc_pool(nb, 2, 64, 4)
    codes.fill_(0xAB)
    scales = B.alloc_scales(nb, 2)
    scales.fill_(7.0)
    B.quantize(kp, bits=4, kind=0, n_kv_heads=2, d_head=64, codes=codes, scales=scales, block_ids=ids)
    torch.cuda.synchronize()
    ref_codes, ref_scales = oracle.quantize_tiles(bf16_bits_to_f32(c.k_slots), 4)
    got = unpack_pool(_img(codes), "k", 4, 64)
    sc = scales.cpu().numpy()
    for b in range(nb):
        if b in (0, 1, 3):
            assert np.array_equal(got[b * 16:(b + 1) * 16], ref_codes[b * 16:(b + 1) * 16])
            assert np.array_equal(sc[b].view(np.uint16), ref_scales[b].view(np.uint16))
        else:
            assert (_img(codes)[b] == 0xAB).all() and (sc[b] == 7.0).all()
    assert np.isinf(sc[1, 0]) and sc[0, 0] == 0


def _quant_case(c, bits):
    """device int pools from the GPU quantizer, plus the oracle's own codes"""
    kp, vp = upload_pools(c)
    kc, ks = B.quantize(kp, bits=bits, kind=0, n_kv_heads=c.n_kv, d_head=c.d)
    vc, vs = B.quantize(vp, bits=bits, kind=1, n_kv_heads=c.n_kv, d_head=c.d)
    del kp, vp
    return kc, vc, ks, vs


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("n_heads,n_kv,d", [(64, 8, 128), (32, 8, 64), (16, 4, 64)])
def test_quantized_decode_parity(lib, bits, n_heads, n_kv, d):
    c = make_decode_case(n_heads, n_kv, d, "bf16", [8000, 1, 17, 4000, 515, 8000, 2222, 33], 404 + d + n_heads,
                         pool_factor=1.1)
    kc, vc, ks, vs = _quant_case(c, bits)
    rk, rks = oracle.quantize_tiles(bf16_bits_to_f32(c.k_slots), bits)
    rv, rvs = oracle.quantize_tiles(bf16_bits_to_f32(c.v_slots), bits)
    # the decode consumes exactly the oracle's codes
    assert np.array_equal(unpack_pool(_img(kc), "k", bits, d), rk)
    assert np.array_equal(unpack_pool(_img(vc), "v", bits, d), rv)
    got = dev_to_f64(gpu_decode(c, kp=kc, vp=vc, kv_bits=bits, k_scales=ks, v_scales=vs))
    ref = oracle_decode(c, k_slots=oracle.dequantize(rk, rks), v_slots=oracle.dequantize(rv, rvs))
    assert_close(got, ref, "bf16", f"int{bits}")


@pytest.fixture(scope="module")
def workload4():
    return make_config_case(4)


def _oracle_dequantized(slots, bits, chunk_blocks=1024):
    """float64 values of the oracle's codes for a bf16 slot-form pool. Tiles
    are quantized independently, so chunks of blocks go to the oracle
    separately, on a thread pool (NumPy releases the GIL in these loops)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty(slots.shape, dtype=np.float64)
    step = chunk_blocks * 16

    def one(lo):
        x = bf16_bits_to_f32(slots[lo:lo + step])
        if bits == B.PA_KV_FP8:
            out[lo:lo + step] = oracle.dequantize_fp8(*oracle.quantize_tiles_fp8(x))
        else:
            out[lo:lo + step] = oracle.dequantize(*oracle.quantize_tiles(x, bits))

    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(one, range(0, slots.shape[0], step)))
    return out


@pytest.mark.parametrize("bits", [8, 4, 264])  # 264: fp8 (e4m3)
def test_workload4_quantized_full_batch(lib, workload4, bits):
    """The whole 128 x 8000 batch, in the launch configuration the benchmark
    times, every sequence against the oracle on its own codes."""
    c = workload4
    kc, vc, ks, vs = _quant_case(c, bits)
    got = dev_to_f64(gpu_decode(c, kp=kc, vp=vc, kv_bits=bits, k_scales=ks, v_scales=vs))
    del kc, vc, ks, vs
    kd = _oracle_dequantized(c.k_slots, bits)
    vd = _oracle_dequantized(c.v_slots, bits)
    ref = oracle_decode(c, k_slots=kd, v_slots=vd)
    assert_close(got, ref, "bf16", f"workload4 kv_bits {bits}")


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_quantized_retrieval_probe_exact(lib, bits, d):
    """Codes given directly (scale 1): K zero except a magnet, V encodes
    (slot offset, KV head, block) in digits that fit the code range."""
    qmax = 127 if bits == 8 else 7
    c = make_probe_case(16, 4, d, "bf16", [1, 17, 200, 999, 4100], 405 + d + bits)
    v = oracle.as_f64(c.v_slots, "bf16")
    if bits == 4:  # digits must fit [-7, 7]: re-encode in base 8
        ns = v.shape[0]
        slot = np.arange(ns)
        blk = slot // 16
        v = np.zeros_like(v)
        v[:, :, 0] = ((slot % 16) % 8)[:, None]
        v[:, :, 1] = ((slot % 16) // 8)[:, None]
        v[:, :, 2] = np.arange(c.n_kv)[None, :]
        for j in range(4):
            v[:, :, 3 + j] = ((blk // 8 ** j) % 8)[:, None]
    # digits in the last dim blocks too, so every dim block of a V tile is read back
    v[:, :, d - 1] = ((np.arange(v.shape[0]) % 16) % 8)[:, None]
    v[:, :, d - 17] = np.arange(c.n_kv)[None, :]
    kcode = np.zeros(c.k_slots.shape, dtype=np.int8)
    kq = oracle.as_f64(c.k_slots, "bf16")
    kcode[kq != 0] = qmax
    vcode = v.astype(np.int8)
    nb = c.num_blocks
    kscale = np.full((nb, 4), 40.0 / qmax if bits == 8 else 8.0, dtype=np.float16)
    vscale = np.ones((nb, 4), dtype=np.float16)
    kc = torch.from_numpy(pack_pool(kcode, "k", bits)).cuda()
    vc = torch.from_numpy(pack_pool(vcode, "v", bits)).cuda()
    ks = torch.from_numpy(kscale).cuda()
    vs = torch.from_numpy(vscale).cuda()
    got = gpu_decode(c, kp=kc, vp=vc, kv_bits=bits, k_scales=ks, v_scales=vs).float().cpu().numpy()
    for s in range(c.num_seqs):
        t = int(c.extra["tstar"][s])
        sl = c.block_tables[s, t // 16] * 16 + t % 16
        for h in range(16):
            assert np.array_equal(got[s, h], v[sl, h // 4]), (bits, s, h, got[s, h][:8], v[sl, h // 4][:8])


@pytest.mark.parametrize("tile_bytes,grid,ordered", [(4096, 64, True), (4096, 7, False), (1024, 300, True),
                                                     (16, 3, True), (65536, 5, False)])
def test_hbm_read_probe_reads_every_listed_tile(lib, tile_bytes, grid, ordered):
    """The read probe's per-workgroup XOR equals the XOR of the tiles that
    workgroup is assigned (w, w + grid, ...), so every listed tile is read
    whole; order entries outside the buffer are skipped."""
    g = np.random.default_rng(tile_bytes + grid)
    n_buf = max(8, (1 << 22) // tile_bytes)
    host = g.integers(0, 256, n_buf * tile_bytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    order = None
    tiles = np.arange(n_buf)
    if ordered:
        tiles = np.concatenate([g.permutation(n_buf), [-1, n_buf, n_buf + 7], g.integers(0, n_buf, 50)]).astype(np.int32)
        order = torch.from_numpy(tiles).cuda()
    got = B.hbm_read_probe(buf, tile_bytes, order=order, grid=grid).cpu().numpy().view(np.uint32)
    tile_xor = np.bitwise_xor.reduce(host.view(np.uint32).reshape(n_buf, tile_bytes // 4), axis=1)
    want = np.zeros(grid, dtype=np.uint32)
    for t, tid in enumerate(tiles):
        if 0 <= tid < n_buf:
            want[t % grid] ^= tile_xor[tid]
    assert np.array_equal(got, want)
