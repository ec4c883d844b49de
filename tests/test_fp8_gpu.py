"""GPU: fp8 (OCP e4m3) KV. The quantizer is bit-exact with the oracle (random
tiles, and tiles built on rounding ties, subnormals and saturation); the
decode reads every e4m3 code exactly (a retrieval probe whose retrieved V
rows hold all 254 finite codes) and matches the oracle on exactly
dequantized codes."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_429_amd import binding as B
from synth import make_config_case, make_decode_case, make_probe_case
from synth.gen import bf16_bits_to_f32, f32_to_bf16_bits
from tests.gpu_util import assert_close, dev_to_f64, gpu_decode, np_to_dev, oracle_decode, upload_meta, upload_pools
from tests.layout_ref import pack_pool, unpack_pool

pytestmark = pytest.mark.gpu
FP8 = B.PA_KV_FP8


def _img(t):
    return t.cpu().numpy().view(np.uint8)


def _codes(pool, kind, d):
    return unpack_pool(_img(pool), kind, 8, d).view(np.uint8)


@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("d", [64, 128])
def test_quantize_fp8_bitexact(lib, kind, d):
    c = make_decode_case(8, 4, d, "bf16", [300, 77], 9000 + d, pool_factor=1.5)
    kp, vp = upload_pools(c)
    src, slots = (kp, c.k_slots) if kind == "k" else (vp, c.v_slots)
    codes, scales = B.quantize(src, bits=FP8, kind=0 if kind == "k" else 1, n_kv_heads=4, d_head=d)
    torch.cuda.synchronize()
    ref_codes, ref_scales = oracle.quantize_tiles_fp8(bf16_bits_to_f32(slots))
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), ref_scales.view(np.uint16))
    assert np.array_equal(_codes(codes, kind, d), ref_codes)
    assert np.array_equal(_img(codes), pack_pool(ref_codes.view(np.int8), kind, 8))


def test_quantize_fp8_ties_subnormals_saturation(lib):
    """A tile whose largest magnitude is 448 has scale 1, so its other values
    are rounded as they stand: exact midpoints between e4m3 values (ties go
    to the even code), subnormal multiples of 2^-9 and their midpoints,
    signed zeros and tiny negatives. Other tiles: all zero (scale 0) and one
    whose fp16 scale overflows."""
    n_kv, d = 2, 64
    c = make_decode_case(4, n_kv, d, "bf16", [48], 9010, pool_factor=1.0)
    special = np.array([1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -9, 3 * 2.0 ** -10, 5 * 2.0 ** -10, 432.0,
                        440.0, 416.0, 424.0, -0.0, -2.0 ** -12, -1.0625, 2.0 ** -7 * 1.0625, 96.0 + 8.0,
                        0.0, 2.0 ** -6, 2.0 ** -6 * 1.0625, -432.0, 7.5 * 2.0 ** -9], np.float32)
    x = bf16_bits_to_f32(c.k_slots).copy()
    g = np.random.default_rng(1)
    x[0:16] = bf16_bits_to_f32(f32_to_bf16_bits((g.standard_normal((16, n_kv, d)) * 50).astype(np.float32)))
    x[0, 0, 0] = 448.0
    x[1, 0, :special.size] = special
    x[0, 1, 0] = -448.0
    x[2, 1, :special.size] = -special
    x[16:32] = 0.0                       # zero tile: scale 0
    x[32:48] = 1.0
    x[40, 0, 3] = 2.0 ** 25              # 2^25 / 448 > 65504: the fp16 scale overflows in head 0
    bits = f32_to_bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(bits), x)  # every value is a bf16 value
    c.k_slots[:] = bits
    kp, _ = upload_pools(c)
    codes, scales = B.quantize(kp, bits=FP8, kind=0, n_kv_heads=n_kv, d_head=d)
    torch.cuda.synchronize()
    ref_codes, ref_scales = oracle.quantize_tiles_fp8(x)
    assert float(ref_scales[0, 0]) == 1.0 and ref_scales[1, 0] == 0 and np.isinf(ref_scales[2, 0])
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), ref_scales.view(np.uint16))
    assert np.array_equal(_codes(codes, "k", d), ref_codes)
    assert ref_codes[1, 0, :special.size].tolist()[:6] == [0x38, 0x3A, 0x00, 0x02, 0x02, 0x02]


def _fp8_case(c):
    kp, vp = upload_pools(c)
    kc, ks = B.quantize(kp, bits=FP8, kind=0, n_kv_heads=c.n_kv, d_head=c.d)
    vc, vs = B.quantize(vp, bits=FP8, kind=1, n_kv_heads=c.n_kv, d_head=c.d)
    del kp, vp
    return kc, vc, ks, vs


@pytest.mark.parametrize("n_heads,n_kv,d", [(64, 8, 128), (32, 8, 64), (8, 8, 128), (12, 4, 128)])
def test_fp8_decode_parity(lib, n_heads, n_kv, d):
    c = make_decode_case(n_heads, n_kv, d, "bf16", [8000, 1, 17, 4000, 515, 8000, 2222, 33], 9020 + n_heads + d,
                         pool_factor=1.1)
    kc, vc, ks, vs = _fp8_case(c)
    rk, rks = oracle.quantize_tiles_fp8(bf16_bits_to_f32(c.k_slots))
    rv, rvs = oracle.quantize_tiles_fp8(bf16_bits_to_f32(c.v_slots))
    assert np.array_equal(_codes(kc, "k", d), rk)
    assert np.array_equal(_codes(vc, "v", d), rv)
    got = dev_to_f64(gpu_decode(c, kp=kc, vp=vc, kv_bits=FP8, k_scales=ks, v_scales=vs))
    ref = oracle_decode(c, k_slots=oracle.dequantize_fp8(rk, rks), v_slots=oracle.dequantize_fp8(rv, rvs))
    assert_close(got, ref, "bf16", "fp8")


@pytest.mark.parametrize("pb", [0, 2, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_retrieval_probe_all_codes_exact(lib, pb, d):
    """K codes are 0 except a magnet (code 0x7E at scale 40/448); V scale 1
    and V row (slot, head) holds code (i + 128 * ((slot + head) % 2)) % 256 at
    dim i (NaN codes replaced by 0), so the retrieved rows cover every finite
    code. The output must be e4m3(code) exactly, dim by dim."""
    c = make_probe_case(16, 4, d, "bf16", [1, 17, 200, 999, 4100, 33, 64, 1500], 9030 + d + pb)
    ns = c.k_slots.shape[0]
    slot = np.arange(ns)[:, None, None]
    head = np.arange(c.n_kv)[None, :, None]
    dim = np.arange(d)[None, None, :]
    vcode = ((dim + (128 if d == 128 else 64) * ((slot + head) % 2)) % 256).astype(np.uint8)
    if d == 64:  # 64 dims per row: four row classes cover the 256 codes
        vcode = ((dim + 64 * ((slot + head) % 4)) % 256).astype(np.uint8)
    vcode[(vcode & 0x7F) == 0x7F] = 0
    kq = oracle.as_f64(c.k_slots, "bf16")
    kcode = np.where(kq != 0, 0x7E, 0).astype(np.uint8)
    nb = c.num_blocks
    ks = torch.from_numpy(np.full((nb, c.n_kv), 40.0 / 448.0, dtype=np.float16)).cuda()
    vs = torch.from_numpy(np.ones((nb, c.n_kv), dtype=np.float16)).cuda()
    kc = torch.from_numpy(pack_pool(kcode.view(np.int8), "k", 8)).cuda()
    vc = torch.from_numpy(pack_pool(vcode.view(np.int8), "v", 8)).cuda()
    got = gpu_decode(c, kp=kc, vp=vc, kv_bits=FP8, k_scales=ks, v_scales=vs,
                     partition_blocks=pb).float().cpu().numpy()
    vals = oracle.e4m3_value(vcode)
    seen = set()
    for s in range(c.num_seqs):
        t = int(c.extra["tstar"][s])
        sl = c.block_tables[s, t // 16] * 16 + t % 16
        for h in range(16):
            assert np.array_equal(got[s, h], vals[sl, h // 4]), (s, h, got[s, h][:8], vals[sl, h // 4][:8])
            seen.update(vcode[sl, h // 4].tolist())
    assert len(seen) >= 200


def test_fp8_prefill_matches_decode(lib):
    """fp8 pools in the prefill: a one-token chunk per sequence equals the
    decode of the same query on the same codes (the whole 128 x 8000 batch is
    checked against the oracle in test_kvops_gpu.py; chunk parity in
    test_prefill_gpu.py)."""
    c = make_decode_case(8, 2, 128, "bf16", [40, 333, 17], 9040, pool_factor=1.2)
    kc, vc, ks, vs = _fp8_case(c)
    tables, ctx = upload_meta(c)
    q = np_to_dev(c.q, "bf16")
    cu = torch.arange(c.num_seqs + 1, dtype=torch.int32, device="cuda")
    pre = B.prefill_chunk(q, cu, kc, vc, tables, ctx, n_kv_heads=2, max_q_len=1, max_context_len=333, kv_bits=FP8,
                          k_scales=ks, v_scales=vs)
    dec = gpu_decode(c, kp=kc, vp=vc, kv_bits=FP8, k_scales=ks, v_scales=vs)
    assert_close(dev_to_f64(pre), dev_to_f64(dec), "bf16", "fp8 q_len 1 vs decode")
