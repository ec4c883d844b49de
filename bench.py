"""Benchmark: paged decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2|3|4a|4b|4f|5d|5p|5|append]
                    [--kv-bits 16|8|4|264] [--no-cpu-baseline]

A step is one paged_attn_decode call (all G query heads of every KV head,
every sequence of the batch, split-context merge included) over one layer's
cache. The default workload is the Llama-3-8B-shaped bf16 decode layer (32
query / 8 KV heads, d 128, 64 sequences with context U[512, 4096], seed
4292). Inputs are seeded synthetic N(0,1) data written into device pools
before timing; steps cycle through several identical copies of the layer's
pools (as a model's layers would) so that consecutive steps do not re-read
the same memory from the last-level cache.

Timing: after the warm-up, K steps run back to back; the wall clock around
them gives the line's value, and HIP events recorded on the launch stream
at the start and end of the same timed region give the kernel time of the
roofline (their span / K, launch gaps between the steps included). The
default line (workload 2) also times the other two bf16 decode workloads,
the 70B-class prefix-shared layer and the mixed step's decode half, the
same way, under "other_bf16_decode".

The line also carries the device's measured read ceiling (the library's
read probe: random 4 KiB tiles, and a stream) and the decode's fraction of
it, beside the fraction of the 8 TB/s spec peak.

The line printed carries the achieved HBM bandwidth over algorithmic bytes
(K/V of every attended token once per KV head, plus Q, O, the table entries
and lengths read), the decode tokens/s per layer, a roofline object for the
decode kernel (HIP-event time on the launch stream) and the CPU oracle's
throughput on the host (a bounded sample of the same workload).
"""
import argparse
import json
import os
import sys
import time

# thread counts for the CPU oracle's BLAS, fixed before numpy loads
try:
    _CORES = len(os.sched_getaffinity(0))
except AttributeError:  # pragma: no cover
    _CORES = os.cpu_count() or 1
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(_CORES))

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (% of peak) and decode tokens/s per layer"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# counter summaries under profiles/ (name of the kernel and workload)
PROFILE_NAME = {"2": "decode_kernel_llama3_8b_bf16", "3": "prefix_pass_and_decode_kernel_prefix_shared_70b_bf16",
                "4a": "decode_kernel_quant_kv_70b_int8", "4b": "decode_kernel_quant_kv_70b_int4",
                "4f": "decode_kernel_quant_kv_70b_fp8",
                "5d": "decode_kernel_mixed_step_decode_bf16", "5p": "prefill_tile_kernel_chunk2048_ctx6000_bf16"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="2")
    ap.add_argument("--layers", type=int, default=4, help="copies of the layer's pools cycled through")
    ap.add_argument("--partition-blocks", type=int, default=0)
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window in tokens for the decode workloads (0: full attention)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="workload 2 only: skip timing the other bf16 decode workloads (70B prefix-shared, "
                         "mixed-step decode half) beside it")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip measuring the device's read ceiling (random 4 KiB tiles and a stream)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--kv-bits", type=int, default=16,
                    help="pool format of the append workload: 16 (bf16), 8, 4 or 264 (fp8 e4m3)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many MiB (calibrates "
                         "the HBM byte counters) and print its size and time")
    return ap.parse_args()


def copy_probe(mib, reps):
    """A plain device-to-device copy of a known size: FETCH_SIZE / WRITE_SIZE
    read on it give the factor between those counters and real bytes."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        t.append((a, b))
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in t]))
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "reps": reps,
                      "median_ms": round(ms, 4), "copy_GBps": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def kernel_source_hash():
    """sha256 (first 16 hex digits) of the library's kernel sources, the key
    under which profiles/*.hbm.md records counter-measured traffic."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "paged_kv_cache_429_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(profile):
    """HBM bytes per launch from a committed counter summary (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy calibration), or None when the summary is
    missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", profile + ".hbm.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_hash"):
                k, v = line.split(":", 1)
                vals[k] = v.strip()
    if vals.get("source_hash") != kernel_source_hash() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(vals["traffic_bytes_per_launch"])


PA_KV_FP8 = 264  # kv_bits code of fp8 (e4m3) pools in the library's ABI


def storage_bits(kv_bits):
    return 8 if kv_bits == PA_KV_FP8 else kv_bits


def read_ceiling(torch, B, gib=4, reps=10, decode_bytes=0):
    """The device's measured read bandwidth on the decode's access pattern:
    the library's read probe over a `gib` GiB buffer, once as 4 KiB tiles in
    a random order (one (block, KV head) bf16 tile at d_head 128) and once as
    a stream; GB/s from HIP events around `reps` passes after two warm-ups.
    With decode_bytes, also random tiles over a buffer of the decode step's
    own byte count at a few grid sizes (a small grid leaves CUs idle at the
    end of a pass, as a decode launch of that many workgroups does)."""
    tile = 4096
    n = (gib << 30) // tile
    buf = torch.empty(n * tile, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    g = torch.Generator(device="cpu").manual_seed(4290)
    order = torch.randperm(n, generator=g).to(torch.int32).cuda()
    grid = 16384  # many more workgroups than resident slots: no idle CUs at the end of a pass
    xo = torch.empty(grid, dtype=torch.int32, device="cuda")
    out = {}
    for name, o in (("random_4k_tiles_GBps", order), ("stream_GBps", None)):
        for _ in range(2):
            B.hbm_read_probe(buf, tile, order=o, grid=grid, xor_out=xo)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            B.hbm_read_probe(buf, tile, order=o, grid=grid, xor_out=xo)
        e.record()
        torch.cuda.synchronize()
        out[name] = round(n * tile * reps / (s.elapsed_time(e) * 1e-3) / 1e9, 1)
    del buf, order
    out.update({"buffer_bytes": n * tile, "reps": reps, "loads": "16-byte nontemporal", "workgroups": grid})
    if decode_bytes:
        n = max(1, int(decode_bytes) // tile)
        buf = torch.empty(n * tile, dtype=torch.uint8, device="cuda")
        buf.fill_(1)
        order = torch.randperm(n, generator=g).to(torch.int32).cuda()
        by_grid = {}
        for grid in (768, 1536, 16384):
            xo = torch.empty(grid, dtype=torch.int32, device="cuda")
            for _ in range(2):
                B.hbm_read_probe(buf, tile, order=order, grid=grid, xor_out=xo)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(2 * reps):
                B.hbm_read_probe(buf, tile, order=order, grid=grid, xor_out=xo)
            e.record()
            torch.cuda.synchronize()
            by_grid[str(grid)] = round(n * tile * 2 * reps / (s.elapsed_time(e) * 1e-3) / 1e9, 1)
        del buf, order
        out["decode_bytes_random_4k_tiles_GBps_by_workgroups"] = by_grid
        out["decode_bytes_buffer"] = n * tile
    return out


def decode_bytes(case, kv_bits, window=0):
    """Algorithmic bytes of one decode step: every attended token's K and V
    once per KV head (shared blocks once), scales, Q, O, table entries, lengths.
    With a sliding window only the last `window` tokens of each sequence are
    attended, and only the blocks holding them are looked up."""
    n_kv, d = case.n_kv, case.d
    ctx = case.context_lens.astype(np.int64)
    nblk = -(-ctx // 16)
    if window:
        first_blk = np.maximum(ctx - window, 0) // 16
        tokens = int(np.minimum(ctx, window).sum())
        blocks = int((nblk - first_blk).sum())
        nblk = nblk - first_blk
    elif case.shared_prefix_blocks:
        P = case.shared_prefix_blocks
        tokens = P * 16 + int(np.sum(ctx - P * 16))
        blocks = P + int(np.sum(nblk - P))
    else:
        tokens = int(ctx.sum())
        blocks = int(nblk.sum())
    elem = 2 if case.dtype == "bf16" else 4
    kv = tokens * n_kv * d * 2 * storage_bits(kv_bits) / 8
    scales = blocks * n_kv * 2 * 2 if storage_bits(kv_bits) < 16 else 0
    qo = 2 * case.num_seqs * case.n_heads * d * elem
    meta = int(nblk.sum()) * 4 + case.num_seqs * 4
    return kv + scales + qo + meta


def build_case(workload):
    from synth import make_config_case, make_mixed_case
    if workload in ("2", "3"):
        return make_config_case(int(workload)), 16
    if workload in ("4a", "4b", "4f"):
        return make_config_case(4), {"4a": 8, "4b": 4, "4f": PA_KV_FP8}[workload]
    if workload == "5d":
        return make_mixed_case()[1], 16
    raise SystemExit(f"unknown workload {workload}")


def to_dev(x, dtype, torch):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def cpu_baseline(case, kv_bits, budget_s, window=0):
    """The oracle, as it stands, on whole sequences of the same workload until
    about `budget_s` seconds of host time; throughput in the metric's unit.
    Decoding the pools to float64 (and quantizing them, for int KV) is
    preparation and is not timed; gather + attention are."""
    import oracle
    q = oracle.as_f64(case.q, case.dtype)
    if kv_bits == PA_KV_FP8:
        kc, ksc = oracle.quantize_tiles_fp8(oracle.as_f64(case.k_slots, case.dtype).astype(np.float32))
        vc, vsc = oracle.quantize_tiles_fp8(oracle.as_f64(case.v_slots, case.dtype).astype(np.float32))
        kf, vf = oracle.dequantize_fp8(kc, ksc), oracle.dequantize_fp8(vc, vsc)
        del kc, vc
    elif kv_bits < 16:
        kc, ksc = oracle.quantize_tiles(oracle.as_f64(case.k_slots, case.dtype).astype(np.float32), kv_bits)
        vc, vsc = oracle.quantize_tiles(oracle.as_f64(case.v_slots, case.dtype).astype(np.float32), kv_bits)
        kf, vf = oracle.dequantize(kc, ksc), oracle.dequantize(vc, vsc)
        del kc, vc
    else:
        kf, vf = oracle.as_f64(case.k_slots, case.dtype), oracle.as_f64(case.v_slots, case.dtype)
    order = np.random.default_rng(0).permutation(case.num_seqs)
    done = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 <= budget_s:  # whole sequences, repeating the batch if it is short
        s = int(order[len(done) % len(order)])
        oracle.paged_decode(q, kf, vf, case.block_tables, case.context_lens, n_kv=case.n_kv, seqs=[s],
                            window=window or None)
        done.append(s)
    el = time.perf_counter() - t0
    sub = case.context_lens[done].astype(np.int64)
    if window:
        sub = np.minimum(sub, window)
    per_tok = case.n_kv * case.d * 2 * storage_bits(kv_bits) / 8
    elem = 2 if case.dtype == "bf16" else 4
    byts = float(sub.sum()) * per_tok + 2 * len(done) * case.n_heads * case.d * elem
    return {
        "value": round(byts / el / 1e9, 4),
        "unit": "GB/s",
        "cores": _CORES,
        "kind": "oracle",
        "sample": (f"{len(done)} sequence decodes drawn from the {case.num_seqs}-sequence batch "
                   f"({int(sub.sum())} attended tokens) in {el:.1f} s; float64 NumPy, all heads"),
        "seqs_per_s": round(len(done) / el, 3),
    }


def prefill_flops(c):
    """4 d flops (Q.K and P.V) per (query head, visible key) pair of the chunk."""
    total = 0
    for s in range(c.num_seqs):
        qlen = int(c.cu_q_lens[s + 1] - c.cu_q_lens[s])
        n = int(c.context_lens[s])
        pos = n - qlen + np.arange(qlen, dtype=np.int64)
        total += int((pos + 1).sum())
    return 4 * c.d * c.n_heads * total


def prefill_cpu_baseline(c, budget_s):
    """The oracle on chunk rows spread over the chunk (whole rows, all heads)
    until about `budget_s` seconds; GFLOP/s over the same flop count."""
    import oracle
    q = oracle.as_f64(c.q, c.dtype)
    kf, vf = oracle.as_f64(c.k_slots, c.dtype), oracle.as_f64(c.v_slots, c.dtype)
    qlen = int(c.cu_q_lens[1] - c.cu_q_lens[0])
    order = np.random.default_rng(0).permutation(qlen)
    done = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 <= budget_s and len(done) < qlen:
        r = [int(x) for x in order[len(done):len(done) + 16]]
        oracle.paged_prefill(q, c.cu_q_lens, kf, vf, c.block_tables, c.context_lens, n_kv=c.n_kv, rows=r)
        done.extend(r)
    el = time.perf_counter() - t0
    pos = int(c.context_lens[0]) - qlen + np.asarray(done, dtype=np.int64)
    fl = 4 * c.d * c.n_heads * int((pos + 1).sum())
    return {"value": round(fl / el / 1e9, 3), "unit": "GFLOP/s", "cores": _CORES, "kind": "oracle",
            "sample": f"{len(done)} of {qlen} chunk rows (all heads, causal) in {el:.1f} s; float64 NumPy"}


def prefill_main(a, torch, B, CONFIGS):
    """Workload 5: the 2048-token causal chunk over 6000 cached tokens alone
    ('5p'), or the whole mixed step ('5': the chunk on one stream and the 64
    decodes concurrently on a second, both bracketed by events on the
    first)."""
    from synth import make_mixed_case
    pre, dec = make_mixed_case()
    kp = B.alloc_pool(pre.num_blocks, pre.n_kv, pre.d, 16)
    vp = B.alloc_pool(pre.num_blocks, pre.n_kv, pre.d, 16)
    slots = torch.arange(pre.num_blocks * 16, dtype=torch.int64, device="cuda")
    B.kv_write(to_dev(pre.k_slots, "bf16", torch), to_dev(pre.v_slots, "bf16", torch), slots, kp, vp,
               n_kv_heads=pre.n_kv)
    qp = to_dev(pre.q, "bf16", torch)
    cu = torch.from_numpy(pre.cu_q_lens.astype(np.int32)).cuda()
    tp = torch.from_numpy(np.ascontiguousarray(pre.block_tables)).cuda()
    cp = torch.from_numpy(pre.context_lens.astype(np.int32)).cuda()
    op = torch.empty_like(qp)
    qd = to_dev(dec.q, "bf16", torch)
    td = torch.from_numpy(np.ascontiguousarray(dec.block_tables)).cuda()
    cd = torch.from_numpy(dec.context_lens.astype(np.int32)).cuda()
    od = torch.empty_like(qd)
    mixed = a.workload == "5"
    s_main = torch.cuda.current_stream()
    s_dec = torch.cuda.Stream() if mixed else None
    ws = B.decode_workspace(dec.num_seqs, dec.n_heads, dec.n_kv, dec.d, dec.max_context_len, 0,
                            stream=s_dec) if mixed else None
    torch.cuda.synchronize()

    def step():
        # mixed: the chunk and the decodes of one step run concurrently on two
        # streams (they only read the pools); a step starts once the previous
        # one (and the start event on the main stream) is done, and the main
        # stream joins the decode stream before the step's end
        if mixed:
            s_dec.wait_stream(s_main)
        B.prefill_chunk(qp, cu, kp, vp, tp, cp, n_kv_heads=pre.n_kv, max_q_len=pre.max_q_len,
                        max_context_len=pre.max_context_len, out=op, stream=s_main)
        if mixed:
            B.decode(qd, kp, vp, td, cd, n_kv_heads=dec.n_kv, max_context_len=dec.max_context_len, out=od,
                     workspace=ws, stream=s_dec)
            s_main.wait_stream(s_dec)

    def timed(n):
        # n steps back to back: the wall clock around them, and HIP events on
        # the main stream at the start and end of the same region
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(s_main)
        for _ in range(n):
            step()
        e1.record(s_main)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1)

    for _ in range(a.warmup):
        step()
    wall, ev_ms = timed(a.steps)
    flops = prefill_flops(pre)
    k_avg = ev_ms / a.steps
    ms_step = wall * 1e3 / a.steps
    res = {
        "metric": "causal chunked-prefill attention: achieved MFMA TFLOP/s (% of bf16 dense peak)"
                  if not mixed else "mixed chunked-prefill step: step time, prefill TFLOP/s and decode GB/s",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2) if not mixed else round(ms_step * 1e3, 2),
        "unit": "TFLOP/s" if not mixed else "us per step",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": not mixed, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": CONFIGS[5]["workload"] + (" [prefill chunk]" if not mixed else " [whole step]"),
                   "chunk_tokens": pre.max_q_len, "context_tokens": int(pre.context_lens[0]),
                   "n_heads": pre.n_heads, "n_kv_heads": pre.n_kv, "d_head": pre.d, "seed": pre.seed,
                   "decode_seqs": dec.num_seqs if mixed else 0},
        "flops_per_step": flops,
        "roofline": {"bound": "mfma", "kernel": "prefill_tile_kernel" if not mixed else "prefill_tile_kernel+decode_kernel",
                     "achieved": round(flops / (k_avg * 1e-3) / 1e12, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flops / (k_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None if mixed else measured_traffic(PROFILE_NAME["5p"]),
                     "kernel_avg_us": round(k_avg * 1e3, 3)},
    }
    if mixed:
        res["decode_algorithmic_bytes"] = int(decode_bytes(dec, 16))
        res["decode_tokens_per_s"] = round(dec.num_seqs / (ms_step * 1e-3), 1)
        res["prefill_tokens_per_s"] = round(pre.max_q_len / (ms_step * 1e-3), 1)
    if not a.no_cpu_baseline and not mixed:
        res["cpu_baseline"] = prefill_cpu_baseline(pre, a.cpu_seconds)
    print(json.dumps(res), flush=True)


def append_main(a, torch, B, CONFIGS):
    """Workload 'append': paged_kv_append writing every token of the
    Llama-3-8B-shaped layer's 64 sequences (contexts U[512, 4096]) into an
    empty pool in one call, as a prompt prefill would, through the block
    table; for quantized pools (--kv-bits 8, 4, 264) the blocks are quantized
    on write. Algorithmic bytes: the new K and V rows read, the pool bytes of
    their tokens written, and for quantized pools the scales written and the
    staging tiles of the partly filled last blocks written. One decode
    step's append (one token per sequence, rewriting each sequence's last
    position; timing only) is timed beside it."""
    from synth import make_config_case
    c = make_config_case(2)
    bits = a.kv_bits
    quant = bits in (8, 4, PA_KV_FP8)
    S, nkv, d = c.num_seqs, c.n_kv, c.d
    ctx = c.context_lens.astype(np.int64)
    tokens = int(ctx.sum())
    g = torch.Generator(device="cuda").manual_seed(4292)
    kn = torch.randn((tokens, nkv, d), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((tokens, nkv, d), generator=g, device="cuda").to(torch.bfloat16)
    kp = B.alloc_pool(c.num_blocks, nkv, d, bits)
    vp = B.alloc_pool(c.num_blocks, nkv, d, bits)
    ks = vs = kst = vst = None
    if quant:
        ks, vs = B.alloc_scales(c.num_blocks, nkv), B.alloc_scales(c.num_blocks, nkv)
        kst = torch.zeros((S, nkv, 16, d), dtype=torch.bfloat16, device="cuda")
        vst = torch.zeros_like(kst)
    tables = torch.from_numpy(np.ascontiguousarray(c.block_tables)).cuda()
    lens = torch.from_numpy(ctx.astype(np.int32)).cuda()
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)).cuda()
    cu1 = torch.arange(S + 1, dtype=torch.int32, device="cuda")
    k1, v1 = kn[:S].contiguous(), vn[:S].contiguous()

    def fill():
        B.kv_append(kn, vn, cu, tables, lens, kp, vp, n_kv_heads=nkv, max_new=int(ctx.max()), kv_bits=bits,
                    k_scales=ks, v_scales=vs, k_stage=kst, v_stage=vst)

    def one_token():
        B.kv_append(k1, v1, cu1, tables, lens, kp, vp, n_kv_heads=nkv, max_new=1, kv_bits=bits,
                    k_scales=ks, v_scales=vs, k_stage=kst, v_stage=vst)

    def timed(fn, n):
        # n calls back to back: the wall clock around them, and HIP events on
        # the stream at the start and end of the same region (ms per call)
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) / n

    for _ in range(a.warmup):
        fill()
        one_token()
    wall, k_avg = timed(fill, a.steps)
    _, step_ms = timed(one_token, a.steps)
    sb = storage_bits(bits)
    partial = int((ctx % 16 != 0).sum())
    byts = 2 * tokens * nkv * d * 2 + 2 * tokens * nkv * d * sb // 8
    if quant:
        byts += 2 * int((-(-ctx // 16)).sum()) * nkv * 2 + 2 * partial * nkv * 16 * d * 2
    ms = wall * 1e3 / a.steps
    res = {
        "metric": "paged KV append (whole contexts through the block table): achieved HBM GB/s",
        "value": round(byts / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": {16: "bf16", 8: "bf16 -> int8", 4: "bf16 -> int4", PA_KV_FP8: "bf16 -> fp8 e4m3"}[bits],
        "data": "synthetic",
        "config": {"workload": CONFIGS[2]["workload"] + " [append of every context token in one call]",
                   "tokens": tokens, "num_seqs": S, "n_kv_heads": nkv, "d_head": d, "kv_bits": bits},
        "algorithmic_bytes_per_step": int(byts),
        "roofline": {"bound": "hbm", "kernel": "kv_append_kernel", "achieved": round(byts / (k_avg * 1e-3) / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(byts / (k_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel_avg_us": round(k_avg * 1e3, 3)},
        "decode_step_append_us": round(step_ms * 1e3, 2),
    }
    print(json.dumps(res), flush=True)


def measure_decode(torch, B, case, kv_bits, steps, warmup, n_layers, partition_blocks=0, window=0):
    """Device pools for the case (one copy written by paged_kv_write,
    quantized if asked, replicated for n_layers layers that the steps cycle
    through), then `warmup` steps and `steps` timed steps back to back.
    Returns (wall seconds of the timed steps, milliseconds between HIP events
    recorded on the launch stream at the start and end of the same timed
    region)."""
    src_bits = 32 if case.dtype == "f32" else 16
    kp = B.alloc_pool(case.num_blocks, case.n_kv, case.d, src_bits)
    vp = B.alloc_pool(case.num_blocks, case.n_kv, case.d, src_bits)
    slots = torch.arange(case.num_blocks * 16, dtype=torch.int64, device="cuda")
    B.kv_write(to_dev(case.k_slots, case.dtype, torch), to_dev(case.v_slots, case.dtype, torch), slots, kp, vp,
               n_kv_heads=case.n_kv)
    ks = vs = None
    if storage_bits(kv_bits) < 16:
        kp, ks = B.quantize(kp, bits=kv_bits, kind=0, n_kv_heads=case.n_kv, d_head=case.d)
        vp, vs = B.quantize(vp, bits=kv_bits, kind=1, n_kv_heads=case.n_kv, d_head=case.d)
    layers = [(kp, vp, ks, vs)]
    for _ in range(n_layers - 1):
        layers.append(tuple(None if t is None else t.clone() for t in (kp, vp, ks, vs)))
    q = to_dev(case.q, case.dtype, torch)
    tables = torch.from_numpy(np.ascontiguousarray(case.block_tables)).cuda()
    ctx = torch.from_numpy(np.ascontiguousarray(case.context_lens)).cuda()
    out = torch.empty_like(q)
    mcl = case.max_context_len
    ws = B.decode_workspace(case.num_seqs, case.n_heads, case.n_kv, case.d, mcl, partition_blocks)
    torch.cuda.synchronize()

    def step(i):
        k_, v_, ks_, vs_ = layers[i % len(layers)]
        B.decode(q, k_, v_, tables, ctx, n_kv_heads=case.n_kv, max_context_len=mcl, kv_bits=kv_bits,
                 k_scales=ks_, v_scales=vs_, out=out, workspace=ws, partition_blocks=partition_blocks,
                 window=window or None)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = t_start.elapsed_time(t_end)
    del layers, kp, vp, ks, vs, ws
    return wall, ev_ms


def extra_decode_configs(torch, B, steps, warmup, n_layers):
    """The other bf16 decode workloads, timed the same way: the 70B-class
    prefix-shared layer and the decode half of the mixed step."""
    out = {}
    for wl, key in (("3", "prefix_shared_70b_bf16"), ("5d", "mixed_step_decode_bf16")):
        case, kv_bits = build_case(wl)
        wall, ev_ms = measure_decode(torch, B, case, kv_bits, steps, warmup, n_layers)
        byts = decode_bytes(case, kv_bits)
        k_us = ev_ms * 1e3 / steps
        out[key] = {"workload": wl, "us_per_step": round(wall * 1e6 / steps, 3), "kernel_avg_us": round(k_us, 3),
                    "GBps": round(byts / (k_us * 1e-6) / 1e9, 2),
                    "frac": round(byts / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "tokens_per_s_per_layer": round(case.num_seqs / (wall / steps), 1),
                    "algorithmic_bytes_per_step": int(byts)}
        del case
        torch.cuda.empty_cache()
    return out


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    from paged_kv_cache_429_amd import binding as B
    from synth import CONFIGS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if a.copy_probe_mib:
        copy_probe(a.copy_probe_mib, max(1, a.steps))
        return
    if a.workload in ("5", "5p"):
        prefill_main(a, torch, B, CONFIGS)
        return
    if a.workload == "append":
        append_main(a, torch, B, CONFIGS)
        return
    t_gen = time.perf_counter()
    case, kv_bits = build_case(a.workload)
    gen_s = time.perf_counter() - t_gen
    wall, ev_ms = measure_decode(torch, B, case, kv_bits, a.steps, a.warmup, a.layers, a.partition_blocks, a.window)
    mcl = case.max_context_len
    byts = decode_bytes(case, kv_bits, a.window)
    ms_step = wall * 1e3 / a.steps
    value = byts / (ms_step * 1e-3) / 1e9
    k_avg = ev_ms / a.steps
    achieved = byts / (k_avg * 1e-3) / 1e9
    name = {"2": 2, "3": 3, "4a": 4, "4b": 4, "4f": 4, "5d": 5}[a.workload]
    wl = CONFIGS[name]["workload"] + ({"4a": " [int8]", "4b": " [int4]", "4f": " [fp8 e4m3]",
                                       "5d": " [decode half]"}.get(a.workload, ""))
    if a.window:
        wl += f" [sliding window {a.window}]"
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {32: "f32", 16: "bf16", 8: "bf16 q / int8 kv", 4: "bf16 q / int4 kv",
                  PA_KV_FP8: "bf16 q / fp8 e4m3 kv"}[kv_bits],
        "data": "synthetic",
        "config": {
            "workload": wl,
            "num_seqs": case.num_seqs, "n_heads": case.n_heads, "n_kv_heads": case.n_kv, "d_head": case.d,
            "block_size": 16, "kv_bits": kv_bits, "total_context_tokens": int(case.context_lens.sum()),
            "max_context_len": mcl, "seed": case.seed, "layers_cycled": a.layers, "window": a.window,
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s_per_layer": round(case.num_seqs / (ms_step * 1e-3), 1),
        "algorithmic_bytes_per_step": int(byts),
        "roofline": {
            "bound": "hbm",
            # the prefix-shared batch runs the prefix pass (a launch of the
            # tile kernel over each tile's common run) before the decode; the
            # events span both launches of the call
            "kernel": "decode_kernel" if a.workload != "3" else "prefill_tile_kernel<prefix pass>+decode_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(PROFILE_NAME[a.workload] + (f"_window{a.window}" if a.window else "")),
            # HIP events on the launch stream at the start and end of the
            # timed region: its K back-to-back steps, launch gaps included
            "kernel_avg_us": round(k_avg * 1e3, 3),
            "kernel_time": "events around the timed region / steps",
        },
        "input_generation_s": round(gen_s, 2),
    }
    if a.workload == "2" and not a.window and not a.no_extra:
        # the other bf16 decode workloads, so one default run times all three
        res["other_bf16_decode"] = extra_decode_configs(torch, B, a.steps, a.warmup, a.layers)
    if not a.no_read_probe:
        # the same box's measured read ceiling, beside the spec peak
        rc = read_ceiling(torch, B, decode_bytes=byts)
        res["measured_read"] = rc
        res["roofline"]["frac_of_measured_random_tiles"] = round(achieved / rc["random_4k_tiles_GBps"], 4)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, kv_bits, a.cpu_seconds, a.window)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
