"""Seeded synthetic inputs: queries, paged K/V pools, block tables, lengths.

Every array is drawn from numpy's PCG64 through SeedSequence children, so a
case is a pure function of its seed. Large N(0, 1) pools are generated in
fixed-size chunks, one child stream per chunk, on a thread pool; the result
does not depend on the number of threads.

Pools are handed out in *slot* form: ``k_slots[b * 16 + o, h, :]`` is the key
of slot ``o`` of physical block ``b`` for KV head ``h``. That is the logical
content of the cache; how the library lays a block out in device memory is the
library's business (it is written there by ``paged_kv_write``).

bfloat16 values are carried as uint16 bit patterns (numpy has no bfloat16).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

from .configs import BLOCK_SIZE, CONFIGS, config_seed

_CHUNK = 1 << 22


def _workers(n_chunks: int) -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(8, cores, n_chunks))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); NaN -> 0x7FC0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(ss: np.random.SeedSequence, n: int, dtype: str) -> np.ndarray:
    """n N(0,1) draws as float32 ('f32') or bfloat16 bits ('bf16')."""
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    if n == 0:
        return out
    n_chunks = -(-n // _CHUNK)
    kids = ss.spawn(n_chunks)

    def fill(i: int) -> None:
        lo = i * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        if dtype == "f32":
            g.standard_normal(out=out[lo:hi], dtype=np.float32)
        else:
            tmp = np.empty(hi - lo, dtype=np.float32)
            g.standard_normal(out=tmp, dtype=np.float32)
            out[lo:hi] = f32_to_bf16_bits(tmp)

    w = _workers(n_chunks)
    if w == 1:
        for i in range(n_chunks):
            fill(i)
    else:
        with ThreadPoolExecutor(w) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


@dataclass
class DecodeCase:
    """One batch of single-query (decode) attention over a paged cache.

    q            [num_seqs, n_heads, d]          float32 or bf16 bits
    k_slots      [num_blocks * 16, n_kv, d]      float32 or bf16 bits
    v_slots      same as k_slots
    block_tables [num_seqs, max_blocks] int32; entries >= ceil(ctx/16) are -1
    context_lens [num_seqs] int32, including the token being decoded
    """

    n_heads: int
    n_kv: int
    d: int
    dtype: str
    q: np.ndarray
    k_slots: np.ndarray
    v_slots: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    num_blocks: int
    block_size: int = BLOCK_SIZE
    name: str = ""
    seed: int = 0
    shared_prefix_blocks: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])


@dataclass
class PrefillCase:
    """A batch of prefill chunks over a paged cache.

    The chunk of sequence s holds q_len_s = cu_q_lens[s+1] - cu_q_lens[s]
    query tokens; they are the last q_len_s of its context_lens[s] tokens, and
    their keys/values are already in the pool.
    q [total_q, n_heads, d]
    """

    n_heads: int
    n_kv: int
    d: int
    dtype: str
    q: np.ndarray
    cu_q_lens: np.ndarray
    k_slots: np.ndarray
    v_slots: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    num_blocks: int
    block_size: int = BLOCK_SIZE
    name: str = ""
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_q_lens).astype(np.int32)

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])


def _blocks(n: int) -> int:
    return -(-int(n) // BLOCK_SIZE)


def _build_tables(ctx_list, shared_prefix_blocks, perm):
    """Assign physical ids, in order from `perm`: shared prefix first, then
    each sequence's private blocks in sequence order."""
    nseq = len(ctx_list)
    nb = [_blocks(c) for c in ctx_list]
    mb = max([1] + nb)
    tables = np.full((nseq, mb), -1, dtype=np.int32)
    P = shared_prefix_blocks
    cursor = P
    for s in range(nseq):
        if P:
            tables[s, :P] = perm[:P]
        k = nb[s] - P
        tables[s, P:nb[s]] = perm[cursor:cursor + k]
        cursor += k
    return tables, cursor


def make_decode_case(n_heads, n_kv, d, dtype, ctx, seed, *, pool_blocks=None, pool_factor=None,
                     shared_prefix_tokens=0, name="", ss_children=None) -> DecodeCase:
    """Build a decode case with the given context lengths.

    Streams (SeedSequence children of `seed`): [lengths, permutation, q, k, v];
    the lengths stream is used by the callers that draw lengths.
    """
    assert n_heads % n_kv == 0
    ctx = np.asarray(ctx, dtype=np.int64)
    assert shared_prefix_tokens % BLOCK_SIZE == 0
    P = shared_prefix_tokens // BLOCK_SIZE
    if P:
        assert (ctx >= shared_prefix_tokens).all()
    kids = ss_children if ss_children is not None else np.random.SeedSequence(seed).spawn(5)
    need = P + int(sum(_blocks(c) - P for c in ctx))
    if pool_blocks is None:
        pool_blocks = int(math.ceil(pool_factor * need)) if pool_factor else need
    assert pool_blocks >= need
    perm = np.random.Generator(np.random.PCG64(kids[1])).permutation(pool_blocks).astype(np.int32)
    tables, used = _build_tables(ctx.tolist(), P, perm)
    assert used == need
    S = len(ctx)
    q = _normal(kids[2], S * n_heads * d, dtype).reshape(S, n_heads, d)
    k = _normal(kids[3], pool_blocks * BLOCK_SIZE * n_kv * d, dtype).reshape(pool_blocks * BLOCK_SIZE, n_kv, d)
    v = _normal(kids[4], pool_blocks * BLOCK_SIZE * n_kv * d, dtype).reshape(pool_blocks * BLOCK_SIZE, n_kv, d)
    return DecodeCase(n_heads, n_kv, d, dtype, q, k, v, tables, ctx.astype(np.int32), pool_blocks,
                      name=name, seed=int(seed), shared_prefix_blocks=P)


def _lognormal_lengths(g, n, median, sigma, lo, hi):
    x = np.rint(median * np.exp(sigma * g.standard_normal(n)))
    return np.clip(x, lo, hi).astype(np.int64)


def make_config_case(index: int, *, num_seqs: int | None = None, seed: int | None = None) -> DecodeCase:
    """Decode case of workload `index` (1..4). `num_seqs` takes the first
    sequences of the same length draw (a smaller case of the same mix)."""
    cfg = CONFIGS[index]
    seed = config_seed(index) if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(5)
    g_len = np.random.Generator(np.random.PCG64(kids[0]))
    kw = dict(name=cfg["name"], ss_children=kids)
    if index == 1:
        ctx = np.array(cfg["ctx"], dtype=np.int64)
        if num_seqs is not None:
            ctx = ctx[:num_seqs]
        return make_decode_case(cfg["n_heads"], cfg["n_kv"], cfg["d"], cfg["dtype"], ctx, seed,
                                pool_blocks=cfg["pool_blocks"], **kw)
    if index == 2:
        n = cfg["num_seqs"]
        ctx = g_len.integers(cfg["ctx_lo"], cfg["ctx_hi"], size=n, endpoint=True)
        if num_seqs is not None:
            ctx = ctx[:num_seqs]
        return make_decode_case(cfg["n_heads"], cfg["n_kv"], cfg["d"], cfg["dtype"], ctx, seed,
                                pool_factor=cfg["pool_factor"], **kw)
    if index == 3:
        n = cfg["num_seqs"]
        tails = g_len.integers(cfg["tail_lo"], cfg["tail_hi"], size=n, endpoint=True)
        if num_seqs is not None:
            tails = tails[:num_seqs]
        ctx = cfg["prefix_tokens"] + tails
        return make_decode_case(cfg["n_heads"], cfg["n_kv"], cfg["d"], cfg["dtype"], ctx, seed,
                                shared_prefix_tokens=cfg["prefix_tokens"], **kw)
    if index == 4:
        n = cfg["num_seqs"] if num_seqs is None else num_seqs
        ctx = np.full(n, cfg["ctx_fixed"], dtype=np.int64)
        return make_decode_case(cfg["n_heads"], cfg["n_kv"], cfg["d"], cfg["dtype"], ctx, seed, **kw)
    raise ValueError("workload 5 is a mixed step: use make_mixed_case")


def make_mixed_case(*, seed: int | None = None, decode_seqs: int | None = None,
                    chunk_tokens: int | None = None, cached_tokens: int | None = None):
    """Workload 5: one causal prefill chunk plus a batch of decode sequences,
    all in one pool. Returns (PrefillCase, DecodeCase) sharing k_slots/v_slots."""
    cfg = CONFIGS[5]
    seed = config_seed(5) if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(7)
    g_len = np.random.Generator(np.random.PCG64(kids[0]))
    nd = cfg["decode_seqs"] if decode_seqs is None else decode_seqs
    dec_ctx = _lognormal_lengths(g_len, cfg["decode_seqs"], cfg["decode_median"], cfg["decode_sigma"],
                                 cfg["decode_lo"], cfg["decode_hi"])[:nd]
    chunk = cfg["chunk_tokens"] if chunk_tokens is None else chunk_tokens
    cached = cfg["cached_tokens"] if cached_tokens is None else cached_tokens
    pre_ctx = cached + chunk
    H, Hkv, d, dt = cfg["n_heads"], cfg["n_kv"], cfg["d"], cfg["dtype"]
    all_ctx = [pre_ctx] + dec_ctx.tolist()
    need = sum(_blocks(c) for c in all_ctx)
    perm = np.random.Generator(np.random.PCG64(kids[1])).permutation(need).astype(np.int32)
    tables, used = _build_tables(all_ctx, 0, perm)
    k = _normal(kids[3], need * BLOCK_SIZE * Hkv * d, dt).reshape(need * BLOCK_SIZE, Hkv, d)
    v = _normal(kids[4], need * BLOCK_SIZE * Hkv * d, dt).reshape(need * BLOCK_SIZE, Hkv, d)
    q_pre = _normal(kids[2], chunk * H * d, dt).reshape(chunk, H, d)
    q_dec = _normal(kids[5], nd * H * d, dt).reshape(nd, H, d)
    pre = PrefillCase(H, Hkv, d, dt, q_pre, np.array([0, chunk], dtype=np.int32), k, v,
                      np.ascontiguousarray(tables[:1, :_blocks(pre_ctx)]), np.array([pre_ctx], dtype=np.int32),
                      need, name=cfg["name"] + "/prefill", seed=seed)
    mb = max(1, max(_blocks(c) for c in dec_ctx)) if nd else 1
    dec = DecodeCase(H, Hkv, d, dt, q_dec, k, v, np.ascontiguousarray(tables[1:, :mb]),
                     dec_ctx.astype(np.int32), need, name=cfg["name"] + "/decode", seed=seed)
    return pre, dec


def make_prefill_case(n_heads, n_kv, d, dtype, ctx, q_lens, seed, *, pool_factor=None, name="") -> PrefillCase:
    """General prefill batch: sequence s has context ctx[s], of which the last
    q_lens[s] tokens are the chunk being prefilled."""
    ctx = np.asarray(ctx, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    assert (q_lens <= ctx).all() and (q_lens >= 0).all()
    base = make_decode_case(n_heads, n_kv, d, dtype, ctx, seed, pool_factor=pool_factor, name=name)
    kids = np.random.SeedSequence([seed, 1]).spawn(1)
    total = int(q_lens.sum())
    q = _normal(kids[0], total * n_heads * d, dtype).reshape(total, n_heads, d)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return PrefillCase(n_heads, n_kv, d, dtype, q, cu, base.k_slots, base.v_slots, base.block_tables,
                       base.context_lens, base.num_blocks, name=name, seed=int(seed))


# ----------------------------------------------------------------------------
# Structural transforms of a case (pure data movement)
# ----------------------------------------------------------------------------

def used_slot_mask(case) -> np.ndarray:
    """Boolean [num_blocks * 16]: slots that some sequence reads (t < ctx)."""
    used = np.zeros(case.num_blocks * BLOCK_SIZE, dtype=bool)
    for s in range(case.num_seqs):
        n = int(case.context_lens[s])
        if n <= 0:
            continue
        t = np.arange(n)
        b = case.block_tables[s, t // BLOCK_SIZE]
        used[b.astype(np.int64) * BLOCK_SIZE + t % BLOCK_SIZE] = True
    return used


def poison_unused(case, kind: str = "nan"):
    """Copy of `case` whose never-read slots (the tail of each last block and
    every unreferenced block) hold NaN (kind='nan') or +-1e4 (kind='big')."""
    used = used_slot_mask(case)
    k = case.k_slots.copy()
    v = case.v_slots.copy()
    bad = ~used
    if case.dtype == "f32":
        val_k = np.float32(np.nan) if kind == "nan" else np.float32(1e4)
        val_v = np.float32(np.nan) if kind == "nan" else np.float32(-1e4)
    else:
        val_k = np.uint16(0x7FC0) if kind == "nan" else f32_to_bf16_bits(np.array([1e4], np.float32))[0]
        val_v = np.uint16(0x7FC0) if kind == "nan" else f32_to_bf16_bits(np.array([-1e4], np.float32))[0]
    k[bad] = val_k
    v[bad] = val_v
    return replace(case, k_slots=k, v_slots=v)


def permute_pool(case, seed: int):
    """Relabel physical blocks by a random bijection pi: block b moves to pi[b]
    and every table entry e becomes pi[e]. The logical content of every
    sequence is unchanged."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    pi = g.permutation(case.num_blocks).astype(np.int64)
    bs = BLOCK_SIZE
    src = case.k_slots.reshape(case.num_blocks, bs, *case.k_slots.shape[1:])
    dst = np.empty_like(src)
    dst[pi] = src
    vsrc = case.v_slots.reshape(case.num_blocks, bs, *case.v_slots.shape[1:])
    vdst = np.empty_like(vsrc)
    vdst[pi] = vsrc
    t = case.block_tables.astype(np.int64)
    t2 = np.where(t >= 0, pi[np.clip(t, 0, None)], -1).astype(np.int32)
    out = replace(case, k_slots=dst.reshape(case.k_slots.shape), v_slots=vdst.reshape(case.v_slots.shape),
                  block_tables=t2)
    out.extra = dict(case.extra, perm=pi)
    return out


def private_twin(case: DecodeCase) -> DecodeCase:
    """Same sequences, but every sequence gets its own copy of the shared
    prefix blocks (appended after the original pool)."""
    P = case.shared_prefix_blocks
    assert P > 0
    S, bs = case.num_seqs, BLOCK_SIZE
    NB = case.num_blocks
    NB2 = NB + S * P
    shp = case.k_slots.shape[1:]
    k = np.empty((NB2 * bs,) + shp, dtype=case.k_slots.dtype)
    v = np.empty_like(k)
    k[:NB * bs] = case.k_slots
    v[:NB * bs] = case.v_slots
    tables = case.block_tables.copy()
    for s in range(S):
        for j in range(P):
            src = int(case.block_tables[s, j])
            dst = NB + s * P + j
            k[dst * bs:(dst + 1) * bs] = case.k_slots[src * bs:(src + 1) * bs]
            v[dst * bs:(dst + 1) * bs] = case.v_slots[src * bs:(src + 1) * bs]
            tables[s, j] = dst
    return replace(case, k_slots=k, v_slots=v, block_tables=tables, num_blocks=NB2, shared_prefix_blocks=0,
                   name=case.name + "/private")


# ----------------------------------------------------------------------------
# Retrieval probes (closed-form outputs)
# ----------------------------------------------------------------------------

def _probe_digits(n_slots, n_kv, d):
    """V[slot, h] = [slot % 16, h, block % 128, block // 128, 0, ...]; every
    digit is an integer in [0, 127], exact in fp32, bf16 and int8."""
    v = np.zeros((n_slots, n_kv, d), dtype=np.float32)
    slot = np.arange(n_slots)
    v[:, :, 0] = (slot % BLOCK_SIZE)[:, None]
    v[:, :, 1] = np.arange(n_kv)[None, :]
    v[:, :, 2] = ((slot // BLOCK_SIZE) % 128)[:, None]
    v[:, :, 3] = ((slot // BLOCK_SIZE) // 128)[:, None]
    return v


def make_probe_case(n_heads, n_kv, d, dtype, ctx, seed, *, pool_factor=1.25, magnet=40.0):
    """Decode probe: K is zero except one 'magnet' key per sequence at a
    seeded position t*, equal to magnet*e0 in every KV head; every query is
    magnet*e0. The magnet's score exceeds every other by magnet^2/sqrt(d)
    (>= 141 for d <= 128), so every other softmax weight underflows to 0 in
    float32 and the output must equal V at t* exactly. V encodes each slot's
    offset, KV head and physical block (see _probe_digits)."""
    base = make_decode_case(n_heads, n_kv, d, "f32", ctx, seed, pool_factor=pool_factor)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3])))
    S = base.num_seqs
    tstar = np.array([g.integers(0, int(c)) for c in base.context_lens], dtype=np.int64)
    nslots = base.num_blocks * BLOCK_SIZE
    k = np.zeros((nslots, n_kv, d), dtype=np.float32)
    for s in range(S):
        b = int(base.block_tables[s, tstar[s] // BLOCK_SIZE])
        k[b * BLOCK_SIZE + tstar[s] % BLOCK_SIZE, :, 0] = magnet
    v = _probe_digits(nslots, n_kv, d)
    q = np.zeros((S, n_heads, d), dtype=np.float32)
    q[:, :, 0] = magnet
    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    out = replace(base, dtype=dtype, q=q, k_slots=k, v_slots=v, name="probe")
    out.extra = dict(tstar=tstar)
    return out


def make_prefix_probe_case(n_heads, n_kv, d, dtype, prefix_tokens, tails, seed, *, shared_pos, tail_magnet):
    """Decode probe over a shared prefix: every sequence's table points its
    first prefix_tokens / 16 blocks at the same physical blocks, followed by
    a private tail of tails[s] tokens. K is zero except a 'shared' magnet
    40*e0 at prefix position shared_pos (seen by every sequence) and, for
    each sequence with tail_magnet[s], a 'tail' magnet 80*e0 at a seeded
    position of its tail; every query is 40*e0. Scores are then 0, 1600 and
    3200 (exact), i.e. gaps of at least 1600/sqrt(d) >= 141 between the
    largest score and every other, so every other softmax weight underflows
    to 0 in float32: the output is V at the sequence's tail magnet if it
    has one, else V at shared_pos, exactly. V encodes each slot's offset,
    KV head and physical block (see _probe_digits)."""
    assert prefix_tokens % BLOCK_SIZE == 0 and 0 <= shared_pos < prefix_tokens
    tails = np.asarray(tails, dtype=np.int64)
    assert (tails >= 1).all() and len(tail_magnet) == len(tails)
    ctx = prefix_tokens + tails
    base = make_decode_case(n_heads, n_kv, d, "f32", ctx, seed, shared_prefix_tokens=prefix_tokens)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 5])))
    S = base.num_seqs
    nslots = base.num_blocks * BLOCK_SIZE
    k = np.zeros((nslots, n_kv, d), dtype=np.float32)

    def slot(s, t):
        return int(base.block_tables[s, t // BLOCK_SIZE]) * BLOCK_SIZE + t % BLOCK_SIZE

    k[slot(0, shared_pos), :, 0] = 40.0
    tstar = np.full(S, shared_pos, dtype=np.int64)
    for s in range(S):
        if tail_magnet[s]:
            tstar[s] = prefix_tokens + int(g.integers(0, int(tails[s])))
            k[slot(s, int(tstar[s])), :, 0] = 80.0
    v = _probe_digits(nslots, n_kv, d)
    q = np.zeros((S, n_heads, d), dtype=np.float32)
    q[:, :, 0] = 40.0
    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    out = replace(base, dtype=dtype, q=q, k_slots=k, v_slots=v, name="prefix_probe")
    out.extra = dict(tstar=tstar)
    return out


def make_prefill_probe_case(n_heads, n_kv, d, dtype, ctx, q_lens, seed):
    """Causal prefill probe: key t is (t // 64, t % 64, 0, ...) and every query
    is (2**17, 2**11, 0, ...), so scores are exact integers strictly
    increasing in t with gaps of 2**11 (>= 181 after the 1/sqrt(d) scale, for
    d <= 128). A causal query at absolute position p therefore puts all its
    weight on key p, and its output must equal V at p exactly; a query that
    sees key p+1 returns V[p+1] instead."""
    ctx = np.asarray(ctx, dtype=np.int64)
    assert int(ctx.max()) // 64 < 128
    base = make_prefill_case(n_heads, n_kv, d, "f32", ctx, q_lens, seed, pool_factor=1.25)
    nslots = base.num_blocks * BLOCK_SIZE
    k = np.zeros((nslots, n_kv, d), dtype=np.float32)
    for s in range(base.num_seqs):
        n = int(ctx[s])
        t = np.arange(n)
        slots = base.block_tables[s, t // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + t % BLOCK_SIZE
        k[slots, :, 0] = (t // 64)[:, None]
        k[slots, :, 1] = (t % 64)[:, None]
    v = _probe_digits(nslots, n_kv, d)
    q = np.zeros_like(base.q, dtype=np.float32)
    q[:, :, 0] = 2.0 ** 17
    q[:, :, 1] = 2.0 ** 11
    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return replace(base, dtype=dtype, q=q, k_slots=k, v_slots=v, name="prefill_probe")


# ----------------------------------------------------------------------------
# Prefix sharing in clusters
# ----------------------------------------------------------------------------

def make_clustered_prefix_case(n_heads, n_kv, d, dtype, clusters, seed, *, pool_factor=1.1, name="clusters"):
    """Decode case whose sequences come in clusters, each cluster pointing the
    first `prefix_blocks` entries of every member's table at the same
    physical blocks (prefix caching at block granularity) and the rest at
    private blocks. clusters: list of (prefix_blocks, [ctx of each member]).
    A member may be shorter than its cluster's prefix: it then references
    only the shared blocks it covers (its slots past ctx are never read)."""
    kids = np.random.SeedSequence(seed).spawn(5)
    ctx, plan = [], []
    for pb_, members in clusters:
        for c in members:
            ctx.append(int(c))
            plan.append(int(pb_))
    ctx = np.asarray(ctx, dtype=np.int64)
    need = 0
    for pb_, members in clusters:
        need += pb_
        need += sum(max(0, _blocks(c) - pb_) for c in members)
    pool_blocks = int(math.ceil(pool_factor * need))
    perm = np.random.Generator(np.random.PCG64(kids[1])).permutation(pool_blocks).astype(np.int32)
    mb = max(1, max(_blocks(c) for c in ctx))
    tables = np.full((len(ctx), mb), -1, dtype=np.int32)
    cursor, s = 0, 0
    for pb_, members in clusters:
        shared = perm[cursor:cursor + pb_]
        cursor += pb_
        for c in members:
            nb = _blocks(c)
            k = min(nb, pb_)
            tables[s, :k] = shared[:k]
            priv = max(0, nb - pb_)
            tables[s, k:k + priv] = perm[cursor:cursor + priv]
            cursor += priv
            s += 1
    assert cursor == need
    S = len(ctx)
    q = _normal(kids[2], S * n_heads * d, dtype).reshape(S, n_heads, d)
    k = _normal(kids[3], pool_blocks * BLOCK_SIZE * n_kv * d, dtype).reshape(pool_blocks * BLOCK_SIZE, n_kv, d)
    v = _normal(kids[4], pool_blocks * BLOCK_SIZE * n_kv * d, dtype).reshape(pool_blocks * BLOCK_SIZE, n_kv, d)
    return DecodeCase(n_heads, n_kv, d, dtype, q, k, v, tables, ctx.astype(np.int32), pool_blocks, name=name,
                      seed=int(seed))


def privatize(case: DecodeCase) -> DecodeCase:
    """Same sequences with no physical block referenced twice: every
    (sequence, logical block) gets its own copy of the block it pointed at,
    appended after the original pool."""
    S, bs = case.num_seqs, BLOCK_SIZE
    nblk = [_blocks(c) for c in case.context_lens]
    NB = case.num_blocks
    NB2 = NB + sum(nblk)
    shp = case.k_slots.shape[1:]
    k = np.empty((NB2 * bs,) + shp, dtype=case.k_slots.dtype)
    v = np.empty_like(k)
    k[:NB * bs] = case.k_slots
    v[:NB * bs] = case.v_slots
    tables = case.block_tables.copy()
    dst = NB
    for s in range(S):
        for j in range(nblk[s]):
            src = int(case.block_tables[s, j])
            k[dst * bs:(dst + 1) * bs] = case.k_slots[src * bs:(src + 1) * bs]
            v[dst * bs:(dst + 1) * bs] = case.v_slots[src * bs:(src + 1) * bs]
            tables[s, j] = dst
            dst += 1
    return replace(case, k_slots=k, v_slots=v, block_tables=tables, num_blocks=NB2, shared_prefix_blocks=0,
                   name=case.name + "/private")
