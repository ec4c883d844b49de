// Causal chunked-prefill attention over a paged KV cache, for gfx950.
//
// What is computed ("jovanaeducation" guide a2-inf-2, section "Chunked
// prefill"; "KV cache, continuous batching and paged attention", section
// "Scheduling prefill and decode"): a prompt is processed in chunks; chunk
// row i of sequence s sits at absolute position ctx_s - q_len_s + i and
// attends keys 0..position through the block table, so the chunk computes
// exactly the rows a whole-prompt causal prefill would.
//
// MFMA path (bf16 / int8 / int4 KV). One workgroup (4 waves) per (sequence,
// KV head, tile of chunk rows). The 16 MFMA columns of a column group are
// 16/G chunk tokens x G query heads of the KV head; each wave owns C column
// groups for the whole key range, so there is no cross-wave merge. Key
// blocks are streamed in pairs: the workgroup loads both blocks' K and V
// tiles into LDS once (register prefetch of the next pair overlaps the
// current pair's math) and every wave reads its MFMA operands from there:
//   S^T[32 keys x 16 cols] = K * Q^T,   O^T[d x 16 cols] += V^T * P^T
// Scores above the causal diagonal are masked by select. A wave skips the
// math of key pairs that lie entirely after its last row.
//
// fp32 KV: each (chunk row, KV head) runs the decode VALU loop with the
// row's causal context.
#include <type_traits>

#include "pa_attn.h"

namespace pa {

template <int D, int FMT, int C>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p, int ntile) {
    using M = Mfma<D, FMT>;
    constexpr int TILE = M::TILE;
    constexpr int NCHUNK = 4 * TILE / 16;                    // 16-byte chunks per key pair
    constexpr int PER_T = (NCHUNK + kThreads - 1) / kThreads;
    __shared__ __attribute__((aligned(16))) uint8_t kv_lds[4 * TILE];  // K b0 | K b1 | V b0 | V b1

    const int G = p.group;
    const int H = p.n_heads;
    const int TPG = 16 / G;
    const int QT = kWaves * C * TPG;
    const int unit = blockIdx.x;
    const int kvh = unit % p.n_kv;
    const int rest = unit / p.n_kv;
    const int qt = rest % ntile;
    const int s = rest / ntile;
    const int q0 = p.cu_q_lens[s];
    const int qlen = p.cu_q_lens[s + 1] - q0;
    const int i0 = qt * QT;
    if (i0 >= qlen) return;
    const int ctx = min(p.ctx[s], p.ctx_cap);
    const int shift = ctx - qlen;  // absolute position of chunk row 0

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int q = lane >> 4;
    const int ctok = col / G;
    const int gh = col - ctok * G;
    const bool col_ok = col < TPG * G;

    const int i_last = min(qlen, i0 + QT) - 1;
    const int kend = shift + i_last + 1;  // keys [0, kend) are visible to some row
    // with a sliding window, keys before kbeg are visible to no row
    const int kbeg = p.window > 0 ? max(0, shift + i0 - p.window + 1) : 0;

    // per column group: row, causal limit (and window start), Q operand
    int pos[C], plo[C];
    bool store_row[C];
    u32x4 qop[C][M::KSTEPS];
    const uint16_t* qbase = reinterpret_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int cg = 0; cg < C; ++cg) {
        const int i = i0 + (wave * C + cg) * TPG + ctok;
        const bool row_ok = col_ok && i < qlen;
        const int ps = shift + i;
        store_row[cg] = row_ok;
        const bool live = row_ok && ps >= 0;
        pos[cg] = live ? ps : kend - 1;  // dead columns see every key (their Q is 0) and are not stored
        plo[cg] = live && p.window > 0 ? ps - p.window + 1 : -1;
#pragma unroll
        for (int kk = 0; kk < M::KSTEPS; ++kk) {
            if (live) {
                qop[cg][kk] = *reinterpret_cast<const u32x4*>(qbase + ((size_t)(q0 + i) * H + kvh * G + gh) * D +
                                                               M::dbase(kk, q));
            } else {
                qop[cg][kk] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    const int wave_first_row = i0 + wave * C * TPG;
    const int wave_last_row = min(qlen - 1, i0 + (wave * C + C) * TPG - 1);
    // last key any row of this wave sees (-1: the wave has no rows), and the
    // first (the window's start of its first row)
    const int wave_kmax = wave_first_row < qlen ? shift + wave_last_row : -1;
    const int wave_kmin = p.window > 0 ? shift + wave_first_row - p.window + 1 : 0;

    float m[C], l[C];
    f32x4 acc[C][M::NB];
#pragma unroll
    for (int cg = 0; cg < C; ++cg) {
        m[cg] = kNegInf;
        l[cg] = 0.f;
#pragma unroll
        for (int nb = 0; nb < M::NB; ++nb) acc[cg][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int32_t* trow = p.tables + (size_t)s * p.max_blocks;
    const uint8_t* kpool = reinterpret_cast<const uint8_t*>(p.k_pool);
    const uint8_t* vpool = reinterpret_cast<const uint8_t*>(p.v_pool);
    const int nblk = kend > 0 ? (kend + kBlock - 1) / kBlock : 0;
    const int npairs = (nblk + 1) >> 1;

    int my_id = 0;
    int idwin = -1;
    u32x4 pre[PER_T];
    auto fetch = [&](int k) {
        if (((2 * k) >> 6) != idwin) {
            idwin = (2 * k) >> 6;
            my_id = load_ids(p.tables, trow, idwin << 6, min(64, nblk - (idwin << 6)), p.num_blocks);
        }
        const int j0 = (2 * k) & 63;
        const int id0 = readlane(my_id, j0);
        const int id1 = (2 * k + 1 < nblk) ? readlane(my_id, j0 + 1) : id0;
#pragma unroll
        for (int r = 0; r < PER_T; ++r) {
            const int c = tid + r * kThreads;
            if (c < NCHUNK) {
                const int ti = c / (TILE / 16);
                const int off = (c - ti * (TILE / 16)) * 16;
                const int id = (ti & 1) ? id1 : id0;
                const uint8_t* base = ti < 2 ? kpool : vpool;
                pre[r] = *reinterpret_cast<const u32x4*>(base + ((size_t)id * p.n_kv + kvh) * TILE + off);
            }
        }
    };

    const int k0 = kbeg / (2 * kBlock);  // first pair any row sees
    if (npairs > k0) fetch(k0);
    for (int k = k0; k < npairs; ++k) {
        const int j0 = (2 * k) & 63;
        const int id0 = readlane(my_id, j0);
        const bool has1 = 2 * k + 1 < nblk;
        const int id1 = has1 ? readlane(my_id, j0 + 1) : id0;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < PER_T; ++r) {
            const int c = tid + r * kThreads;
            if (c < NCHUNK) *reinterpret_cast<u32x4*>(kv_lds + c * 16) = pre[r];
        }
        __syncthreads();
        if (k + 1 < npairs) fetch(k + 1);

        const int key0 = 32 * k;
        if (key0 > wave_kmax) continue;  // every row of this wave is before this pair
        if (key0 + 31 < wave_kmin) continue;  // ... or past this pair's window

        float ks0 = 1.f, ks1 = 1.f, vs0 = 1.f, vs1 = 1.f;
        if (is_quant<FMT>()) {
            ks0 = fp16_bits_to_f32(p.k_scales[(size_t)id0 * p.n_kv + kvh]);
            ks1 = fp16_bits_to_f32(p.k_scales[(size_t)id1 * p.n_kv + kvh]);
            vs0 = fp16_bits_to_f32(p.v_scales[(size_t)id0 * p.n_kv + kvh]);
            vs1 = fp16_bits_to_f32(p.v_scales[(size_t)id1 * p.n_kv + kvh]);
        }
        typename M::KRaw kr0, kr1;
        M::load_k(kv_lds, lane, kr0);
        M::load_k(kv_lds + TILE, lane, kr1);

        u32x4 pop[C];
        const int tok0 = key0 + 4 * q;
        const int tok1 = tok0 + kBlock;
#pragma unroll
        for (int cg = 0; cg < C; ++cg) {
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
            f32x4 s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < M::KSTEPS; ++kk) {
                s0 = mfma_16x16x32(M::k_operand(kr0, kk), qop[cg][kk], s0);
                s1 = mfma_16x16x32(M::k_operand(kr1, kk), qop[cg][kk], s1);
            }
            const float c0 = p.scale_log2 * ks0;
            const float c1 = p.scale_log2 * ks1;
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = (tok0 + i <= pos[cg] && tok0 + i >= plo[cg]) ? s0[i] * c0 : kNegInf;
                x[4 + i] = (has1 && tok1 + i <= pos[cg] && tok1 + i >= plo[cg]) ? s1[i] * c1 : kNegInf;
            }
            float mx = x[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
            mx = wave_max_xor(mx, 16);
            mx = wave_max_xor(mx, 32);
            const float mnew = fmaxf(m[cg], mx);
            // without a window mnew is finite (key 0 is visible to every
            // column, and pairs are in order); with one, a column whose window
            // starts past this pair has seen no key yet and its state stays 0
            const float mref = (mnew == kNegInf) ? 0.f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(m[cg] - mref);
            m[cg] = mnew;
            float pr[8];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                pr[i] = __builtin_amdgcn_exp2f(x[i] - mref);
                psum += pr[i];
            }
            l[cg] = l[cg] * alpha + psum;
#pragma unroll
            for (int nb = 0; nb < M::NB; ++nb) acc[cg][nb] *= alpha;
            pop[cg][0] = pack_bf16x2(pr[0] * vs0, pr[1] * vs0);
            pop[cg][1] = pack_bf16x2(pr[2] * vs0, pr[3] * vs0);
            pop[cg][2] = pack_bf16x2(pr[4] * vs1, pr[5] * vs1);
            pop[cg][3] = pack_bf16x2(pr[6] * vs1, pr[7] * vs1);
        }

        // V slots past the context (only in the sequence's last pair) may hold anything
        const bool tail = !has1 || (2 * k + 2) * kBlock > ctx;
        uint32_t msk0[2] = {0xffffffffu, 0xffffffffu};
        uint32_t msk1[2] = {0xffffffffu, 0xffffffffu};
        if (tail) {
#pragma unroll
            for (int w2 = 0; w2 < 2; ++w2) {
                const int ta = tok0 + 2 * w2, tb = tok1 + 2 * w2;
                msk0[w2] = (ta < ctx ? 0x0000ffffu : 0u) | (ta + 1 < ctx ? 0xffff0000u : 0u);
                msk1[w2] = (has1 && tb < ctx ? 0x0000ffffu : 0u) | (has1 && tb + 1 < ctx ? 0xffff0000u : 0u);
            }
        }
        typename M::VRaw vr0, vr1;
        M::load_v(kv_lds + 2 * TILE, lane, vr0);
        M::load_v(kv_lds + 3 * TILE, lane, vr1);
#pragma unroll
        for (int nb = 0; nb < M::NB; ++nb) {
            const u32x2 a0 = M::v_half(vr0, nb);
            const u32x2 a1 = M::v_half(vr1, nb);
            u32x4 vop;
            vop[0] = a0[0] & msk0[0];
            vop[1] = a0[1] & msk0[1];
            vop[2] = a1[0] & msk1[0];
            vop[3] = a1[1] & msk1[1];
#pragma unroll
            for (int cg = 0; cg < C; ++cg) acc[cg][nb] = mfma_16x16x32(vop, pop[cg], acc[cg][nb]);
        }
    }

    uint16_t* obase = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
    for (int cg = 0; cg < C; ++cg) {
        float lt = l[cg];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        if (!store_row[cg]) continue;
        const int i = i0 + (wave * C + cg) * TPG + ctok;
        const bool live = shift + i >= 0;
        const float inv = live ? 1.f / lt : 0.f;
        uint16_t* orow = obase + ((size_t)(q0 + i) * H + kvh * G + gh) * D;
#pragma unroll
        for (int nb = 0; nb < M::NB; ++nb) {
            u32x2 o;
            o[0] = pack_bf16x2(acc[cg][nb][0] * inv, acc[cg][nb][1] * inv);
            o[1] = pack_bf16x2(acc[cg][nb][2] * inv, acc[cg][nb][3] * inv);
            *reinterpret_cast<u32x2*>(orow + nb * 16 + 4 * q) = o;
        }
    }
}

// -----------------------------------------------------------------------------
// Tile path (bf16 KV, d_head 128, G dividing 32). One workgroup of 8 waves
// per (sequence, KV head, tile of 256/G chunk tokens); wave w owns 32 query
// rows (32/G tokens x G heads), one 32-column MFMA tile, so every MFMA is
// 32x32x16 with all columns in use, and two waves share each SIMD (one
// wave issues while the other waits on LDS; a SIMD overlaps one wave's
// MFMAs with another's VALU work only a little, so the stage costs about
// the sum of the two). Keys stream through LDS in
// stages of 64 (four blocks of K, then four of V, 32 KiB), double-buffered:
// the next stage's loads are in flight while this stage is computed, and
// one barrier per stage hands the buffer over. Per stage and wave:
//   S^T[64 keys x 32 rows] = K Q^T      (16 MFMA, K rows read from LDS)
//   online softmax per row (column), causal mask by select on the diagonal
//   O^T[128 x 32 rows]     += V^T P^T   (16 MFMA, V^T read from LDS)
// The S^T accumulator of a lane is exactly its P^T operand (keys
// 8*(r/4) + 4*(l/32) + r%4 of its column), and the V^T operand reads the
// same keys as one 16-byte run from the staged V layout.
//
// PREFIX: the prefix pass of a decode step. The rows are those of 256/G
// consecutive decode sequences (a tile) instead of chunk tokens, the keys a
// range of the tile's common leading run of blocks (whole stages), which
// every row sees whole (no mask). Every workgroup of the tile first finds
// that run (the same way, so they agree); the result is a log-sum-exp
// partial per row.
// -----------------------------------------------------------------------------
constexpr int kTileWaves = 8;
constexpr int kTileThreads = kTileWaves * kWave;
constexpr int kStageBlocks = 4;
constexpr int kStageKeys = kStageBlocks * kBlock;   // 64
constexpr int kTile128 = kBlock * 128 * 2;          // 4 KiB
constexpr int kStageBytes = 2 * kStageBlocks * kTile128;

// Longest leading run of blocks that the n (>= 2) sequences from s0 on all
// hold at the same physical ids, ending at least one token before the end
// of the shortest of them; 0 if n < 2. Whole workgroup; every thread gets
// the result. Blocks are compared in windows of 256 from the start, so a
// batch without a common prefix costs one window.
__device__ __forceinline__ int common_run(const PrefillParams& p, int s0, int n, int* red) {
    const int tid = threadIdx.x;
    if (tid == 0) *red = 0x7fffffff;
    __syncthreads();
    int cap = 0x7fffffff;
    for (int i = tid; i < n; i += kTileThreads) {
        const int c = min(p.ctx[s0 + i], p.ctx_cap);
        cap = min(cap, c > 0 ? (c - 1) / kBlock : -1);  // whole blocks before the last token
    }
    atomicMin(red, cap);
    __syncthreads();
    int run = n >= 2 ? max(*red, 0) : 0;
    const int32_t* t0 = p.tables + (size_t)s0 * p.max_blocks;
    for (int j0 = 0; j0 < run; j0 += 256) {
        const int w = min(256, run - j0);
        __syncthreads();  // every thread has read *red
        if (tid == 0) *red = 0x7fffffff;
        __syncthreads();
        int miss = 0x7fffffff;
        for (int e = tid; e < (n - 1) * w; e += kTileThreads) {
            const int i = 1 + e / w;
            const int j = j0 + (e - (i - 1) * w);
            if (p.tables[(size_t)(s0 + i) * p.max_blocks + j] != t0[j]) miss = min(miss, j);
        }
        atomicMin(red, miss);
        __syncthreads();
        if (*red != 0x7fffffff) run = *red;  // uniform: ends the loop
    }
    return run;
}

template <bool PREFIX>
__global__ __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_tile_kernel(PrefillParams p, int ntile) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];
    constexpr int D = 128;
    const int G = p.group;
    const int TPW = 32 / G;  // chunk tokens (prefix: sequences) per wave
    const int QT = kTileWaves * TPW;
    const int unit = blockIdx.x;
    const int kvh = unit % p.n_kv;
    const int rest = unit / p.n_kv;
    // chunk: rows i0.. of sequence s (query rows q0 + i); prefix: sequences
    // i0.. (query rows i), keys of stages [st_begin, st_end)
    int s, q0, qlen, i0, ctx, shift, st_begin = 0, st_end = 0, kp = 0, tile = 0;
    if constexpr (PREFIX) {
        kp = rest % p.kpmax;
        tile = rest / p.kpmax;
        s = tile * QT;  // the tile's first sequence, whose table row is read
        q0 = 0;
        qlen = p.num_seqs;
        i0 = s;
        ctx = 0x3fffffff;  // every key of the run is in every row's context
        shift = 0x3fffffff;
    } else {
        const int qt = rest % ntile;
        s = rest / ntile;
        q0 = p.cu_q_lens[s];
        qlen = p.cu_q_lens[s + 1] - q0;
        i0 = qt * QT;
        if (i0 >= qlen) return;
        ctx = min(p.ctx[s], p.ctx_cap);
        shift = ctx - qlen;  // absolute position of chunk row 0
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;     // column (query row) of the wave's tile
    const int half = lane >> 5;  // k-slot group
    const int H = p.n_heads;

    // the lane's query row and its Q^T operand
    const int i = i0 + wave * TPW + n / G;
    const bool row_ok = i < qlen;
    const int pos = row_ok ? shift + i : -1;
    u32x4 qop[8];
    {
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)(q0 + i) * H + kvh * G + n % G) * D;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            qop[kk] = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * half) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    if constexpr (PREFIX) {  // the tile's run and this workgroup's range of it (Q loads in flight)
        __shared__ int red;
        int run = common_run(p, s, min(QT, p.num_seqs - s), &red);
        run -= run % kPrefixStageBlocks;
        if (run < kMinPrefixBlocks) run = 0;
        if (kp == 0 && kvh == 0 && tid == 0) p.plan[tile] = run;
        const int nparts = prefix_parts(run, p.kpmax);
        if (kp >= nparts) return;
        const int stages = run / kPrefixStageBlocks;
        st_begin = kp * stages / nparts;
        st_end = (kp + 1) * stages / nparts;
    }
    const int wfirst = i0 + wave * TPW;
    int wave_kmax = 0, nblk, nstage;
    // with a sliding window: the first key any row of the workgroup sees, and
    // the window starts of the wave's first and last rows
    int wave_klo = 0, wave_khi = 0;
    if constexpr (PREFIX) {
        nblk = st_end * kStageBlocks;
        nstage = st_end;
    } else {
        const int i_last = min(qlen, i0 + QT) - 1;
        const int kend = shift + i_last + 1;  // keys [0, kend) are visible to some row
        wave_kmax = wfirst < qlen ? shift + min(qlen - 1, wfirst + TPW - 1) : -1;
        nblk = (kend + kBlock - 1) / kBlock;
        nstage = (kend + kStageKeys - 1) / kStageKeys;
        st_end = nstage;
        if (p.window > 0) {
            st_begin = max(0, shift + i0 - p.window + 1) / kStageKeys;
            wave_klo = shift + wfirst - p.window + 1;
            wave_khi = shift + min(qlen - 1, wfirst + TPW - 1) - p.window + 1;
        }
    }
    const int plo = p.window > 0 ? pos - p.window + 1 : -1;  // the row's first visible key

    const int32_t* trow = p.tables + (size_t)s * p.max_blocks;
    const uint8_t* kpool = reinterpret_cast<const uint8_t*>(p.k_pool);
    const uint8_t* vpool = reinterpret_cast<const uint8_t*>(p.v_pool);

    // Staging. K goes straight from global memory into LDS: load j of wave w
    // moves 1 KiB piece c = w + W j of the stage (W waves): block c / 4,
    // bytes (64 (c % 4) + lane) * 16 of its tile, lane by lane into
    // consecutive 16 bytes, so a stage's K tiles land in LDS as stored. V goes through registers into a layout
    // made for the P.V operand: the 8 keys a lane feeds one MFMA
    // (slots 4h..4h+3 and 8+4h..8+4h+3 of one dim, h = the lane's k-slot
    // group) form one 16-byte run at [block][h][dim], so eight consecutive
    // lanes read 128 contiguous bytes (no bank conflicts). Thread t stages V
    // chunks c = t, t + T, ... of the stage (T threads): block c / 256, dim
    // (c % 256) / 2, slots 8 ((c % 256) % 2) .. +7, split into two 8-byte runs.
    constexpr int KLD = kStageBlocks * kTile128 / 1024 / kTileWaves;  // K loads per wave per stage
    constexpr int VCH = kStageBlocks * kTile128 / 16 / kTileThreads;  // V chunks per thread per stage
    int win = -1, win_id = 0;
    u32x4 vstg[VCH];
    auto prefetch = [&](int st, uint8_t* buf) {
        if ((st * kStageBlocks) >> 6 != win) {  // ids of the next 64 blocks
            win = (st * kStageBlocks) >> 6;
            win_id = load_ids(p.tables, trow, win << 6, min(64, nblk - (win << 6)), p.num_blocks);
        }
#pragma unroll
        for (int j = 0; j < KLD; ++j) {
            const int c = wave + kTileWaves * j;     // 1 KiB piece of the stage's K
            const int blk = c >> 2;
            const int off = (64 * (c & 3) + lane) * 16;
            const int jb = st * kStageBlocks + blk;  // logical block (wave-uniform)
            if (jb >= nblk) continue;                // past the last visible key (masked scores)
            const int id = __shfl(win_id, jb & 63);
            lds_dma16(kpool + ((size_t)id * p.n_kv + kvh) * kTile128 + off, buf + blk * kTile128 + (off - lane * 16));
        }
#pragma unroll
        for (int j = 0; j < VCH; ++j) {
            const int c = tid + kTileThreads * j;
            const int jb = st * kStageBlocks + (c >> 8);
            // past the last visible block the window holds id 0 (a valid
            // block), whose keys the commit masks out
            const int id = __shfl(win_id, jb & 63);
            vstg[j] = *reinterpret_cast<const u32x4*>(vpool + ((size_t)id * p.n_kv + kvh) * kTile128 + (c & 255) * 16);
        }
    };
    // Write the staged V chunks, zeroing keys at or past the context (their
    // contents may be anything, and 0 * NaN = NaN), which covers the blocks
    // past the last visible one. K needs no care (masked scores are replaced
    // by -inf).
    auto commit = [&](int st, uint8_t* buf) {
        uint8_t* vbuf = buf + kStageBlocks * kTile128;
        // only a stage reaching the context's end has keys to zero (tested
        // for the whole stage first, so the other stages take no selects)
        const bool ends = (st + 1) * kStageKeys > ctx;
#pragma unroll
        for (int j = 0; j < VCH; ++j) {
            const int c = tid + kTileThreads * j;
            const int blk = c >> 8;
            const int d = (c & 255) >> 1;
            const int sh = c & 1;
            u32x4 v = vstg[j];
            const int key0 = (st * kStageBlocks + blk) * kBlock + 8 * sh;
            if (ends && key0 + 8 > ctx) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = key0 + 2 * e < ctx ? 0x0000ffffu : 0u;
                    const uint32_t hi = key0 + 2 * e + 1 < ctx ? 0xffff0000u : 0u;
                    v[e] &= lo | hi;
                }
            }
            uint8_t* row = vbuf + blk * kTile128 + d * 16 + sh * 8;
            *reinterpret_cast<u32x2*>(row) = u32x2{v[0], v[1]};                      // slots 8sh + 0..3
            *reinterpret_cast<u32x2*>(row + kTile128 / 2) = u32x2{v[2], v[3]};       // slots 8sh + 4..7
        }
    };

    float m = kNegInf, l = 0.f;
    f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

    // One stage of keys for the wave's 32 rows. The reference maximum m of a
    // row moves only when a score exceeds it by more than kSlack (log2
    // units); probabilities are then at most 2^kSlack, and the accumulator is
    // rescaled only in the rare stage where some row's reference moves. When
    // it moves it moves to the row's new maximum, whose own term is then
    // exactly 2^0.
    constexpr float kSlack = 8.f;
    auto stage = [&](const uint8_t* buf, int kb, auto diag_tag) __attribute__((always_inline)) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        const uint8_t* kst = buf;
        const uint8_t* vst = buf + kStageBlocks * kTile128;
        f32x16 sc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sc[kt] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(
                    kst + (2 * kt + n / 16) * kTile128 + ((2 * kk + half) * 16 + n % 16) * 16);
                sc[kt] = mfma_32x32x16(a, qop[kk], sc[kt]);
            }
        }
        // scores in log2 units, -inf past the row's position on a diagonal stage
        float mx = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = sc[kt][r] * p.scale_log2;
                if (DIAG) {  // causal diagonal, or a window's start, inside the stage
                    const int key = kb + 32 * kt + 8 * (r / 4) + 4 * half + r % 4;
                    x = key <= pos && key >= plo ? x : kNegInf;
                }
                sc[kt][r] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool up = mx > m + kSlack;  // false while mx is -inf
        const float mnew = up ? mx : m;
        const float mref = mnew == kNegInf ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m - mref);  // 1 unless moved (0 from -inf)
        m = mnew;
        u32x4 pop[2][2];
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            float pr[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                pr[r] = __builtin_amdgcn_exp2f(sc[kt][r] - mref);
                psum += pr[r];
            }
#pragma unroll
            for (int mh = 0; mh < 2; ++mh) {
                pop[kt][mh][0] = pack_bf16x2(pr[8 * mh + 0], pr[8 * mh + 1]);
                pop[kt][mh][1] = pack_bf16x2(pr[8 * mh + 2], pr[8 * mh + 3]);
                pop[kt][mh][2] = pack_bf16x2(pr[8 * mh + 4], pr[8 * mh + 5]);
                pop[kt][mh][3] = pack_bf16x2(pr[8 * mh + 6], pr[8 * mh + 7]);
            }
        }
        l = l * alpha + psum;
        if (__any(up)) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int d = 32 * dt + n;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int mh = 0; mh < 2; ++mh) {
                    const u32x4 vop = *reinterpret_cast<const u32x4*>(vst + (2 * kt + mh) * kTile128 +
                                                                       half * (kTile128 / 2) + d * 16);
                    acc[dt] = mfma_32x32x16(vop, pop[kt][mh], acc[dt]);
                }
            }
        }
    };

    // One loop step: the next stage's loads go out into the other buffer
    // (last read before the previous barrier), the wave computes stage st
    // (FULL: every row of the workgroup sees all of it; else the wave
    // decides), the staged V of st + 1 is written, and the barrier hands
    // that buffer over.
    auto step = [&](int st, auto full_tag) __attribute__((always_inline)) {
        uint8_t* buf = lds + (st & 1) * kStageBytes;
        uint8_t* nbuf = lds + ((st + 1) & 1) * kStageBytes;
        if (st + 1 < nstage) prefetch(st + 1, nbuf);
        const int kb = st * kStageKeys;
        // Rows of this wave whose position is at least kb + 63 see the whole
        // stage; only a stage on the causal diagonal needs the mask, or, with
        // a window, one holding some row's window start. A stage past every
        // row, or wholly before every row's window, is skipped. (Rows past the
        // chunk end never get stored.)
        if (decltype(full_tag)::value || PREFIX || (kb + kStageKeys - 1 <= shift + wfirst && kb >= wave_khi)) {
            stage(buf, kb, std::false_type{});
        } else if (kb <= wave_kmax && kb + kStageKeys - 1 >= wave_klo) {
            stage(buf, kb, std::true_type{});
        }
        if (st + 1 < nstage) {
            commit(st + 1, nbuf);
            __builtin_amdgcn_s_waitcnt(0);  // this thread's K loads have landed
        }
        __syncthreads();
    };
    // stages [full_lo, full_hi) are whole for every row of the workgroup: no
    // mask and no per-wave choice, so they run in a loop of their own
    int full_lo = st_begin, full_hi = nstage;
    if constexpr (!PREFIX) {
        full_hi = min(nstage, max(st_begin, (shift + i0 + 1) / kStageKeys));
        if (p.window > 0) {
            const int khi = shift + min(qlen - 1, i0 + QT - 1) - p.window + 1;  // last row's window start
            full_lo = max(st_begin, (max(khi, 0) + kStageKeys - 1) / kStageKeys);
        }
        if (full_lo > full_hi) full_lo = full_hi;
    }

    prefetch(st_begin, lds + (st_begin & 1) * kStageBytes);
    commit(st_begin, lds + (st_begin & 1) * kStageBytes);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's K loads have landed
    __syncthreads();
    for (int st = st_begin; st < full_lo; ++st) step(st, std::false_type{});
    for (int st = full_lo; st < full_hi; ++st) step(st, std::true_type{});
    for (int st = full_hi; st < nstage; ++st) step(st, std::false_type{});

    const float lt = l + __shfl_xor(l, 32);
    if (!row_ok) return;
    if constexpr (PREFIX) {
        // partial of the row in slot kp: (max, sum) in log2 units and the
        // unnormalised accumulator
        const size_t row = ((size_t)i * H + kvh * G + n % G) * p.pslots + kp;
        float* arow = p.part_acc + row * D;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const f32x4 o = {acc[dt][4 * rr + 0], acc[dt][4 * rr + 1], acc[dt][4 * rr + 2], acc[dt][4 * rr + 3]};
                *reinterpret_cast<f32x4*>(arow + 32 * dt + 8 * rr + 4 * half) = o;
            }
        }
        if (half == 0) *reinterpret_cast<f32x2*>(p.part_ml + row * 2) = f32x2{m, lt};
        return;
    }
    const float inv = 1.f / lt;
    uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + ((size_t)(q0 + i) * H + kvh * G + n % G) * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            u32x2 o;
            o[0] = pack_bf16x2(acc[dt][4 * rr + 0] * inv, acc[dt][4 * rr + 1] * inv);
            o[1] = pack_bf16x2(acc[dt][4 * rr + 2] * inv, acc[dt][4 * rr + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * rr + 4 * half) = o;
        }
    }
}

// fp32: one workgroup per (chunk row, KV head), the decode VALU loop over the
// row's causal context.
template <int D>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(PrefillParams pp) {
    __shared__ WaveState<D> st;
    __shared__ float qs[16 * D];
    const int unit = blockIdx.x;
    const int kvh = unit % pp.n_kv;
    const int rest = unit / pp.n_kv;
    const int i = rest % pp.max_q_len;
    const int s = rest / pp.max_q_len;
    const int q0 = pp.cu_q_lens[s];
    const int qlen = pp.cu_q_lens[s + 1] - q0;
    if (i >= qlen) return;
    const int ctx = min(pp.ctx[s], pp.ctx_cap);
    const int pos = ctx - qlen + i;

    DecodeParams p{};
    p.q = pp.q;
    p.k_pool = pp.k_pool;
    p.v_pool = pp.v_pool;
    p.out = pp.out;
    p.num_blocks = pp.num_blocks;
    p.n_heads = pp.n_heads;
    p.n_kv = pp.n_kv;
    p.group = pp.group;
    p.pmax = 1;
    p.pslots = 1;
    p.scale_log2 = pp.scale_log2;
    p.tables = pp.tables;

    Unit u;
    u.s = q0 + i;  // output / query row
    u.kvh = kvh;
    u.part = 0;
    u.slot0 = 0;
    u.ctx = pos + 1;
    u.lo = pp.window > 0 ? max(0, pos - pp.window + 1) : 0;
    if (u.ctx <= 0) {
        for (int idx = threadIdx.x; idx < p.group * D; idx += kThreads)
            store_out<D, true>(p, ((size_t)u.s * p.n_heads + kvh * p.group) * D + idx, 0.f);
        return;
    }
    u.nblk = (u.ctx + kBlock - 1) / kBlock;
    u.nparts = 1;
    u.b_begin = u.lo / kBlock;  // blocks wholly before the window are not read
    u.b_end = u.nblk;
    const float* qg = reinterpret_cast<const float*>(p.q) + ((size_t)u.s * p.n_heads + kvh * p.group) * D;
    for (int idx = threadIdx.x; idx < p.group * D; idx += kThreads) qs[idx] = qg[idx];
    __syncthreads();
    f32_wave<D>(p, u, pp.tables + (size_t)s * pp.max_blocks, st, qs);
    epilogue<D, true>(p, u, st, reinterpret_cast<float*>(&st), (int)(sizeof(st) / sizeof(float)));
}

hipError_t take_bad_id_prefill(BadIdRecord* out) {
    const BadIdRecord zero{};
    hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_bad_ids), sizeof(BadIdRecord), 0, hipMemcpyDeviceToHost);
    if (e == hipSuccess && out->flag)
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_bad_ids), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
    return e;
}

template <int D, int FMT, int C>
static hipError_t launch_mfma(const PrefillParams& p, hipStream_t stream) {
    const int tpg = 16 / p.group;
    const int qt = kWaves * C * tpg;
    const int ntile = (p.max_q_len + qt - 1) / qt;
    const size_t grid = (size_t)p.num_seqs * ntile * p.n_kv;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_kernel<D, FMT, C>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p, ntile);
    return hipGetLastError();
}

static hipError_t launch_tile(const PrefillParams& p, hipStream_t stream) {
    const int qt = kTileWaves * (32 / p.group);
    const int ntile = (p.max_q_len + qt - 1) / qt;
    const size_t grid = (size_t)p.num_seqs * ntile * p.n_kv;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(prefill_tile_kernel<false>, dim3((unsigned)grid), dim3(kTileThreads), 0, stream, p, ntile);
    return hipGetLastError();
}

hipError_t launch_prefix(const PrefillParams& p, hipStream_t stream) {
    if (p.group <= 0 || 32 % p.group != 0 || p.kpmax <= 0 || !p.plan) return hipErrorInvalidValue;
    const int ts = kTileWaves * (32 / p.group);
    const size_t grid = (size_t)((p.num_seqs + ts - 1) / ts) * p.kpmax * p.n_kv;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(prefill_tile_kernel<true>, dim3((unsigned)grid), dim3(kTileThreads), 0, stream, p, 0);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(const PrefillParams& p, hipStream_t stream) {
    const size_t grid = (size_t)p.num_seqs * p.max_q_len * p.n_kv;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_f32_kernel<D>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int d, int fmt, hipStream_t stream) {
    constexpr int C = 2;
    if (d == 128) {
        switch (fmt) {
            case FMT_F32: return launch_f32<128>(p, stream);
            case FMT_BF16:
                if (32 % p.group == 0) return launch_tile(p, stream);
                return launch_mfma<128, FMT_BF16, C>(p, stream);
            case FMT_I8: return launch_mfma<128, FMT_I8, C>(p, stream);
            case FMT_I4: return launch_mfma<128, FMT_I4, C>(p, stream);
            case FMT_F8: return launch_mfma<128, FMT_F8, C>(p, stream);
        }
    } else if (d == 64) {
        switch (fmt) {
            case FMT_F32: return launch_f32<64>(p, stream);
            case FMT_BF16: return launch_mfma<64, FMT_BF16, C>(p, stream);
            case FMT_I8: return launch_mfma<64, FMT_I8, C>(p, stream);
            case FMT_I4: return launch_mfma<64, FMT_I4, C>(p, stream);
            case FMT_F8: return launch_mfma<64, FMT_F8, C>(p, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
