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

    // per column group: row, causal limit, Q operand
    int pos[C];
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
    // last key any row of this wave sees (-1: the wave has no rows)
    const int wave_kmax = wave_first_row < qlen ? shift + wave_last_row : -1;

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
    int window = -1;
    u32x4 pre[PER_T];
    auto fetch = [&](int k) {
        if (((2 * k) >> 6) != window) {
            window = (2 * k) >> 6;
            my_id = load_ids(trow, window << 6, min(64, nblk - (window << 6)), p.num_blocks);
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

    if (npairs > 0) fetch(0);
    for (int k = 0; k < npairs; ++k) {
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

        float ks0 = 1.f, ks1 = 1.f, vs0 = 1.f, vs1 = 1.f;
        if (FMT == FMT_I8 || FMT == FMT_I4) {
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
                x[i] = (tok0 + i <= pos[cg]) ? s0[i] * c0 : kNegInf;
                x[4 + i] = (has1 && tok1 + i <= pos[cg]) ? s1[i] * c1 : kNegInf;
            }
            float mx = x[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
            mx = wave_max_xor(mx, 16);
            mx = wave_max_xor(mx, 32);
            const float mnew = fmaxf(m[cg], mx);
            // mnew is finite: key 0 is visible to every column, and pairs are in order
            const float alpha = __builtin_amdgcn_exp2f(m[cg] - mnew);
            m[cg] = mnew;
            float pr[8];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                pr[i] = __builtin_amdgcn_exp2f(x[i] - mnew);
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
    p.scale_log2 = pp.scale_log2;

    Unit u;
    u.s = q0 + i;  // output / query row
    u.kvh = kvh;
    u.part = 0;
    u.ctx = pos + 1;
    if (u.ctx <= 0) {
        for (int idx = threadIdx.x; idx < p.group * D; idx += kThreads)
            store_out<D, true>(p, ((size_t)u.s * p.n_heads + kvh * p.group) * D + idx, 0.f);
        return;
    }
    u.nblk = (u.ctx + kBlock - 1) / kBlock;
    u.nparts = 1;
    u.b_begin = 0;
    u.b_end = u.nblk;
    const float* qg = reinterpret_cast<const float*>(p.q) + ((size_t)u.s * p.n_heads + kvh * p.group) * D;
    for (int idx = threadIdx.x; idx < p.group * D; idx += kThreads) qs[idx] = qg[idx];
    __syncthreads();
    f32_wave<D>(p, u, pp.tables + (size_t)s * pp.max_blocks, st, qs);
    epilogue<D, true>(p, u, st);
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
            case FMT_BF16: return launch_mfma<128, FMT_BF16, C>(p, stream);
            case FMT_I8: return launch_mfma<128, FMT_I8, C>(p, stream);
            case FMT_I4: return launch_mfma<128, FMT_I4, C>(p, stream);
        }
    } else if (d == 64) {
        switch (fmt) {
            case FMT_F32: return launch_f32<64>(p, stream);
            case FMT_BF16: return launch_mfma<64, FMT_BF16, C>(p, stream);
            case FMT_I8: return launch_mfma<64, FMT_I8, C>(p, stream);
            case FMT_I4: return launch_mfma<64, FMT_I4, C>(p, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
