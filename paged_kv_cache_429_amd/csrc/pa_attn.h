// Building blocks shared by the decode and prefill kernels: the MFMA tile
// loaders / dequantisers for each KV format, the fp32 VALU wave loop and the
// log-sum-exp epilogue.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr float kNegInf = -__builtin_huge_valf();

template <int D>
struct WaveState {
    float m[kWaves][16];
    float l[kWaves][16];
    float acc[kWaves][16][D + 4];
};

struct Unit {
    int s, kvh, part, ctx, nblk, nparts, b_begin, b_end;
};

__device__ __forceinline__ int tile_id(const DecodeParams& p, int my_id, int j) {
    return readlane(my_id, j);
}

// -----------------------------------------------------------------------------
// MFMA wave loop
// -----------------------------------------------------------------------------
template <int D, int FMT>
struct Mfma {
    static constexpr int BITS = FmtBits<FMT>::v;
    static constexpr int TILE = 16 * D * BITS / 8;      // bytes of one (block, head) tile
    static constexpr int KSTEPS = D / 32;
    static constexpr int NB = D / 16;
    static constexpr int KDW = D * BITS / 128;          // K dwords per lane per block
    static constexpr int VDW = (FMT == FMT_BF16) ? 2 : 1;  // V dwords per lane per block per nb

    // First dim of the 8 consecutive dims lane group q feeds at k-step kk.
    __device__ static __forceinline__ int dbase(int kk, int q) {
        if (FMT == FMT_BF16) return 32 * kk + 8 * q;
        if (FMT == FMT_I8) return 64 * (kk >> 1) + 16 * q + 8 * (kk & 1);
        return (D == 128 ? 32 : 16) * q + 8 * kk;  // int4
    }

    struct KRaw { uint32_t w[KDW]; };
    struct VRaw { uint32_t w[NB * VDW]; };

    // Tile loads are nontemporal: decode streams every tile once, and the
    // streaming hint lifts the 4 KiB-tile gather rate on gfx950 by ~12%.
    // (The prefill kernel calls the same loaders on LDS, where the hint has
    // no effect.)

    __device__ static __forceinline__ void load_k(const uint8_t* tile, int lane, KRaw& r) {
        if (KDW >= 4) {
#pragma unroll
            for (int u = 0; u < KDW / 4; ++u) {
                u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tile + u * 1024 + lane * 16));
                r.w[4 * u + 0] = v[0];
                r.w[4 * u + 1] = v[1];
                r.w[4 * u + 2] = v[2];
                r.w[4 * u + 3] = v[3];
            }
        } else {  // int4, d = 64: half a 16-byte chunk per lane
            const int t = lane & 15, q = lane >> 4;
            u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(tile + (q >> 1) * 256 + t * 16 + (q & 1) * 8));
            r.w[0] = v[0];
            r.w[1] = v[1];
        }
    }

    __device__ static __forceinline__ u32x4 k_operand(const KRaw& r, int kk) {
        u32x4 a;
        if (FMT == FMT_BF16) {
            a[0] = r.w[4 * kk];
            a[1] = r.w[4 * kk + 1];
            a[2] = r.w[4 * kk + 2];
            a[3] = r.w[4 * kk + 3];
        } else if (FMT == FMT_I8) {
            u32x2 lo = i8x4_to_bf16x4(r.w[2 * kk]);
            u32x2 hi = i8x4_to_bf16x4(r.w[2 * kk + 1]);
            a[0] = lo[0];
            a[1] = lo[1];
            a[2] = hi[0];
            a[3] = hi[1];
        } else {
            a = i4x8_to_bf16x8(r.w[kk]);
        }
        return a;
    }

    __device__ static __forceinline__ void load_v(const uint8_t* tile, int lane, VRaw& r) {
        const int l16 = lane & 15, q = lane >> 4;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int d = nb * 16 + l16;
            if (FMT == FMT_BF16) {
                u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(tile + d * 32 + q * 8));
                r.w[2 * nb] = v[0];
                r.w[2 * nb + 1] = v[1];
            } else if (FMT == FMT_I8) {
                r.w[nb] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(tile + d * 16 + q * 4));
            } else {
                r.w[nb] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(tile + d * 8 + q * 2));
            }
        }
    }

    // bf16 values of tokens 4q..4q+3 at dim row nb*16 + lane%16
    __device__ static __forceinline__ u32x2 v_half(const VRaw& r, int nb) {
        if (FMT == FMT_BF16) {
            u32x2 x;
            x[0] = r.w[2 * nb];
            x[1] = r.w[2 * nb + 1];
            return x;
        } else if (FMT == FMT_I8) {
            return i8x4_to_bf16x4(r.w[nb]);
        } else {
            return i4x4_to_bf16x4(r.w[nb]);
        }
    }
};

// K half and V half of one pair of blocks in flight. They are loaded one
// phase apart (K of the next pair during this pair's softmax and P.V, V of
// the next pair during its Q.K), so only one pair's K and one pair's V are
// ever held in registers.
template <int D, int FMT>
struct KHalf {
    typename Mfma<D, FMT>::KRaw k0, k1;
    float s0, s1;
};

template <int D, int FMT>
struct VHalf {
    typename Mfma<D, FMT>::VRaw v0, v1;
    float s0, s1;
};

template <int D, int FMT>
__device__ __forceinline__ void mfma_wave(const DecodeParams& p, const Unit& u, int my_id, WaveState<D>& st) {
    using M = Mfma<D, FMT>;
    constexpr bool QUANT = (FMT == FMT_I8 || FMT == FMT_I4);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane & 15;
    const int q = lane >> 4;
    const int G = p.group;
    const int H = p.n_heads;

    // Q^T operand: column g = query head kvh*G + g, eight dims per k-step.
    u32x4 qop[M::KSTEPS];
    {
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)u.s * H + u.kvh * G + g) * D;
#pragma unroll
        for (int kk = 0; kk < M::KSTEPS; ++kk) {
            if (g < G) {
                qop[kk] = *reinterpret_cast<const u32x4*>(qrow + M::dbase(kk, q));
            } else {
                qop[kk] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }

    float m = kNegInf;
    float l = 0.f;
    f32x4 acc[M::NB];
#pragma unroll
    for (int nb = 0; nb < M::NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k_pool);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v_pool);
    const int nb_part = u.b_end - u.b_begin;
    const int npairs = (nb_part + 1) >> 1;

    // byte offsets of the two tiles of pair k (a missing second block
    // repeats the first, which is then masked out)
    auto tiles = [&](int k, size_t& t0, size_t& t1, int& i0, int& i1) {
        const int j0 = 2 * k;
        i0 = tile_id(p, my_id, j0);
        i1 = (j0 + 1) < nb_part ? tile_id(p, my_id, j0 + 1) : i0;
        t0 = ((size_t)i0 * p.n_kv + u.kvh) * M::TILE;
        t1 = ((size_t)i1 * p.n_kv + u.kvh) * M::TILE;
    };
    auto issue_k = [&](int k, KHalf<D, FMT>& r) {
        size_t t0, t1;
        int i0, i1;
        tiles(k, t0, t1, i0, i1);
        M::load_k(kbase + t0, lane, r.k0);
        M::load_k(kbase + t1, lane, r.k1);
        r.s0 = r.s1 = 1.f;
        if (QUANT) {
            r.s0 = fp16_bits_to_f32(p.k_scales[(size_t)i0 * p.n_kv + u.kvh]);
            r.s1 = fp16_bits_to_f32(p.k_scales[(size_t)i1 * p.n_kv + u.kvh]);
        }
    };
    auto issue_v = [&](int k, VHalf<D, FMT>& r) {
        size_t t0, t1;
        int i0, i1;
        tiles(k, t0, t1, i0, i1);
        M::load_v(vbase + t0, lane, r.v0);
        M::load_v(vbase + t1, lane, r.v1);
        r.s0 = r.s1 = 1.f;
        if (QUANT) {
            r.s0 = fp16_bits_to_f32(p.v_scales[(size_t)i0 * p.n_kv + u.kvh]);
            r.s1 = fp16_bits_to_f32(p.v_scales[(size_t)i1 * p.n_kv + u.kvh]);
        }
    };

    // S^T for pair k, scaled to log2 units and masked by select: x[0..3] are
    // tokens 4q..4q+3 of the first block, x[4..7] those of the second.
    auto qk = [&](int k, const KHalf<D, FMT>& r, float* x) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
        f32x4 s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < M::KSTEPS; ++kk) {
            s0 = mfma_16x16x32(M::k_operand(r.k0, kk), qop[kk], s0);
            s1 = mfma_16x16x32(M::k_operand(r.k1, kk), qop[kk], s1);
        }
        const int tok0 = (u.b_begin + 2 * k) * kBlock + 4 * q;
        const int tok1 = tok0 + kBlock;
        const bool has1 = 2 * k + 1 < nb_part;
        const float c0 = p.scale_log2 * r.s0;
        const float c1 = p.scale_log2 * r.s1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = (tok0 + i < u.ctx) ? s0[i] * c0 : kNegInf;
            x[4 + i] = (has1 && tok1 + i < u.ctx) ? s1[i] * c1 : kNegInf;
        }
    };

    // online-softmax update with the scores of pair k; returns the
    // probabilities (not yet scaled by the V scales) in pr
    auto softmax = [&](const float* x, float* pr) {
        float mx = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        const float mnew = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pr[i] = __builtin_amdgcn_exp2f(x[i] - mnew);
            psum += pr[i];
        }
        l = l * alpha + psum;
#pragma unroll
        for (int nb = 0; nb < M::NB; ++nb) acc[nb] *= alpha;
    };

    auto pv = [&](int k, const VHalf<D, FMT>& r, const float* pr) {
        u32x4 pop;
        pop[0] = pack_bf16x2(pr[0] * r.s0, pr[1] * r.s0);
        pop[1] = pack_bf16x2(pr[2] * r.s0, pr[3] * r.s0);
        pop[2] = pack_bf16x2(pr[4] * r.s1, pr[5] * r.s1);
        pop[3] = pack_bf16x2(pr[6] * r.s1, pr[7] * r.s1);
        // Tokens past the context (and a missing second block) have weight 0,
        // but their V slots may hold anything (0 * NaN = NaN): zero them.
        const int j0 = 2 * k;
        const bool has1 = j0 + 1 < nb_part;
        const int tok0 = (u.b_begin + j0) * kBlock + 4 * q;
        const int tok1 = tok0 + kBlock;
        const bool tail = !has1 || (u.b_begin + j0 + 2) * kBlock > u.ctx;
        uint32_t msk0[2] = {0xffffffffu, 0xffffffffu};
        uint32_t msk1[2] = {0xffffffffu, 0xffffffffu};
        if (tail) {
#pragma unroll
            for (int w2 = 0; w2 < 2; ++w2) {
                const int ta = tok0 + 2 * w2, tb = tok1 + 2 * w2;
                msk0[w2] = (ta < u.ctx ? 0x0000ffffu : 0u) | (ta + 1 < u.ctx ? 0xffff0000u : 0u);
                msk1[w2] = (has1 && tb < u.ctx ? 0x0000ffffu : 0u) | (has1 && tb + 1 < u.ctx ? 0xffff0000u : 0u);
            }
        }
#pragma unroll
        for (int nb = 0; nb < M::NB; ++nb) {
            const u32x2 a0 = M::v_half(r.v0, nb);
            const u32x2 a1 = M::v_half(r.v1, nb);
            u32x4 vop;
            vop[0] = a0[0] & msk0[0];
            vop[1] = a0[1] & msk0[1];
            vop[2] = a1[0] & msk1[0];
            vop[3] = a1[1] & msk1[1];
            acc[nb] = mfma_16x16x32(vop, pop, acc[nb]);
        }
    };

    // Waves take pairs wave, wave+4, ... In the steady loop the next pair
    // always exists, so every load is unconditional and the wait before each
    // use covers only the half it reads; the last pair runs after the loop.
    int k = wave;
    if (k < npairs) {
        KHalf<D, FMT> kr;
        VHalf<D, FMT> vr;
        issue_k(k, kr);
        issue_v(k, vr);
        float x[8], pr[8];
        for (; k + kWaves < npairs; k += kWaves) {
            qk(k, kr, x);
            issue_k(k + kWaves, kr);
            softmax(x, pr);
            pv(k, vr, pr);
            issue_v(k + kWaves, vr);
        }
        qk(k, kr, x);
        softmax(x, pr);
        pv(k, vr, pr);
    }

    // row sum over the four lane groups holding the same column
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (q == 0) {
        st.m[wave][g] = m;
        st.l[wave][g] = l;
    }
#pragma unroll
    for (int nb = 0; nb < M::NB; ++nb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st.acc[wave][g][nb * 16 + 4 * q + i] = acc[nb][i];
    }
}

// -----------------------------------------------------------------------------
// fp32 VALU wave loop (lane = (token t, dim quarter qd) for scores; lane = dim
// for the accumulator).
// -----------------------------------------------------------------------------
// Physical id of block (b_begin + j) for j in a 64-block window starting at
// `base`: lane l holds the id of block base + l; out-of-range ids become 0.
__device__ __forceinline__ int load_ids(const int32_t* trow, int first, int count, int num_blocks) {
    const int lane = threadIdx.x & 63;
    int id = 0;
    if (lane < count) {
        id = trow[first + lane];
        if ((unsigned)id >= (unsigned)num_blocks) id = 0;
    }
    return id;
}

template <int D>
__device__ __forceinline__ void f32_wave(const DecodeParams& p, const Unit& u, const int32_t* trow, WaveState<D>& st,
                                         const float* qs /* LDS [16][D] */) {
    constexpr int TILE = 16 * D * 4;
    constexpr int DL = D / 64;  // accumulator dims per lane
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane & 15;
    const int qd = lane >> 4;
    const int G = p.group;

    float m[16], l[16], acc[16][DL];
#pragma unroll
    for (int g = 0; g < 16; ++g) {
        m[g] = kNegInf;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < DL; ++e) acc[g][e] = 0.f;
    }
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k_pool);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v_pool);
    const int nb_part = u.b_end - u.b_begin;

    int my_id = 0;
    int window = -1;
    for (int j = wave; j < nb_part; j += kWaves) {
        if ((j >> 6) != window) {  // ids of the next 64 blocks
            window = j >> 6;
            my_id = load_ids(trow, u.b_begin + (window << 6), min(64, nb_part - (window << 6)), p.num_blocks);
        }
        const int id = tile_id(p, my_id, j & 63);
        const size_t toff = ((size_t)id * p.n_kv + u.kvh) * TILE;
        const float* kt = reinterpret_cast<const float*>(kbase + toff);
        const float* vt = reinterpret_cast<const float*>(vbase + toff);
        float part[16];
#pragma unroll
        for (int g = 0; g < 16; ++g) part[g] = 0.f;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            const int cc = qd * (D / 16) + c;  // 4-dim chunk index
            const f32x4 kv = *reinterpret_cast<const f32x4*>(kt + (cc * 16 + t) * 4);
#pragma unroll
            for (int g = 0; g < 16; ++g) {
                if (g < G) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) part[g] += qs[g * D + cc * 4 + e] * kv[e];
                }
            }
        }
        const int tok = (u.b_begin + j) * kBlock + t;
        const bool valid = tok < u.ctx;
        float pt[16];
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            if (g < G) {
                float dot = part[g];
                dot += __shfl_xor(dot, 16);
                dot += __shfl_xor(dot, 32);
                const float x = valid ? dot * p.scale_log2 : kNegInf;
                float mx = x;
                mx = wave_max_xor(mx, 1);
                mx = wave_max_xor(mx, 2);
                mx = wave_max_xor(mx, 4);
                mx = wave_max_xor(mx, 8);
                const float mnew = fmaxf(m[g], mx);
                const float alpha = __builtin_amdgcn_exp2f(m[g] - mnew);
                const float pv = __builtin_amdgcn_exp2f(x - mnew);
                float sum = pv;
                sum += __shfl_xor(sum, 1);
                sum += __shfl_xor(sum, 2);
                sum += __shfl_xor(sum, 4);
                sum += __shfl_xor(sum, 8);
                l[g] = l[g] * alpha + sum;
                m[g] = mnew;
#pragma unroll
                for (int e = 0; e < DL; ++e) acc[g][e] *= alpha;
                pt[g] = pv;
            }
        }
        // P.V: lane holds dims lane + 64e; V tile is dim-major (16 tokens per row)
#pragma unroll
        for (int e = 0; e < DL; ++e) {
            const int d = lane + 64 * e;
            float vrow[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(vt + d * 16 + 4 * c);
#pragma unroll
                for (int z = 0; z < 4; ++z) vrow[4 * c + z] = v4[z];
            }
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) {
                if ((u.b_begin + j) * kBlock + tt < u.ctx) {
#pragma unroll
                    for (int g = 0; g < 16; ++g) {
                        if (g < G) acc[g][e] += __shfl(pt[g], tt) * vrow[tt];
                    }
                }
            }
        }
    }
#pragma unroll
    for (int g = 0; g < 16; ++g) {
        if (g < G) {
            if (lane == 0) {
                st.m[wave][g] = m[g];
                st.l[wave][g] = l[g];
            }
#pragma unroll
            for (int e = 0; e < DL; ++e) st.acc[wave][g][lane + 64 * e] = acc[g][e];
        }
    }
}

// -----------------------------------------------------------------------------
// Epilogue: merge the waves' softmax states through LDS, then write the output
// (single-partition sequence) or this partition's partial (max, sum,
// unnormalised accumulator) for the merge kernel.
// -----------------------------------------------------------------------------
template <int D, bool F32OUT>
__device__ __forceinline__ void store_out(const DecodeParams& p, size_t idx, float v) {
    if (F32OUT) {
        reinterpret_cast<float*>(p.out)[idx] = v;
    } else {
        reinterpret_cast<uint16_t*>(p.out)[idx] = (uint16_t)f32_to_bf16_bits(v);
    }
}

// Partials cross workgroups that may run on different XCDs, whose L2 caches
// are not coherent with each other. They are written and read with
// agent-scope relaxed atomics, which the compiler issues as
// coherence-point accesses (no whole-cache write-back or invalidate, which
// an agent-scope fence would cost on every workgroup).
__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Log-sum-exp merge of the partials of (sequence s, KV head kvh), in
// partition order (m and l are in log2 units):
//   M = max_p m_p,  o = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M)
// The partials are fetched kChunk partitions at a time with independent
// loads (one round trip per chunk, not per partition); the running
// (M, L, O) is rescaled when a later chunk raises the maximum.
template <int D, bool F32OUT>
__device__ __forceinline__ void merge_partials(const DecodeParams& p, int s, int kvh, int nparts) {
    constexpr int kChunk = 8;
    const int G = p.group;
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int g = idx / D, d = idx - g * D;
        const size_t h = (size_t)s * p.n_heads + kvh * G + g;
        const float* ml = p.part_ml + h * p.pmax * 2;
        const float* acc = p.part_acc + h * p.pmax * D + d;
        float M = kNegInf, L = 0.f, O = 0.f;
        for (int p0 = 0; p0 < nparts; p0 += kChunk) {
            float mv[kChunk], lv[kChunk], av[kChunk];
#pragma unroll
            for (int c = 0; c < kChunk; ++c) {
                const bool ok = p0 + c < nparts;
                mv[c] = ok ? load_agent(ml + 2 * (p0 + c)) : kNegInf;
                lv[c] = ok ? load_agent(ml + 2 * (p0 + c) + 1) : 0.f;
                av[c] = ok ? load_agent(acc + (size_t)(p0 + c) * D) : 0.f;
            }
            float Mc = M;
#pragma unroll
            for (int c = 0; c < kChunk; ++c) Mc = fmaxf(Mc, mv[c]);
            const float r = __builtin_amdgcn_exp2f(M - Mc);  // 0 on the first chunk (M = -inf)
            L *= r;
            O *= r;
#pragma unroll
            for (int c = 0; c < kChunk; ++c) {
                const float e = __builtin_amdgcn_exp2f(mv[c] - Mc);  // 0 for padding (m = -inf)
                L += e * lv[c];
                O += e * av[c];
            }
            M = Mc;
        }
        store_out<D, F32OUT>(p, h * D + d, O / L);
    }
}

// Merge the waves' softmax states through LDS. A single-partition sequence
// writes its output here. Otherwise the workgroup writes its partition's
// partial (max, sum, unnormalised accumulator), and the last workgroup of
// the (sequence, KV head) to arrive merges all partials and re-arms the
// arrival counter (zero between calls).
template <int D, bool F32OUT>
__device__ __forceinline__ void epilogue(const DecodeParams& p, const Unit& u, WaveState<D>& st) {
    __syncthreads();
    const int G = p.group;
    const int H = p.n_heads;
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int g = idx / D, d = idx - g * D;
        float M = st.m[0][g];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, st.m[w][g]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = __builtin_amdgcn_exp2f(st.m[w][g] - M);  // 0 for a wave without blocks
            L += e * st.l[w][g];
            O += e * st.acc[w][g][d];
        }
        const size_t h = (size_t)u.s * H + u.kvh * G + g;
        if (u.nparts == 1) {
            store_out<D, F32OUT>(p, h * D + d, O / L);
        } else {
            const size_t row = h * p.pmax + u.part;
            store_agent(p.part_acc + row * D + d, O);
            if (d == 0) {
                store_agent(p.part_ml + row * 2, M);
                store_agent(p.part_ml + row * 2 + 1, L);
            }
        }
    }
    if (u.nparts == 1) return;

    __shared__ int last;
    // Every thread's partial stores have reached the coherence point before
    // the workgroup's arrival is counted.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        int* cnt = p.counters + (size_t)u.s * p.n_kv + u.kvh;
        const int before = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = (before == u.nparts - 1);
        // every other partition has arrived: re-arm the counter for the next call
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;
    merge_partials<D, F32OUT>(p, u.s, u.kvh, u.nparts);
}

}  // namespace pa
