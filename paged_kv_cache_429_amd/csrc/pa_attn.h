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

    __device__ static __forceinline__ void load_k(const uint8_t* tile, int lane, KRaw& r) {
        if (KDW >= 4) {
#pragma unroll
            for (int u = 0; u < KDW / 4; ++u) {
                u32x4 v = *reinterpret_cast<const u32x4*>(tile + u * 1024 + lane * 16);
                r.w[4 * u + 0] = v[0];
                r.w[4 * u + 1] = v[1];
                r.w[4 * u + 2] = v[2];
                r.w[4 * u + 3] = v[3];
            }
        } else {  // int4, d = 64: half a 16-byte chunk per lane
            const int t = lane & 15, q = lane >> 4;
            u32x2 v = *reinterpret_cast<const u32x2*>(tile + (q >> 1) * 256 + t * 16 + (q & 1) * 8);
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
                u32x2 v = *reinterpret_cast<const u32x2*>(tile + d * 32 + q * 8);
                r.w[2 * nb] = v[0];
                r.w[2 * nb + 1] = v[1];
            } else if (FMT == FMT_I8) {
                r.w[nb] = *reinterpret_cast<const uint32_t*>(tile + d * 16 + q * 4);
            } else {
                r.w[nb] = *reinterpret_cast<const uint16_t*>(tile + d * 8 + q * 2);
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

// Registers of one pair of blocks in flight.
template <int D, int FMT>
struct PairRegs {
    typename Mfma<D, FMT>::KRaw k0, k1;
    typename Mfma<D, FMT>::VRaw v0, v1;
    float ks0, ks1, vs0, vs1;
    bool has1;
};

template <int D, int FMT>
__device__ __forceinline__ void mfma_wave(const DecodeParams& p, const Unit& u, int my_id, WaveState<D>& st) {
    using M = Mfma<D, FMT>;
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

    // issue the loads of pair k (blocks 2k, 2k+1 of the partition)
    auto issue = [&](int k, PairRegs<D, FMT>& r) {
        const int j0 = 2 * k;
        r.has1 = (j0 + 1) < nb_part;
        const int id0 = tile_id(p, my_id, j0);
        const int id1 = r.has1 ? tile_id(p, my_id, j0 + 1) : id0;
        const size_t t0 = ((size_t)id0 * p.n_kv + u.kvh) * M::TILE;
        const size_t t1 = ((size_t)id1 * p.n_kv + u.kvh) * M::TILE;
        M::load_k(kbase + t0, lane, r.k0);
        M::load_k(kbase + t1, lane, r.k1);
        M::load_v(vbase + t0, lane, r.v0);
        M::load_v(vbase + t1, lane, r.v1);
        r.ks0 = r.ks1 = r.vs0 = r.vs1 = 1.f;
        if (FMT == FMT_I8 || FMT == FMT_I4) {
            r.ks0 = fp16_bits_to_f32(p.k_scales[(size_t)id0 * p.n_kv + u.kvh]);
            r.ks1 = fp16_bits_to_f32(p.k_scales[(size_t)id1 * p.n_kv + u.kvh]);
            r.vs0 = fp16_bits_to_f32(p.v_scales[(size_t)id0 * p.n_kv + u.kvh]);
            r.vs1 = fp16_bits_to_f32(p.v_scales[(size_t)id1 * p.n_kv + u.kvh]);
        }
    };

    // online-softmax update with pair k
    auto compute = [&](int k, const PairRegs<D, FMT>& r) {
        const int j0 = 2 * k;
        const bool has1 = r.has1;
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
        f32x4 s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < M::KSTEPS; ++kk) {
            s0 = mfma_16x16x32(M::k_operand(r.k0, kk), qop[kk], s0);
            s1 = mfma_16x16x32(M::k_operand(r.k1, kk), qop[kk], s1);
        }
        // scores of tokens (b0: 4q+i) and (b1: 4q+i), in log2 units; masked by select
        const int tok0 = (u.b_begin + j0) * kBlock + 4 * q;
        const int tok1 = tok0 + kBlock;
        const float c0 = p.scale_log2 * r.ks0;
        const float c1 = p.scale_log2 * r.ks1;
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = (tok0 + i < u.ctx) ? s0[i] * c0 : kNegInf;
            x[4 + i] = (has1 && tok1 + i < u.ctx) ? s1[i] * c1 : kNegInf;
        }
        float mx = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        const float mnew = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        float pr[8];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pr[i] = __builtin_amdgcn_exp2f(x[i] - mnew);
            psum += pr[i];
        }
        l = l * alpha + psum;
#pragma unroll
        for (int nb = 0; nb < M::NB; ++nb) acc[nb] *= alpha;

        u32x4 pop;
        pop[0] = pack_bf16x2(pr[0] * r.vs0, pr[1] * r.vs0);
        pop[1] = pack_bf16x2(pr[2] * r.vs0, pr[3] * r.vs0);
        pop[2] = pack_bf16x2(pr[4] * r.vs1, pr[5] * r.vs1);
        pop[3] = pack_bf16x2(pr[6] * r.vs1, pr[7] * r.vs1);

        // Tokens past the context (and a missing second block) get weight 0,
        // but their V slots may hold anything (0 * NaN = NaN): zero them.
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

    // Two pairs in flight: the loads of the next pair overlap this pair's math.
    PairRegs<D, FMT> ra, rb;
    int k = wave;
    if (k < npairs) issue(k, ra);
    while (k < npairs) {
        const int kn = k + kWaves;
        if (kn < npairs) issue(kn, rb);
        compute(k, ra);
        if (kn >= npairs) break;
        const int kn2 = kn + kWaves;
        if (kn2 < npairs) issue(kn2, ra);
        compute(kn, rb);
        k = kn2;
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
            p.part_acc[row * D + d] = O;
            if (d == 0) {
                p.part_ml[row * 2] = M;
                p.part_ml[row * 2 + 1] = L;
            }
        }
    }
}

}  // namespace pa
