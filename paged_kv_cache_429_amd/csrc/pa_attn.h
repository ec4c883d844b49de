// Building blocks shared by the decode and prefill kernels: the MFMA tile
// loaders / dequantisers for each KV format, the fp32 VALU wave loop and the
// log-sum-exp epilogue.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

// No floating-point contraction in the attention arithmetic: the same
// source expression must round the same way wherever it is inlined (the
// shared-prefix and per-sequence paths must agree bit for bit, and what the
// compiler can prove about a mask would otherwise decide whether a multiply
// and an add fuse).
#pragma clang fp contract(off)

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

// slot0: partial slots before this unit's partitions (the prefix pass's);
// partition `part` stores its partial in slot slot0 + part. lo: first
// attended token (the sliding window's start, else 0).
struct Unit {
    int s, kvh, part, ctx, nblk, nparts, b_begin, b_end, slot0, lo;
};

// Block ids of a partition, spread over its four waves. Wave w visits the
// pairs w, w + 4, w + 8, ..., so lane 2n + e of its id register holds the id
// of block 2 (w + 4n) + e of the partition: 64 lanes cover the wave's share
// of up to 256 blocks. trow is the sequence's row of the table array
// `tables`. Blocks at or past nb read as 0; ids outside the pool read as 0
// and are recorded (never dereferenced past the pool).
__device__ __forceinline__ int wave_id_slot() {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    return 2 * (w + kWaves * (lane >> 1)) + (lane & 1);
}
// The table entries of load_wave_ids as stored (unchecked; 0 past nb).
__device__ __forceinline__ int load_wave_ids_raw(const int32_t* trow, int first, int nb) {
    const int j = wave_id_slot();
    return j < nb ? trow[first + j] : 0;
}
// Entries of load_wave_ids_raw(trow, first, >= nb) checked against the pool
// for the nb blocks the partition uses (0 past them).
__device__ __forceinline__ int check_wave_ids(int raw, const int32_t* tables, const int32_t* trow, int first, int nb,
                                              int num_blocks) {
    const int j = wave_id_slot();
    return j < nb ? checked_id(raw, (long)(trow - tables) + first + j, num_blocks) : 0;
}
__device__ __forceinline__ int load_wave_ids(const int32_t* tables, const int32_t* trow, int first, int nb,
                                             int num_blocks) {
    return check_wave_ids(load_wave_ids_raw(trow, first, nb), tables, trow, first, nb, num_blocks);
}

// Id of block e (0 or 1) of pair k, one of this wave's pairs (k = w + 4n,
// wave-uniform), from the register load_wave_ids filled.
__device__ __forceinline__ int pair_id(int ids, int k, int e) {
    return readlane(ids, 2 * (k / kWaves) + e);
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
        if (FMT == FMT_I8 || FMT == FMT_F8) return 64 * (kk >> 1) + 16 * q + 8 * (kk & 1);
        return (D == 128 ? 32 : 16) * q + 8 * kk;  // int4
    }

    struct KRaw { uint32_t w[KDW]; };
    struct VRaw { uint32_t w[NB * VDW]; };

    // Tile loads are nontemporal by default: decode streams a private tile
    // once, and the streaming hint lifts the 4 KiB-tile gather rate on gfx950
    // by ~12%. Tiles that several workgroups read (shared prefix blocks) are
    // loaded with the default, cache-friendly policy. (The prefill kernel
    // calls the same loaders on LDS, where the hint has no effect.)
    template <bool NT, typename T>
    __device__ static __forceinline__ T ld(const T* a) {
        if constexpr (NT) {
            return __builtin_nontemporal_load(a);
        } else {
            return *a;
        }
    }

    template <bool NT = true>
    __device__ static __forceinline__ void load_k(const uint8_t* tile, int lane, KRaw& r) {
        if (KDW >= 4) {
#pragma unroll
            for (int u = 0; u < KDW / 4; ++u) {
                u32x4 v = ld<NT>(reinterpret_cast<const u32x4*>(tile + u * 1024 + lane * 16));
                r.w[4 * u + 0] = v[0];
                r.w[4 * u + 1] = v[1];
                r.w[4 * u + 2] = v[2];
                r.w[4 * u + 3] = v[3];
            }
        } else {  // int4, d = 64: half a 16-byte chunk per lane
            const int t = lane & 15, q = lane >> 4;
            u32x2 v = ld<NT>(reinterpret_cast<const u32x2*>(tile + (q >> 1) * 256 + t * 16 + (q & 1) * 8));
            r.w[0] = v[0];
            r.w[1] = v[1];
        }
    }

    // The decode path takes int8 / int4 codes offset by kOff = 128 / 136 (a
    // few ALU ops per element instead of an exact signed widening); the
    // scores subtract kOff * sum(q) and the accumulator kOff * sum(P), both
    // in fp32.
    static constexpr bool kOffset = (FMT == FMT_I4 || FMT == FMT_I8);
    static constexpr float kOff = (FMT == FMT_I4) ? 136.f : 128.f;
    static constexpr uint32_t kOffBf16 = (FMT == FMT_I4) ? 0x4308u : 0x4300u;  // kOff as bf16
    // int4 decode operands come with each group of eight k in the order
    // 0, 2, 4, 6, 1, 3, 5, 7 (i4x8_to_bf16x8_off136_eo); Q and P follow it
    static constexpr bool kEvenOdd = (FMT == FMT_I4);

    __device__ static __forceinline__ u32x4 k_operand_dec(const KRaw& r, int kk) {
        if constexpr (FMT == FMT_I4) {
            return i4x8_to_bf16x8_off136_eo(r.w[kk]);
        } else if constexpr (FMT == FMT_I8) {
            const u32x2 lo = i8x4_to_bf16x4_off128(r.w[2 * kk]);
            const u32x2 hi = i8x4_to_bf16x4_off128(r.w[2 * kk + 1]);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
            return k_operand(r, kk);
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
        } else if (FMT == FMT_F8) {
            const u32x2 lo = f8x4_to_bf16x4(r.w[2 * kk]);
            const u32x2 hi = f8x4_to_bf16x4(r.w[2 * kk + 1]);
            a[0] = lo[0];
            a[1] = lo[1];
            a[2] = hi[0];
            a[3] = hi[1];
        } else {
            a = i4x8_to_bf16x8(r.w[kk]);
        }
        return a;
    }

    template <bool NT = true>
    __device__ static __forceinline__ void load_v(const uint8_t* tile, int lane, VRaw& r) {
        const int l16 = lane & 15, q = lane >> 4;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int d = nb * 16 + l16;
            if (FMT == FMT_BF16) {
                u32x2 v = ld<NT>(reinterpret_cast<const u32x2*>(tile + d * 32 + q * 8));
                r.w[2 * nb] = v[0];
                r.w[2 * nb + 1] = v[1];
            } else if (FMT == FMT_I8 || FMT == FMT_F8) {
                r.w[nb] = ld<NT>(reinterpret_cast<const uint32_t*>(tile + d * 16 + q * 4));
            } else {  // int4: tokens 4q..4q+3 of dim d, in the 8-token piece (d % 16, q / 2, nb)
                r.w[nb] = ld<NT>(reinterpret_cast<const uint16_t*>(tile + ((l16 * 2 + q / 2) * NB + nb) * 4 +
                                                                   (q % 2) * 2));
            }
        }
    }

    // V operand of a pair for the decode P.V product: lane (l16, q) holds,
    // for dim row nb*16 + l16, the 8 consecutive tokens 8 (q % 2) .. + 7 of
    // the pair's block q / 2 -- one contiguous run of a V tile row (16 or 8
    // bytes for bf16 and int8 / fp8, so each load instruction moves 1 KiB or
    // 512 B). An int4 tile keeps the NB 4-byte runs a lane needs next to each
    // other, so it loads all of them as 4 NB contiguous bytes.
    static constexpr int VPDW = (FMT == FMT_BF16) ? 4 : (FMT == FMT_I8 || FMT == FMT_F8 ? 2 : 1);  // dwords per nb
    struct VPairRaw { uint32_t w[NB * VPDW]; };

    template <bool NT = true>
    __device__ static __forceinline__ void load_v_pair(const uint8_t* tile0, const uint8_t* tile1, int lane,
                                                       VPairRaw& r) {
        const int l16 = lane & 15, q = lane >> 4;
        const uint8_t* t = (q < 2) ? tile0 : tile1;
        constexpr int ROW = 16 * BITS / 8;  // bytes of a V tile row (16 tokens of one dim)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint8_t* a = t + (nb * 16 + l16) * ROW + (q & 1) * (ROW / 2);
            if (FMT == FMT_BF16) {
                const u32x4 v = ld<NT>(reinterpret_cast<const u32x4*>(a));
                r.w[4 * nb] = v[0];
                r.w[4 * nb + 1] = v[1];
                r.w[4 * nb + 2] = v[2];
                r.w[4 * nb + 3] = v[3];
            } else if (FMT == FMT_I8 || FMT == FMT_F8) {
                const u32x2 v = ld<NT>(reinterpret_cast<const u32x2*>(a));
                r.w[2 * nb] = v[0];
                r.w[2 * nb + 1] = v[1];
            }
        }
        if constexpr (FMT == FMT_I4) {  // the lane's NB runs: piece (l16, q % 2) of the tile
            const uint8_t* a = t + (l16 * 2 + (q & 1)) * NB * 4;
#pragma unroll
            for (int u = 0; u < NB / 4; ++u) {
                const u32x4 v = ld<NT>(reinterpret_cast<const u32x4*>(a + 16 * u));
                r.w[4 * u + 0] = v[0];
                r.w[4 * u + 1] = v[1];
                r.w[4 * u + 2] = v[2];
                r.w[4 * u + 3] = v[3];
            }
        }
    }

    // bf16 operand (8 tokens) of dim block nb; int8 / int4 come offset by kOff
    __device__ static __forceinline__ u32x4 v_pair_op(const VPairRaw& r, int nb) {
        u32x4 a;
        if (FMT == FMT_BF16) {
            a[0] = r.w[4 * nb];
            a[1] = r.w[4 * nb + 1];
            a[2] = r.w[4 * nb + 2];
            a[3] = r.w[4 * nb + 3];
        } else if (FMT == FMT_F8) {
            const u32x2 lo = f8x4_to_bf16x4(r.w[2 * nb]);
            const u32x2 hi = f8x4_to_bf16x4(r.w[2 * nb + 1]);
            a[0] = lo[0];
            a[1] = lo[1];
            a[2] = hi[0];
            a[3] = hi[1];
        } else if (FMT == FMT_I8) {  // offset by kOff (see k_operand_dec)
            const u32x2 lo = i8x4_to_bf16x4_off128(r.w[2 * nb]);
            const u32x2 hi = i8x4_to_bf16x4_off128(r.w[2 * nb + 1]);
            a[0] = lo[0];
            a[1] = lo[1];
            a[2] = hi[0];
            a[3] = hi[1];
        } else {
            a = i4x8_to_bf16x8_off136_eo(r.w[nb]);  // offset by kOff, even-odd order (see k_operand_dec)
        }
        return a;
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
        } else if (FMT == FMT_F8) {
            return f8x4_to_bf16x4(r.w[nb]);
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
    typename Mfma<D, FMT>::VPairRaw v;
    float s0, s1;
};

// Online-softmax state of the 16 MFMA columns of one wave: running max m and
// sum l (log2 units; lane group q holds its partial sum) and the
// unnormalised O^T accumulator.
template <int D>
struct ColState {
    float m, l;
    f32x4 acc[D / 16];
    // offset formats: kOff * sum(P) of the lane's column (every element; an
    // MFMA of a constant kOff operand with the P operands), rescaled with acc
    f32x4 corr;
};

template <int D>
__device__ __forceinline__ void col_init(ColState<D>& c) {
    c.m = kNegInf;
    c.l = 0.f;
    c.corr = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) c.acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Every step below acts on each of the 16 columns independently (an MFMA
// output element depends only on its own column of the B operand, and the
// reductions run over the lane groups of one column), so a column's result
// does not depend on what the other columns hold. The shared-prefix path
// relies on this to reproduce the per-sequence path bit for bit.

// S^T of a pair for the 16 query columns of qop: s0 holds tokens 4q..4q+3
// of the first block, s1 those of the second.
template <int D, int FMT>
__device__ __forceinline__ void pair_scores(const KHalf<D, FMT>& r, const u32x4* qop, f32x4& s0, f32x4& s1) {
    using M = Mfma<D, FMT>;
    s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < M::KSTEPS; ++kk) {
        s0 = mfma_16x16x32(M::k_operand_dec(r.k0, kk), qop[kk], s0);
        s1 = mfma_16x16x32(M::k_operand_dec(r.k1, kk), qop[kk], s1);
    }
}

// Scores in log2 units (c0, c1 fold 1/sqrt(d), log2 e and the K scales),
// masked by select: tokens at or past ctx or before lo (a sliding window's
// start), and a missing second block, get -inf. tok0 is the lane's first
// token (pair start + 4q).
__device__ __forceinline__ void scale_mask(const f32x4& s0, const f32x4& s1, float c0, float c1, int tok0, int ctx,
                                           bool has1, int lo, float* x) {
    const int tok1 = tok0 + kBlock;
    // a pair wholly in context (the usual case; the test is wave-uniform,
    // as tok0 - 4q is) needs no select
    const int t0 = tok0 - 4 * ((threadIdx.x & 63) >> 4);
    if (has1 && t0 >= lo && t0 + 2 * kBlock <= ctx) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = s0[i] * c0;
            x[4 + i] = s1[i] * c1;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = (tok0 + i < ctx && tok0 + i >= lo) ? s0[i] * c0 : kNegInf;
        x[4 + i] = (has1 && tok1 + i < ctx && tok1 + i >= lo) ? s1[i] * c1 : kNegInf;
    }
}

// Online-softmax update of every column with one pair's scores; returns the
// probabilities in pr. A column whose scores are all -inf is left unchanged.
template <int D>
__device__ __forceinline__ void softmax_update(ColState<D>& c, const float* x, float* pr) {
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float mnew = fmaxf(c.m, mx);
    // While a column has seen no finite score its state stays zero (exp2 of
    // -inf - 0); otherwise this is the usual rescale by 2^(m - mnew).
    const float mref = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(c.m - mref);
    c.m = mnew;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(x[i] - mref);
        psum += pr[i];
    }
    c.l = c.l * alpha + psum;
    // alpha is exactly 1 in every column of the wave unless some maximum
    // moved; multiplying by 1 changes nothing, so that common case skips it
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) c.acc[nb] *= alpha;
        c.corr *= alpha;
    }
}

// O^T += V^T P^T for one pair. The k index of the product runs over the
// pair's 32 tokens so that lane group q holds tokens 8 (q % 2) .. + 7 of
// block q / 2 (the V operand is then one contiguous run of a V tile row).
// The probabilities arrive in the S^T layout (lane group q: tokens
// 4q..4q+3 of each block); two cross-row swaps regroup them within each
// column. t0 is the pair's first token; bf16 and fp8 V slots at or past ctx
// (and a missing second block) are zeroed, since their contents may be
// anything (0 * NaN = NaN). Columns with own == false contribute a zero P
// column (their accumulator is unchanged).
template <int D, int FMT>
__device__ __forceinline__ void pv_update(ColState<D>& c, const VHalf<D, FMT>& r, const float* pr, int t0, int ctx,
                                          bool has1, bool own) {
    using M = Mfma<D, FMT>;
    const int q = (threadIdx.x & 63) >> 4;
    // a: block 0 tokens 4q..4q+3, b: block 1 tokens 4q..4q+3 (bf16 pairs)
    uint32_t a0 = pack_bf16x2(pr[0] * r.s0, pr[1] * r.s0);
    uint32_t a1 = pack_bf16x2(pr[2] * r.s0, pr[3] * r.s0);
    uint32_t b0 = pack_bf16x2(pr[4] * r.s1, pr[5] * r.s1);
    uint32_t b1 = pack_bf16x2(pr[6] * r.s1, pr[7] * r.s1);
    if (!own) a0 = a1 = b0 = b1 = 0u;
    // Rows (lane groups) 0..3 of a = a@0..a@3, likewise b. After the 32-lane
    // swap a = [a@0 a@1 b@0 b@1], b = [a@2 a@3 b@2 b@3]; after the 16-lane
    // swap a = [a@0 a@2 b@0 b@2] (first four tokens of the group's run) and
    // b = [a@1 a@3 b@1 b@3] (last four).
    auto regroup = [](uint32_t& x, uint32_t& y) {
        const auto r32 = __builtin_amdgcn_permlane32_swap(x, y, false, false);
        const auto r16 = __builtin_amdgcn_permlane16_swap(r32[0], r32[1], false, false);
        x = r16[0];
        y = r16[1];
    };
    regroup(a0, b0);
    regroup(a1, b1);
    u32x4 pop = {a0, a1, b0, b1};
    if constexpr (M::kEvenOdd) pop = bf16x8_even_odd(pop);
    const int blk = q >> 1;
    const int tok = t0 + kBlock * blk + 8 * (q & 1);  // first token of this lane group's run
    // Integer codes (the offset formats) are finite whatever the pool holds,
    // and the P of a token at or past ctx is exactly 0, so only bf16 and fp8
    // tiles, whose bytes may hold NaN, need the V mask.
    const bool tail = !M::kOffset && (!has1 || t0 + 2 * kBlock > ctx);
    uint32_t msk[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    if (tail) {
        const bool blk_ok = blk == 0 || has1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            msk[w] = (blk_ok && tok + 2 * w < ctx ? 0x0000ffffu : 0u) | (blk_ok && tok + 2 * w + 1 < ctx ? 0xffff0000u : 0u);
        }
    }
    if constexpr (M::kOffset) {  // kOff * the P values exactly as the MFMA sees them
        const uint32_t k2 = M::kOffBf16 * 0x10001u;
        c.corr = mfma_16x16x32(u32x4{k2, k2, k2, k2}, pop, c.corr);
    }
#pragma unroll
    for (int nb = 0; nb < M::NB; ++nb) {
        u32x4 vop = M::v_pair_op(r.v, nb);
        if constexpr (!M::kOffset) {
            vop[0] &= msk[0];
            vop[1] &= msk[1];
            vop[2] &= msk[2];
            vop[3] &= msk[3];
        }
        c.acc[nb] = mfma_16x16x32(vop, pop, c.acc[nb]);
    }
}

// Write one wave's column states to LDS slot `wave` (row sums completed
// over the four lane groups of each column).
template <int D, bool OFFSET = false>
__device__ __forceinline__ void col_to_lds(ColState<D>& c, WaveState<D>& st, int wave) {
    const int lane = threadIdx.x & 63;
    const int g = lane & 15;
    const int q = lane >> 4;
    float l = c.l;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if constexpr (OFFSET) {  // remove the operand offset's share of the accumulator
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) c.acc[nb] -= c.corr[0];
    }
    if (q == 0) {
        st.m[wave][g] = c.m;
        st.l[wave][g] = l;
    }
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st.acc[wave][g][nb * 16 + 4 * q + i] = c.acc[nb][i];
    }
}

template <int D, int FMT, bool NT = true>
__device__ __forceinline__ void issue_k_pair(const DecodeParams& p, int kvh, int i0, int i1, KHalf<D, FMT>& r) {
    using M = Mfma<D, FMT>;
    const int lane = threadIdx.x & 63;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k_pool);
    M::template load_k<NT>(kbase + ((size_t)i0 * p.n_kv + kvh) * M::TILE, lane, r.k0);
    M::template load_k<NT>(kbase + ((size_t)i1 * p.n_kv + kvh) * M::TILE, lane, r.k1);
    r.s0 = r.s1 = 1.f;
    if (is_quant<FMT>()) {
        r.s0 = fp16_bits_to_f32(p.k_scales[(size_t)i0 * p.n_kv + kvh]);
        r.s1 = fp16_bits_to_f32(p.k_scales[(size_t)i1 * p.n_kv + kvh]);
    }
}

template <int D, int FMT, bool NT = true>
__device__ __forceinline__ void issue_v_pair(const DecodeParams& p, int kvh, int i0, int i1, VHalf<D, FMT>& r) {
    using M = Mfma<D, FMT>;
    const int lane = threadIdx.x & 63;
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v_pool);
    M::template load_v_pair<NT>(vbase + ((size_t)i0 * p.n_kv + kvh) * M::TILE,
                                vbase + ((size_t)i1 * p.n_kv + kvh) * M::TILE, lane, r.v);
    r.s0 = r.s1 = 1.f;
    if (is_quant<FMT>()) {
        r.s0 = fp16_bits_to_f32(p.v_scales[(size_t)i0 * p.n_kv + kvh]);
        r.s1 = fp16_bits_to_f32(p.v_scales[(size_t)i1 * p.n_kv + kvh]);
    }
}

// kOff * (sum of the column's Q^T operand values) for the offset formats,
// else 0: the score correction of offset K codes.
template <int D, int FMT>
__device__ __forceinline__ float q_offset(const u32x4* qop) {
    using M = Mfma<D, FMT>;
    if constexpr (!M::kOffset) {
        return 0.f;
    } else {
        float sum = 0.f;
#pragma unroll
        for (int kk = 0; kk < M::KSTEPS; ++kk) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sum += __uint_as_float(qop[kk][e] << 16);
                sum += __uint_as_float(qop[kk][e] & 0xffff0000u);
            }
        }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        return M::kOff * sum;
    }
}

// Q^T operand of column `col` (query head qh of sequence s), eight dims per
// k-step; zero for an unused column.
template <int D, int FMT>
__device__ __forceinline__ void load_qop(const DecodeParams& p, int s, int qh, bool used, u32x4* qop) {
    using M = Mfma<D, FMT>;
    const int q = (threadIdx.x & 63) >> 4;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)s * p.n_heads + qh) * D;
#pragma unroll
    for (int kk = 0; kk < M::KSTEPS; ++kk) {
        qop[kk] = used ? *reinterpret_cast<const u32x4*>(qrow + M::dbase(kk, q)) : u32x4{0u, 0u, 0u, 0u};
        if constexpr (M::kEvenOdd) qop[kk] = bf16x8_even_odd(qop[kk]);
    }
}

// Software-pipelined run of pairs k, k + 4, ... of one wave (pair k must
// exist; the run continues while more(next) holds). K of the next pair loads
// during this pair's softmax and P.V, V of the next pair during its Q.K; the
// last pair of the run is peeled off so that every load in the loop is
// unconditional and the wait before each use covers only the half it reads.
//   ids(k, i0, i1)          physical ids of the pair's blocks
//   geo(k, t0, ctx, has1)   first token, the context that masks it, and
//                           whether its second block exists
// NT selects the streaming load policy; lanes with own == false (columns of
// another sequence) see -inf scores and a zero P column, which leave their
// state unchanged. Returns the first pair after the run.
template <int D, int FMT, bool NT, typename Ids, typename More, typename Geo>
__device__ __forceinline__ int pair_run(const DecodeParams& p, int kvh, const u32x4* qop, ColState<D>& cs, int k,
                                        Ids ids, More more, Geo geo, bool own = true, int lo = 0) {
    const int q = (threadIdx.x & 63) >> 4;
    const float qoff = q_offset<D, FMT>(qop);
    KHalf<D, FMT> kr;
    VHalf<D, FMT> vr;
    auto step = [&](int kk, bool prefetch) {
        int t0, ctx;
        bool has1;
        geo(kk, t0, ctx, has1);
        f32x4 s0, s1;
        pair_scores<D, FMT>(kr, qop, s0, s1);
        // take the K scales before the prefetch replaces them
        const float c0 = p.scale_log2 * kr.s0;
        const float c1 = p.scale_log2 * kr.s1;
        int n0 = 0, n1 = 0;
        if (prefetch) {
            ids(kk + kWaves, n0, n1);
            issue_k_pair<D, FMT, NT>(p, kvh, n0, n1, kr);
        }
        float x[8], pr[8];
        if constexpr (Mfma<D, FMT>::kOffset) {
            s0 -= qoff;
            s1 -= qoff;
        }
        scale_mask(s0, s1, c0, c1, t0 + 4 * q, ctx, has1, lo, x);
        if (!own) {  // a column of another sequence: no update
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = kNegInf;
        }
        softmax_update(cs, x, pr);
        pv_update<D, FMT>(cs, vr, pr, t0, ctx, has1, own);
        if (prefetch) issue_v_pair<D, FMT, NT>(p, kvh, n0, n1, vr);
    };
    int i0, i1;
    ids(k, i0, i1);
    issue_k_pair<D, FMT, NT>(p, kvh, i0, i1, kr);
    issue_v_pair<D, FMT, NT>(p, kvh, i0, i1, vr);
    for (; more(k + kWaves); k += kWaves) step(k, true);
    step(k, false);
    return k + kWaves;
}

// Pairs whose loads are in flight ahead of the one being computed in the
// per-sequence path: two for int4, whose pairs are small (4 KiB), so that a
// CU keeps more bytes in flight; one for bf16 and int8 (int8 runs out of
// registers at two). The prefetch distance changes when a pair's loads are
// issued, never its arithmetic.
template <int FMT>
constexpr int prefetch_pairs() {
    return FMT == FMT_I4 ? 2 : 1;
}

// pair_run with two pairs in flight: the n >= 1 pairs k, k + 4, ...,
// k + 4 (n - 1) of one wave. The loads of pair i + PD (PD = 1 or 2) go out while pair
// i is computed: its K once pair i's scores are taken, its V once pair i's
// P.V is done, into the register slot pair i used. Steady-state loads are
// unconditional and the last pairs are peeled off, so the wait before each
// use covers only the half it reads.
//   ids(k, i0, i1)          physical ids of the pair's blocks
//   geo(k, t0, ctx, has1)   first token, the context that masks it, and
//                           whether its second block exists
// NT selects the streaming load policy; lanes with own == false (columns of
// another sequence) see -inf scores and a zero P column, which leave their
// state unchanged. Returns the first pair after the run.
template <int D, int FMT, bool NT, int PD, typename Ids, typename Geo>
__device__ __forceinline__ int pair_run_deep(const DecodeParams& p, int kvh, const u32x4* qop, ColState<D>& cs,
                                             int k, int n, Ids ids, Geo geo, bool own = true, int lo = 0) {
    static_assert(PD == 1 || PD == 2, "prefetch distance");
    const int q = (threadIdx.x & 63) >> 4;
    const float qoff = q_offset<D, FMT>(qop);
    KHalf<D, FMT> kr[PD];
    VHalf<D, FMT> vr[PD];
    auto pair_of = [&](int i) { return k + i * kWaves; };
    // pair i into register slot SLOT
    auto issue = [&](auto slot_tag, int i) {
        constexpr int SLOT = decltype(slot_tag)::value;
        int i0, i1;
        ids(pair_of(i), i0, i1);
        issue_k_pair<D, FMT, NT>(p, kvh, i0, i1, kr[SLOT]);
        issue_v_pair<D, FMT, NT>(p, kvh, i0, i1, vr[SLOT]);
    };
    // pair i from slot SLOT; if PREFETCH, pair pf goes into the same slot
    auto step = [&](auto slot_tag, auto prefetch_tag, int i, int pf) {
        constexpr int SLOT = decltype(slot_tag)::value;
        constexpr bool PREFETCH = decltype(prefetch_tag)::value;
        int t0, ctx;
        bool has1;
        geo(pair_of(i), t0, ctx, has1);
        f32x4 s0, s1;
        pair_scores<D, FMT>(kr[SLOT], qop, s0, s1);
        // take the K scales before the prefetch replaces them
        const float c0 = p.scale_log2 * kr[SLOT].s0;
        const float c1 = p.scale_log2 * kr[SLOT].s1;
        int n0 = 0, n1 = 0;
        if (PREFETCH) {
            ids(pair_of(pf), n0, n1);
            issue_k_pair<D, FMT, NT>(p, kvh, n0, n1, kr[SLOT]);
        }
        float x[8], pr[8];
        if constexpr (Mfma<D, FMT>::kOffset) {
            s0 -= qoff;
            s1 -= qoff;
        }
        scale_mask(s0, s1, c0, c1, t0 + 4 * q, ctx, has1, lo, x);
        if (!own) {  // a column of another sequence: no update
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = kNegInf;
        }
        softmax_update(cs, x, pr);
        pv_update<D, FMT>(cs, vr[SLOT], pr, t0, ctx, has1, own);
        if (PREFETCH) issue_v_pair<D, FMT, NT>(p, kvh, n0, n1, vr[SLOT]);
    };
    constexpr std::integral_constant<int, 0> s0_{};
    constexpr std::integral_constant<int, PD - 1> s1_{};
    constexpr std::true_type yes{};
    constexpr std::false_type no{};
    if constexpr (PD == 1) {
        issue(s0_, 0);
        int i = 0;
        for (; i + 1 < n; ++i) step(s0_, yes, i, i + 1);
        step(s0_, no, i, 0);
    } else {
        issue(s0_, 0);
        if (n > 1) issue(s1_, 1);
        int i = 0;
        for (; i + 3 < n; i += 2) {
            step(s0_, yes, i, i + 2);
            step(s1_, yes, i + 1, i + 3);
        }
        // one to three pairs left
        if (i + 2 < n) {
            step(s0_, yes, i, i + 2);
            step(s1_, no, i + 1, 0);
            step(s0_, no, i + 2, 0);
        } else if (i + 1 < n) {
            step(s0_, no, i, 0);
            step(s1_, no, i + 1, 0);
        } else {
            step(s0_, no, i, 0);
        }
    }
    return k + n * kWaves;
}

// One wave of a (sequence, KV head, partition) workgroup: pairs wave,
// wave + 4, ... of the partition, the G query heads of the KV head in
// columns 0..G-1.
template <int D, int FMT>
__device__ __forceinline__ void mfma_wave(const DecodeParams& p, const Unit& u, int wave_ids, WaveState<D>& st) {
    using M = Mfma<D, FMT>;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane & 15;

    u32x4 qop[M::KSTEPS];
    load_qop<D, FMT>(p, u.s, u.kvh * p.group + g, g < p.group, qop);
    ColState<D> cs;
    col_init(cs);

    const int nb_part = u.b_end - u.b_begin;
    const int npairs = (nb_part + 1) >> 1;
    if (wave < npairs) {
        // a missing second block repeats the first, which is then masked out
        auto ids = [&](int k, int& i0, int& i1) {
            i0 = pair_id(wave_ids, k, 0);
            i1 = (2 * k + 1) < nb_part ? pair_id(wave_ids, k, 1) : i0;
        };
        auto geo = [&](int k, int& t0, int& ctx, bool& has1) {
            t0 = (u.b_begin + 2 * k) * kBlock;
            ctx = u.ctx;
            has1 = 2 * k + 1 < nb_part;
        };
        if constexpr (prefetch_pairs<FMT>() == 2) {
            pair_run_deep<D, FMT, true, 2>(p, u.kvh, qop, cs, wave, (npairs - wave + kWaves - 1) / kWaves, ids, geo,
                                           true, u.lo);
        } else {
            pair_run<D, FMT, true>(p, u.kvh, qop, cs, wave, ids, [&](int k) { return k < npairs; }, geo, true, u.lo);
        }
    }
    col_to_lds<D, Mfma<D, FMT>::kOffset>(cs, st, wave);
}

// -----------------------------------------------------------------------------
// fp32 VALU wave loop (lane = (token t, dim quarter qd) for scores; lane = dim
// for the accumulator).
// -----------------------------------------------------------------------------
// Physical id of block (b_begin + j) for j in a 64-block window starting at
// `base`: lane l holds the id of block base + l; out-of-range ids become 0.
__device__ __forceinline__ int load_ids(const int32_t* tables, const int32_t* trow, int first, int count,
                                        int num_blocks) {
    const int lane = threadIdx.x & 63;
    int id = 0;
    if (lane < count) id = checked_id(trow[first + lane], (long)(trow - tables) + first + lane, num_blocks);
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
            my_id = load_ids(p.tables, trow, u.b_begin + (window << 6), min(64, nb_part - (window << 6)),
                             p.num_blocks);
        }
        const int id = readlane(my_id, j & 63);
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
        const bool valid = tok < u.ctx && tok >= u.lo;
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

// Log-sum-exp merge of the partials of (sequence s, KV head kvh), m and l in
// log2 units:
//   M = max_p m_p,  w_p = 2^(m_p - M),  o = (sum_p w_p acc_p) / (sum_p w_p l_p)
// with both sums taken in partition order.
// First every (head, partition) (max, sum) pair is fetched at once into LDS
// scratch `lw` and turned into weights; then each thread fetches its
// outputs' accumulators kChunk partitions at a time with independent loads,
// so a merge costs two or three memory round trips, not one per output.
constexpr int kMergeFloats = 2 * 16 * 256 + 16;  // workgroup scratch: 256 partitions at G = 16

// NT threads take part (a workgroup, or one wave: NT = 64); tid is the
// caller's index among them. lw holds `cap` floats.
template <int NT>
__device__ __forceinline__ void group_sync() {
    if constexpr (NT == kThreads) {
        __syncthreads();
    } else {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

template <int D, bool F32OUT, int NT>
__device__ __forceinline__ void merge_partials(const DecodeParams& p, int s, int kvh, int nparts, float* lw, int cap,
                                               int tid) {
    constexpr int kChunk = 8;
    constexpr int JB = 8;  // outputs per thread per batch
    const int G = p.group;
    const int np = nparts;
    const size_t h0 = (size_t)s * p.n_heads + kvh * G;
    group_sync<NT>();  // lw may still be read by the caller's previous step
    if (2 * G * np + G <= cap) {
        float* lm = lw;               // [G][np] max, then weight
        float* ll = lw + G * np;      // [G][np] sum
        float* lsum = lw + 2 * G * np;  // [G] total weighted sum
        for (int t = tid; t < G * np; t += NT) {
            const int g = t / np, q = t - g * np;
            const float* ml = p.part_ml + ((h0 + g) * p.pslots + q) * 2;
            const float mv = load_agent(ml);
            const float lv = load_agent(ml + 1);
            lm[t] = mv;
            ll[t] = lv;
        }
        group_sync<NT>();
        for (int g = tid; g < G; g += NT) {
            float M = kNegInf;
            for (int q = 0; q < np; ++q) M = fmaxf(M, lm[g * np + q]);
            float L = 0.f;
            for (int q = 0; q < np; ++q) {
                const float e = __builtin_amdgcn_exp2f(lm[g * np + q] - M);
                L += e * ll[g * np + q];
                lm[g * np + q] = e;
            }
            lsum[g] = L;
        }
        group_sync<NT>();
        for (int i0 = 0; i0 < G * D; i0 += JB * NT) {
            float O[JB];
#pragma unroll
            for (int j = 0; j < JB; ++j) O[j] = 0.f;
            for (int q0 = 0; q0 < np; q0 += kChunk) {
                float a[JB][kChunk];
#pragma unroll
                for (int j = 0; j < JB; ++j) {
                    const int idx = i0 + tid + j * NT;
                    const int g = idx / D, d = idx - g * D;
#pragma unroll
                    for (int c = 0; c < kChunk; ++c) {
                        a[j][c] = (idx < G * D && q0 + c < np)
                                      ? load_agent(p.part_acc + ((h0 + g) * p.pslots + q0 + c) * D + d)
                                      : 0.f;
                    }
                }
#pragma unroll
                for (int j = 0; j < JB; ++j) {
                    const int idx = i0 + tid + j * NT;
                    const int g = min(idx / D, G - 1);
#pragma unroll
                    for (int c = 0; c < kChunk; ++c) {
                        if (q0 + c < np) O[j] += lm[g * np + q0 + c] * a[j][c];
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                const int idx = i0 + tid + j * NT;
                if (idx < G * D) store_out<D, F32OUT>(p, h0 * D + idx, O[j] / lsum[idx / D]);
            }
        }
        return;
    }
    // very many partitions: one output per thread at a time, the running
    // (M, L, O) rescaled when a later chunk raises the maximum
    for (int idx = tid; idx < G * D; idx += NT) {
        const int g = idx / D, d = idx - g * D;
        const float* ml = p.part_ml + (h0 + g) * p.pslots * 2;
        const float* acc = p.part_acc + (h0 + g) * p.pslots * D + d;
        float M = kNegInf, L = 0.f, O = 0.f;
        for (int p0 = 0; p0 < np; p0 += kChunk) {
            float mv[kChunk], lv[kChunk], av[kChunk];
#pragma unroll
            for (int c = 0; c < kChunk; ++c) {
                const bool ok = p0 + c < np;
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
        store_out<D, F32OUT>(p, h0 * D + idx, O / L);
    }
}

// Merge the waves' column states held in LDS (in wave order) for columns
// 0..ncols-1 and store each column's result: the output row of a sequence
// with one partial in all, else the partial (max, sum, unnormalised
// accumulator) in slot `slot`. info(col, s, qh, nparts) names the column's
// sequence, query head and number of partials.
template <int D, bool F32OUT, typename Info>
__device__ __forceinline__ void merge_waves_store(const DecodeParams& p, const WaveState<D>& st, int ncols, int slot,
                                                  Info info) {
    for (int idx = threadIdx.x; idx < ncols * D; idx += kThreads) {
        const int col = idx / D, d = idx - col * D;
        float M = st.m[0][col];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, st.m[w][col]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = __builtin_amdgcn_exp2f(st.m[w][col] - M);  // 0 for a wave without blocks
            L += e * st.l[w][col];
            O += e * st.acc[w][col][d];
        }
        int s, qh, nparts;
        info(col, s, qh, nparts);
        const size_t h = (size_t)s * p.n_heads + qh;
        if (nparts == 1) {
            store_out<D, F32OUT>(p, h * D + d, O / L);
        } else {
            const size_t row = h * p.pslots + slot;
            store_agent(p.part_acc + row * D + d, O);
            if (d == 0) {
                store_agent(p.part_ml + row * 2, M);
                store_agent(p.part_ml + row * 2 + 1, L);
            }
        }
    }
}

// Merge the waves' column states in LDS with the np prefix-pass partials of
// the same rows (slots 0..np-1, written by an earlier launch) and store the
// outputs: the path of a unit that is the only decode partition of its
// sequence, which needs no partial of its own.
template <int D, bool F32OUT>
__device__ __forceinline__ void merge_waves_prefix_store(const DecodeParams& p, const Unit& u, const WaveState<D>& st,
                                                         int np) {
    constexpr int kChunk = 4;
    const int G = p.group;
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int col = idx / D, d = idx - col * D;
        const size_t h = (size_t)u.s * p.n_heads + u.kvh * G + col;
        float M = st.m[0][col];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, st.m[w][col]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = __builtin_amdgcn_exp2f(st.m[w][col] - M);  // 0 for a wave without blocks
            L += e * st.l[w][col];
            O += e * st.acc[w][col][d];
        }
        const float* ml = p.part_ml + h * p.pslots * 2;
        const float* acc = p.part_acc + h * p.pslots * D + d;
        for (int q0 = 0; q0 < np; q0 += kChunk) {
            float mv[kChunk], lv[kChunk], av[kChunk];
#pragma unroll
            for (int c = 0; c < kChunk; ++c) {
                const bool ok = q0 + c < np;
                mv[c] = ok ? load_agent(ml + 2 * (q0 + c)) : kNegInf;
                lv[c] = ok ? load_agent(ml + 2 * (q0 + c) + 1) : 0.f;
                av[c] = ok ? load_agent(acc + (size_t)(q0 + c) * D) : 0.f;
            }
            float Mc = M;
#pragma unroll
            for (int c = 0; c < kChunk; ++c) Mc = fmaxf(Mc, mv[c]);
            const float r = __builtin_amdgcn_exp2f(M - Mc);
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

// Count one partition of (sequence s, KV head kvh) as arrived; true for the
// last of its nparts partitions. The arrival word holds the epoch of the
// call that last counted in it and that call's arrivals: a word of another
// epoch (left by an earlier call, complete or not) counts as none. The last
// arrival leaves its epoch with a count of zero, so a replay of the same
// launch (same epoch) starts from zero too. Called by one thread after
// every thread's partial stores have reached the coherence point. The
// compare-and-swap is retried only when another arrival changed the word,
// so it ends after at most nparts tries.
__device__ __forceinline__ bool arrive(const DecodeParams& p, int s, int kvh, int nparts) {
    unsigned long long* w = p.counters + (size_t)s * p.n_kv + kvh;
    const unsigned long long tag = (unsigned long long)p.epoch << 32;
    unsigned long long old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool last;
    while (true) {
        const unsigned long long n = (old >> 32) == (unsigned long long)p.epoch ? (old & 0xffffffffull) : 0ull;
        last = n + 1 >= (unsigned long long)nparts;
        const unsigned long long want = last ? tag : (tag | (n + 1));
        if (__hip_atomic_compare_exchange_strong(w, &old, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            break;
    }
    return last;
}

// Epilogue of a (sequence, KV head, partition) workgroup: merge the waves,
// store, and if this was the last partition of a split sequence to arrive,
// merge all its partials (the prefix pass's first, written by an earlier
// launch, so only this launch's partitions are counted).
// merge_scratch: `cap` floats of LDS, which may alias st.
template <int D, bool F32OUT>
__device__ __forceinline__ void epilogue(const DecodeParams& p, const Unit& u, WaveState<D>& st,
                                         float* merge_scratch, int cap) {
    __syncthreads();
    const int G = p.group;
    const int ntotal = u.slot0 + u.nparts;
    if (u.nparts == 1 && u.slot0 > 0) {
        merge_waves_prefix_store<D, F32OUT>(p, u, st, u.slot0);
        return;
    }
    merge_waves_store<D, F32OUT>(p, st, G, u.slot0 + u.part, [&](int col, int& s, int& qh, int& np) {
        s = u.s;
        qh = u.kvh * G + col;
        np = ntotal;
    });
    if (ntotal == 1) return;

    __shared__ int last;
    // Every thread's partial stores have reached the coherence point before
    // the workgroup's arrival is counted (or, alone, before it merges).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) last = arrive(p, u.s, u.kvh, u.nparts);
    __syncthreads();
    if (!last) return;
    merge_partials<D, F32OUT, kThreads>(p, u.s, u.kvh, ntotal, merge_scratch, cap, threadIdx.x);
}

// -----------------------------------------------------------------------------
// Shared-prefix workgroups ("jovanaeducation" guide a2-inf-2, section "Prefix
// caching"; "KV cache, GQA, paging and continuous batching", section
// "PagedAttention...": sequences with a common prefix point their block
// tables at the same physical blocks).
//
// A group of NS = 16/G consecutive sequences (G = 4 or 8) whose tables name
// the same physical blocks for the first pair of a partition, all full, is
// processed for that (KV head, partition) by the workgroup of the group's
// first sequence, the others' workgroups returning at once: the G query
// heads of the NS sequences fill the 16 MFMA columns (one column set per
// wave). A block pair that every sequence
// of the group shares (same ids, full in every sequence) is loaded once, with
// the cache-friendly policy so that the other groups' workgroups find it in
// L2, and feeds all columns; any other pair is loaded per sequence and feeds
// only that sequence's columns (the others see a zero P column and -inf
// scores, which leave their state unchanged). Pairs are visited in the same
// wave-to-pair order as the per-sequence workgroups, and every column goes
// through the same operations, so a sequence's result does not depend on
// which kind of workgroup computed it: shared blocks give bit-identical
// output to private copies of the same data.
// -----------------------------------------------------------------------------
constexpr int kMaxShareSeqs = 4;  // sequences of a group (16 / G for G = 4 or 8)

// Do the share_n sequences from s0 on all hold the first block pair of
// partition `part`, full, at the same physical ids? Every length and table
// entry is fetched unconditionally (indices clamped into the arrays), so the
// test costs one round of loads rather than a chain of dependent ones.
__device__ __forceinline__ bool group_shares(const DecodeParams& p, int s0, int part) {
    const int b = part * p.pb;
    const int need = (b + 2) * kBlock;
    const int b1 = min(b + 1, p.max_blocks - 1);  // b < max_blocks always
    int ctx[kMaxShareSeqs], e0[kMaxShareSeqs], e1[kMaxShareSeqs];
#pragma unroll
    for (int i = 0; i < kMaxShareSeqs; ++i) {
        const int s = s0 + min(i, p.share_n - 1);
        ctx[i] = p.ctx[s];
        const int32_t* t = p.tables + (size_t)s * p.max_blocks;
        e0[i] = t[b];
        e1[i] = t[b1];
    }
    bool ok = true;
#pragma unroll
    for (int i = 0; i < kMaxShareSeqs; ++i) {
        const int c = min(ctx[i], p.ctx_cap);
        ok = ok && c >= need && num_parts((c + kBlock - 1) / kBlock, p.pb) > part && e0[i] == e0[0] &&
             e1[i] == e1[0];
    }
    return ok;
}

// Block ids of a partition as the shared-group path holds them, one set per
// sequence of the group. bf16 keeps the partition's blocks 0-63 and 64-127
// in two lane registers (partitions of at most 128 blocks): with one
// register per wave its group path no longer fits the register budget of
// three waves per SIMD and spills. The other formats run at two waves per
// SIMD and keep the per-wave layout of the per-sequence path (up to 256).
struct SpanIds {
    int lo, hi;
    __device__ __forceinline__ void load(const int32_t* tables, const int32_t* trow, int first, int nb,
                                         int num_blocks) {
        lo = load_ids(tables, trow, first, min(nb, 64), num_blocks);
        hi = nb > 64 ? load_ids(tables, trow, first + 64, nb - 64, num_blocks) : 0;
    }
    // id of block e of pair k (wave-uniform k, 2k + e < 128)
    __device__ __forceinline__ int get(int k, int e) const {
        const int j = 2 * k + e;
        const int a = readlane(lo, j & 63);
        const int b = readlane(hi, j & 63);
        return j < 64 ? a : b;
    }
};

struct WaveIds {
    int r;
    __device__ __forceinline__ void load(const int32_t* tables, const int32_t* trow, int first, int nb,
                                         int num_blocks) {
        r = load_wave_ids(tables, trow, first, nb, num_blocks);
    }
    __device__ __forceinline__ int get(int k, int e) const { return pair_id(r, k, e); }
};

template <int D, int FMT, int CS, int NS, bool F32OUT>
__device__ __forceinline__ void shared_unit(const DecodeParams& p, int unit, WaveState<D>& st, float* merge_scratch,
                                            int cap) {
    static_assert(CS == 1, "one column set per wave");
    using M = Mfma<D, FMT>;
    const int kvh = unit % p.n_kv;
    const int rest = unit / p.n_kv;
    const int part = rest % p.pmax;
    const int grp = rest / p.pmax;
    const int s0 = grp * NS;
    // a tile whose common run the prefix pass took is planned from the run
    // on, by the per-sequence workgroups alone
    if (p.prefix_ts > 0 && p.plan[s0 / p.prefix_ts] > 0) return;
    if (!group_shares(p, s0, part)) return;

    const int G = p.group;
    const int TPG = 16 / G;  // sequences per column set
    const int b = part * p.pb;
    int ctx[NS], nbp[NS], npairs[NS], nparts[NS];
    int npmax = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        ctx[i] = min(p.ctx[s0 + i], p.ctx_cap);
        const int nblk = (ctx[i] + kBlock - 1) / kBlock;
        nparts[i] = num_parts(nblk, p.pb);
        nbp[i] = part_end(nblk, p.pb, part, nparts[i]) - b;
        npairs[i] = (nbp[i] + 1) >> 1;
        npmax = max(npmax, npairs[i]);
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;
    const int q = lane >> 4;
    const int owner = col / G;  // sequence of this column within its column set
    using Ids = std::conditional_t<FMT == FMT_BF16, SpanIds, WaveIds>;
    Ids my_id[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int32_t* trow = p.tables + (size_t)(s0 + i) * p.max_blocks;
        my_id[i].load(p.tables, trow, b, nbp[i], p.num_blocks);
    }

    u32x4 qop[CS][M::KSTEPS];
    ColState<D> cst[CS];
#pragma unroll
    for (int c = 0; c < CS; ++c) {
        load_qop<D, FMT>(p, s0 + c * TPG + owner, kvh * G + col % G, true, qop[c]);
        col_init(cst[c]);
    }
    // Pair k is shared when every sequence of the group holds both its
    // blocks, full, at the same physical ids.
    auto shared_pair = [&](int k) {
        const int t0 = (b + 2 * k) * kBlock;
        const int a0 = my_id[0].get(k, 0);
        const int a1 = my_id[0].get(k, 1);
        bool sh = true;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (i < NS) {
                sh = sh && t0 + 2 * kBlock <= ctx[i] && my_id[i].get(k, 0) == a0 && my_id[i].get(k, 1) == a1;
            }
        }
        return sh;
    };

    int k = wave;
    if (k < npmax && shared_pair(k)) {
        // the leading run of shared pairs, pipelined like the per-sequence
        // path and with the same per-column operations (every token of a
        // shared pair is in context)
        k = pair_run<D, FMT, false>(
            p, kvh, qop[0], cst[0], k,
            [&](int kk, int& i0, int& i1) {
                i0 = my_id[0].get(kk, 0);
                i1 = my_id[0].get(kk, 1);
            },
            [&](int kk) { return kk < npmax && shared_pair(kk); },
            [&](int kk, int& t0, int& cx, bool& has1) {
                t0 = (b + 2 * kk) * kBlock;
                cx = t0 + 2 * kBlock;
                has1 = true;
            });
    }
    {
        // The rest, sequence by sequence: each sequence's remaining pairs
        // (in order) as one pipelined run that updates only its columns.
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (k < npairs[i]) {
                pair_run<D, FMT, true>(
                    p, kvh, qop[0], cst[0], k,
                    [&](int kk, int& i0, int& i1) {
                        i0 = my_id[i].get(kk, 0);
                        i1 = (2 * kk + 1) < nbp[i] ? my_id[i].get(kk, 1) : i0;
                    },
                    [&](int kk) { return kk < npairs[i]; },
                    [&](int kk, int& t0, int& cx, bool& has1) {
                        t0 = (b + 2 * kk) * kBlock;
                        cx = ctx[i];
                        has1 = 2 * kk + 1 < nbp[i];
                    },
                    owner == i);
            }
        }
    }

    // one column set at a time through the workgroup's LDS state
#pragma unroll
    for (int c = 0; c < CS; ++c) {
        __syncthreads();  // every wave is done with the previous set
        col_to_lds<D, M::kOffset>(cst[c], st, wave);
        __syncthreads();
        merge_waves_store<D, F32OUT>(p, st, 16, part, [&](int cl, int& s, int& qh, int& np) {
            const int i = c * TPG + cl / G;
            s = s0 + i;
            qh = kvh * G + cl % G;
            np = nparts[0];
#pragma unroll
            for (int j = 1; j < NS; ++j) np = (i == j) ? nparts[j] : np;
        });
    }

    __shared__ int last[NS];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x < NS) {
        const int i = threadIdx.x;
        int np = nparts[0];
#pragma unroll
        for (int j = 1; j < NS; ++j) np = (i == j) ? nparts[j] : np;
        last[i] = np > 1 && arrive(p, s0 + i, kvh, np);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        if (i < NS && last[i])
            merge_partials<D, F32OUT, kThreads>(p, s0 + i, kvh, nparts[i], merge_scratch, cap, threadIdx.x);
    }
}

}  // namespace pa
