// Cache-side kernels for gfx950: symmetric int8/int4/fp8 quantization of a
// bf16 pool, and scattering new tokens' K/V into their slots.
//
// Quantization ("jovanaeducation" inference guide a2-inf-2, section
// "KV-cache quantization": every key/value is an integer sharing one scale
// with its group). Group = one (block, KV head) tile of 16 slots x d dims:
//   s = fp16_rne(amax / qmax), code = clamp(rint(x / float(s)), -qmax, qmax)
// with IEEE float32 division and round-half-to-even (v_rndne_f32).
// fp8 (OCP e4m3; the pages name fp8 as the usual choice for the cache, "KV
// cache, continuous batching and paged attention", section "The KV cache"):
//   s = fp16_rne(amax / 448), code = e4m3 nearest x / float(s), ties to the
//   even code, saturating at +-448, sign of x kept; all 0 if s is 0 or inf.
//
// Slot writes ("KV cache, continuous batching and paged attention", section
// "The KV cache": each step computes K/V only for the new token and caches
// them) follow the pool layout: K tiles in 16-byte chunks of consecutive dims
// (slot-minor), V tiles transposed (dim-major; int4 in runs of 8 slots of one
// dim, see v_elem).
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// element number of (slot t, dim i) inside a K tile, x elements per 16 bytes
__device__ __forceinline__ int k_elem(int t, int i, int x) { return ((i / x) * 16 + t) * x + i % x; }

// (slot t, dim i) of element number n of a V tile of D dims at CB bits per
// element: i * 16 + t (transposed, dim-major), except int4, whose element
// (t, i) is number (((i % 16) * 2 + t / 8) * (D / 16) + i / 16) * 8 + t % 8:
// runs of 8 tokens of one dim, those a decode lane reads (the same i % 16
// and token half, every dim block) side by side.
template <int D, int CB>
__device__ __forceinline__ void v_elem(int n, int& t, int& i) {
    if constexpr (CB == 4) {
        constexpr int NB = D / 16;
        const int rest = n / (8 * NB);
        i = ((n / 8) % NB) * 16 + rest / 2;
        t = (rest % 2) * 8 + n % 8;
    } else {
        i = n / 16;
        t = n % 16;
    }
}

// e4m3 code of float32 r (finite): magnitudes from 448 up saturate to 448
// (0x7E); below the smallest normal 2^-6 the code is the multiple of 2^-9
// nearest |r| (rint of |r| * 512, exact, 0..8, where 8 is 2^-6's code);
// otherwise r's exponent and mantissa are rounded to 3 mantissa bits, ties
// to even, in integer arithmetic on the float's bits (a carry moves into the
// exponent), and the exponent rebiased from 127 to 7.
__device__ __forceinline__ uint32_t f32_to_e4m3(float r) {
    const uint32_t sign = (__float_as_uint(r) >> 24) & 0x80u;
    const float a = fabsf(r);
    uint32_t mag;
    if (a >= 448.f) {
        mag = 0x7Eu;
    } else if (a < 0.015625f) {
        mag = (uint32_t)__builtin_rintf(a * 512.f);
    } else {
        const uint32_t b = __float_as_uint(a);
        mag = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
    }
    return sign | mag;
}

// Scale of a tile whose largest magnitude is amax: the fp16 value nearest
// amax / qmax (IEEE float32 division, then round to nearest even), with
// qmax 127 / 7 / 448 for BITS 8 / 4 / 0 (fp8). Returns its float32 value;
// *bits gets its fp16 bit pattern; *zero is set when every code of the tile
// is 0 (scale 0, or for fp8 an infinite scale).
template <int BITS>
__device__ __forceinline__ float tile_scale(float amax, uint16_t* bits, bool* zero) {
    constexpr float qmax = BITS == 0 ? 448.f : (BITS == 8) ? 127.f : 7.f;
    const float s32 = amax / qmax;
    const _Float16 s16 = (_Float16)s32;
    const float sf = (float)s16;
    *bits = __builtin_bit_cast(uint16_t, s16);
    *zero = !(sf > 0.f) || (BITS == 0 && __builtin_isinf(sf));
    return sf;
}

// Code of x under the tile scale sf: clamp(rint(x / sf), -qmax, qmax) for
// integer codes, the e4m3 code nearest x / sf for fp8 (BITS 0); 0 if zero.
// x / sf is the correctly rounded float quotient. For integer codes rsf (a
// reciprocal of sf, within one ulp) stands in for the division: for
// |x * rsf| < 128 the product is within 2^-14.6 of x / sf, so when it lies
// more than 2^-12 from every half-integer both round to the same integer;
// otherwise (and for a non-finite product) the quotient itself is taken.
template <int BITS>
__device__ __forceinline__ int quant_code(float x, float sf, float rsf, bool zero) {
    if (zero) return 0;
    if constexpr (BITS == 0) {
        return (int)f32_to_e4m3(x / sf);
    } else {
        constexpr float qmax = (BITS == 8) ? 127.f : 7.f;
        float r = x * rsf;
        const float h = fabsf(r - __builtin_floorf(r) - 0.5f);  // distance to the nearest half-integer
        const bool exact = !(h > 0x1p-12f && fabsf(r) < 128.f);
        if (__builtin_amdgcn_ballot_w64(exact)) {  // rare: the division only where some lane needs it
            const float q = x / sf;
            r = exact ? q : r;
        }
        float c = __builtin_rintf(r);
        c = fminf(fmaxf(c, -qmax), qmax);
        return (int)c;
    }
}

// BITS 8 or 4 (integer codes) or 0 (fp8 e4m3 codes, one byte each). One
// wave per (block, KV head) tile: the bf16 tile comes in with 16-byte loads
// (its largest magnitude taken on the way) and is kept in LDS, where each
// code reads its source element; the codes leave in 16-byte stores.
template <int D, int BITS, int KIND>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ codes,
                                                      uint16_t* __restrict__ scales, const int32_t* __restrict__ ids,
                                                      int n_ids, int num_blocks, int n_kv) {
    constexpr int N = 16 * D;                       // elements of a tile
    constexpr int CB = BITS == 0 ? 8 : BITS;        // bits per code
    constexpr int IN16 = N * 2 / 16;                // 16-byte pieces of the bf16 tile
    constexpr int OUT16 = N * CB / 8 / 16;          // 16-byte pieces of its codes
    __shared__ __attribute__((aligned(16))) uint16_t stage[4][N];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const long tile = (long)blockIdx.x * 4 + w;
    int b = -1, h = 0;
    if (tile < (long)n_ids * n_kv) {
        const int i_id = (int)(tile / n_kv);
        h = (int)(tile % n_kv);
        b = ids ? ids[i_id] : i_id;
        if ((unsigned)b >= (unsigned)num_blocks) b = -1;
    }
    uint16_t* st = stage[w];
    float amax = 0.f;
    if (b >= 0) {
        const u32x4* t = reinterpret_cast<const u32x4*>(src + ((size_t)b * n_kv + h) * N);
        for (int c = lane; c < IN16; c += 64) {
            const u32x4 v = t[c];
            *reinterpret_cast<u32x4*>(st + 8 * c) = v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                amax = fmaxf(amax, fabsf(__uint_as_float(v[e] << 16)));
                amax = fmaxf(amax, fabsf(__uint_as_float(v[e] & 0xffff0000u)));
            }
        }
    }
    __syncthreads();  // the tile is in LDS
    if (b < 0) return;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));

    uint16_t sbits;
    bool zero;
    const float sf = tile_scale<BITS>(amax, &sbits, &zero);
    const float rsf = __builtin_amdgcn_rcpf(sf);
    if (lane == 0) scales[(size_t)b * n_kv + h] = sbits;

    auto code_of = [&](int n) -> uint32_t {
        // element n of the code tile -> (slot, dim) -> element of the bf16 tile
        int tt, ii;
        if (KIND == 0) {
            constexpr int x = 128 / CB;
            const int c = n / (16 * x);
            tt = (n / x) % 16;
            ii = c * x + n % x;
        } else {
            v_elem<D, CB>(n, tt, ii);
        }
        const int se = (KIND == 0) ? k_elem(tt, ii, 8) : ii * 16 + tt;
        return (uint32_t)quant_code<BITS>(bf16_bits_to_f32(st[se]), sf, rsf, zero);
    };

    u32x4* out = reinterpret_cast<u32x4*>(codes + ((size_t)b * n_kv + h) * (N * CB / 8));
    for (int c = lane; c < OUT16; c += 64) {
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t word = 0;
            if (CB == 8) {
#pragma unroll
                for (int k = 0; k < 4; ++k) word |= (code_of(16 * c + 4 * e + k) & 0xffu) << (8 * k);
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) word |= (code_of(32 * c + 8 * e + k) & 0xfu) << (4 * k);
            }
            o[e] = word;
        }
        out[c] = o;
    }
}

template <int D, int BITS, int KIND>
static hipError_t quant_t(const void* src, void* codes, uint16_t* scales, const int32_t* ids, int n_ids,
                          int num_blocks, int n_kv, hipStream_t stream) {
    const long tiles = (long)n_ids * n_kv;
    if (tiles == 0) return hipSuccess;
    const long grid = (tiles + 3) / 4;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((quantize_kernel<D, BITS, KIND>), dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(src), static_cast<uint8_t*>(codes), scales, ids, n_ids,
                       num_blocks, n_kv);
    return hipGetLastError();
}

hipError_t launch_quantize(const void* src, void* codes, uint16_t* scales, const int32_t* block_ids, int n_ids,
                           int num_blocks, int n_kv, int d, int bits, int kind, hipStream_t stream) {
#define PA_Q(DD, BB, KK) \
    if (d == DD && bits == BB && kind == KK) \
        return quant_t<DD, BB, KK>(src, codes, scales, block_ids, n_ids, num_blocks, n_kv, stream);
    PA_Q(128, 8, 0) PA_Q(128, 8, 1) PA_Q(128, 4, 0) PA_Q(128, 4, 1) PA_Q(128, 0, 0) PA_Q(128, 0, 1)
    PA_Q(64, 8, 0) PA_Q(64, 8, 1) PA_Q(64, 4, 0) PA_Q(64, 4, 1) PA_Q(64, 0, 0) PA_Q(64, 0, 1)
#undef PA_Q
    return hipErrorInvalidValue;
}

// Scatter of source rows to arbitrary slots. One wave per 64 source tokens
// and one KV head. A token is a run head when its slot is the first of a
// block and the next 15 tokens hold that block's next 15 slots in order
// (rows written in order, as a prompt's are): the head's wave writes the
// block's whole K and V tiles with 16-byte stores, K chunk by chunk and V
// transposed through LDS. The 15 tokens after a head are left to it. Every
// other token in range is written by the whole wave: its K row as 16-byte
// chunks, its V row element by element (a V tile is dim-major, so one
// token's elements are 16 slots apart).
template <int D, int EB>
__global__ __launch_bounds__(256) void kv_write_kernel(const uint8_t* __restrict__ ksrc,
                                                      const uint8_t* __restrict__ vsrc,
                                                      const int64_t* __restrict__ slots, int ntok,
                                                      uint8_t* __restrict__ kpool, uint8_t* __restrict__ vpool,
                                                      int num_blocks, int n_kv) {
    constexpr int ROW = D * EB;        // bytes of one token's row of one head
    constexpr int CH = ROW / 16;       // its 16-byte chunks
    constexpr int TILE = 16 * ROW;     // bytes of a (block, head) tile
    constexpr int PER = 16 / EB;       // elements per 16-byte piece
    constexpr int PIECES = TILE / 16;  // 16-byte pieces of a tile
    __shared__ __attribute__((aligned(16))) uint8_t stage[4][TILE];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const long t0 = ((long)blockIdx.x * 4 + w) * 64;
    const int h = blockIdx.y;
    if (t0 >= ntok) return;  // (no workgroup barrier below)
    const int64_t nslots = (int64_t)num_blocks * 16;
    auto slot_of = [&](long t) -> int64_t {  // -1: no token, or a slot that is skipped
        if (t < 0 || t >= ntok) return -1;
        const int64_t s = slots[t];
        return (s >= 0 && s < nslots) ? s : -1;
    };
    auto is_head = [&](long t) -> bool {
        const int64_t s = slot_of(t);
        if (s < 0 || (s & 15) != 0) return false;
        for (int j = 1; j < 16; ++j) {
            if (slot_of(t + j) != s + j) return false;
        }
        return true;
    };
    const int64_t s_me = slot_of(t0 + lane);
    const uint64_t heads = __builtin_amdgcn_ballot_w64(is_head(t0 + lane));              // bit l: token t0 + l
    const uint64_t prev = __builtin_amdgcn_ballot_w64(lane < 15 && is_head(t0 - 15 + lane));  // bit l: t0 - 15 + l
    bool covered = false;  // a head lies 1..15 tokens before this lane's token
    for (int j = 1; j < 16; ++j) {
        const int d = lane - j;
        covered = covered || (d >= 0 ? ((heads >> d) & 1) : ((prev >> (d + 15)) & 1));
    }
    auto shfl_slot = [&](int l) -> int64_t {
        const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)s_me, l);
        const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)((uint64_t)s_me >> 32), l);
        return (int64_t)(((uint64_t)hi << 32) | lo);
    };
    auto src_row = [&](const uint8_t* src, long t) { return src + ((size_t)t * n_kv + h) * ROW; };

    for (uint64_t hm = heads; hm; hm &= hm - 1) {  // whole tiles
        const int l = __builtin_ctzll(hm);
        const long th = t0 + l;
        const size_t tile = ((size_t)(shfl_slot(l) / 16) * n_kv + h) * TILE;
        if (ksrc) {  // tile chunk c of slot t is chunk c of row th + t
            for (int j = lane; j < 16 * CH; j += 64) {
                *reinterpret_cast<u32x4*>(kpool + tile + (size_t)j * 16) =
                    *reinterpret_cast<const u32x4*>(src_row(ksrc, th + j % 16) + (j / 16) * 16);
            }
        }
        if (vsrc) {
            uint8_t* st = stage[w];
            for (int j = lane; j < 16 * CH; j += 64) {  // row t at st + t * ROW
                *reinterpret_cast<u32x4*>(st + (j / CH) * ROW + (j % CH) * 16) =
                    *reinterpret_cast<const u32x4*>(src_row(vsrc, th + j / CH) + (j % CH) * 16);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            for (int q = lane; q < PIECES; q += 64) {  // piece q: dim q / (16 / PER), slots from tf on
                const int i = q / (16 / PER);
                const int tf = (q % (16 / PER)) * PER;
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (EB == 2) {
                        const uint32_t lo = *reinterpret_cast<const uint16_t*>(st + (tf + 2 * e) * ROW + i * 2);
                        const uint32_t hi = *reinterpret_cast<const uint16_t*>(st + (tf + 2 * e + 1) * ROW + i * 2);
                        o[e] = lo | (hi << 16);
                    } else {
                        o[e] = *reinterpret_cast<const uint32_t*>(st + (tf + e) * ROW + i * 4);
                    }
                }
                *reinterpret_cast<u32x4*>(vpool + tile + (size_t)q * 16) = o;
            }
            __builtin_amdgcn_s_waitcnt(0);  // the stage is read before the next head overwrites it
            __builtin_amdgcn_wave_barrier();
        }
    }

    const bool single = s_me >= 0 && !((heads >> lane) & 1) && !covered;
    for (uint64_t sm = __builtin_amdgcn_ballot_w64(single); sm; sm &= sm - 1) {  // tokens on their own
        const int l = __builtin_ctzll(sm);
        const int64_t s = shfl_slot(l);
        const int t = (int)(s % 16);
        const size_t tile = ((size_t)(s / 16) * n_kv + h) * TILE;
        if (ksrc) {
            for (int c = lane; c < CH; c += 64) {
                *reinterpret_cast<u32x4*>(kpool + tile + (size_t)(c * 16 + t) * 16) =
                    *reinterpret_cast<const u32x4*>(src_row(ksrc, t0 + l) + c * 16);
            }
        }
        if (vsrc) {
            for (int i = lane; i < D; i += 64) {
                uint8_t* dst = vpool + tile + (size_t)(i * 16 + t) * EB;
                if (EB == 2) {
                    *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(src_row(vsrc, t0 + l) + i * 2);
                } else {
                    *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src_row(vsrc, t0 + l) + i * 4);
                }
            }
        }
    }
}

template <int D, int EB>
static hipError_t write_t(const void* k_src, const void* v_src, const int64_t* slots, int ntok, void* kp, void* vp,
                          int num_blocks, int n_kv, hipStream_t stream) {
    if (ntok == 0 || n_kv == 0) return hipSuccess;
    const long grid = ((long)ntok + 255) / 256;
    if (grid > 0x7fffffffL || n_kv > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((kv_write_kernel<D, EB>), dim3((unsigned)grid, (unsigned)n_kv), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(k_src), static_cast<const uint8_t*>(v_src), slots, ntok,
                       static_cast<uint8_t*>(kp), static_cast<uint8_t*>(vp), num_blocks, n_kv);
    return hipGetLastError();
}

hipError_t launch_kv_write(const void* k_src, const void* v_src, const int64_t* slots, int num_tokens,
                           void* k_pool, void* v_pool, int num_blocks, int n_kv, int d, int fmt,
                           hipStream_t stream) {
    const int eb = (fmt == FMT_F32) ? 4 : 2;
    if (d == 128 && eb == 2) return write_t<128, 2>(k_src, v_src, slots, num_tokens, k_pool, v_pool, num_blocks, n_kv, stream);
    if (d == 128 && eb == 4) return write_t<128, 4>(k_src, v_src, slots, num_tokens, k_pool, v_pool, num_blocks, n_kv, stream);
    if (d == 64 && eb == 2) return write_t<64, 2>(k_src, v_src, slots, num_tokens, k_pool, v_pool, num_blocks, n_kv, stream);
    if (d == 64 && eb == 4) return write_t<64, 4>(k_src, v_src, slots, num_tokens, k_pool, v_pool, num_blocks, n_kv, stream);
    return hipErrorInvalidValue;
}

// -----------------------------------------------------------------------------
// Append through the block table. Sequence s's new tokens are its last n_s
// positions, ctx_s - n_s .. ctx_s - 1 (rows cu[s] .. cu[s+1]-1 of the
// source); the token at position t goes to slot t % 16 of physical block
// table[s][t / 16]. One wave per (sequence, touched block, KV head, K or V):
// it assembles the block's tile in LDS as 16 slots x D float32 values (the
// new tokens; for a quantized pool also the block's earlier tokens, kept in
// the sequence's bf16 staging tile, and 0 for the slots past the end), then
// writes the tile in the pool's layout with 16-byte stores. A plain pool gets
// only the new tokens' elements; a quantized pool gets the whole tile's codes
// and its scale, recomputed from every token written so far, and the
// staging tile keeps the new tokens of a block left partly filled.
// -----------------------------------------------------------------------------
struct AppendParams {
    const uint8_t* src[2];   // K, V new rows [total][n_kv][D] (bf16 or f32); null = skip
    uint8_t* pool[2];
    uint16_t* scales[2];     // quantized pools
    uint16_t* stage[2];      // bf16 [num_seqs][n_kv][16][D], quantized pools
    const int32_t* cu;
    const int32_t* ctx;
    const int32_t* tables;
    int max_blocks;
    int num_blocks;
    int n_kv;
    int tiles_per_seq;       // blocks a sequence's new tokens can touch
};

// FMT: FMT_F32 / FMT_BF16 (plain pools of that element type) or FMT_I8 /
// FMT_I4 / FMT_F8 (quantized pools, bf16 source).
template <int D, int FMT>
__global__ __launch_bounds__(64) void kv_append_kernel(AppendParams p) {
    constexpr bool QUANT = is_quant<FMT>();
    constexpr int SEB = FMT == FMT_F32 ? 4 : 2;            // source element bytes
    constexpr int CB = FmtBits<FMT>::v;                    // pool bits per element
    constexpr int BITS = FMT == FMT_F8 ? 0 : CB;           // quant_code selector
    constexpr int TILE = 16 * D * CB / 8;                  // pool bytes of one tile
    constexpr int EPC = 128 / CB;                          // elements per 16-byte pool chunk
    // the tile's values: float32 for plain pools, bf16 bits for quantized
    // ones (whose values are all bf16), which halves the LDS of a workgroup
    using TileT = std::conditional_t<QUANT, uint16_t, float>;
    __shared__ TileT tile[16][D + (QUANT ? 2 : 1)];
    auto tv = [&](int t, int i) -> float {
        if constexpr (QUANT) {
            return bf16_bits_to_f32(tile[t][i]);
        } else {
            return tile[t][i];
        }
    };

    const int lane = threadIdx.x;
    const int kind = blockIdx.x & 1;
    int rest = blockIdx.x >> 1;
    const int kvh = rest % p.n_kv;
    rest /= p.n_kv;
    const int q = rest % p.tiles_per_seq;
    const int s = rest / p.tiles_per_seq;
    const uint8_t* src = p.src[kind];
    if (!src) return;
    const int row0 = p.cu[s];
    const int n = p.cu[s + 1] - row0;
    const int ctx = p.ctx[s];
    const int first = ctx - n;  // first new position
    if (n <= 0 || first < 0) return;
    const int j = first / kBlock + q;  // logical block
    if (j > (ctx - 1) / kBlock) return;
    const long tidx = (long)s * p.max_blocks + j;
    const int phys = p.tables[tidx];
    if ((unsigned)phys >= (unsigned)p.num_blocks) {  // never written through: recorded instead
        if (lane == 0) note_bad_id(tidx, phys);
        return;
    }
    const int lo = max(first - kBlock * j, 0);      // new slots [lo, hi)
    const int hi = min(ctx - kBlock * j, kBlock);
    uint16_t* stage = QUANT ? p.stage[kind] + ((size_t)s * p.n_kv + kvh) * kBlock * D : nullptr;

    // the tile's values: 16-byte pieces of the source rows (or staging)
    constexpr int SPP = 16 / SEB;                           // source elements per piece
    for (int c = lane; c < kBlock * D / SPP; c += 64) {
        const int t = c / (D / SPP);
        const int i0 = (c % (D / SPP)) * SPP;
        float v[SPP];
        if (t >= lo && t < hi) {
            const size_t row = (size_t)row0 + kBlock * j + t - first;
            const u32x4 w = *reinterpret_cast<const u32x4*>(src + ((row * p.n_kv + kvh) * D + i0) * SEB);
#pragma unroll
            for (int e = 0; e < SPP; ++e) {
                v[e] = SEB == 4 ? __uint_as_float(w[e]) : bf16_bits_to_f32((w[e / 2] >> (16 * (e % 2))) & 0xffffu);
            }
        } else if (QUANT && t < lo) {  // written by an earlier call: kept in the staging tile
            const u32x4 w = *reinterpret_cast<const u32x4*>(stage + t * D + i0);
#pragma unroll
            for (int e = 0; e < SPP; ++e) v[e] = bf16_bits_to_f32((w[e / 2] >> (16 * (e % 2))) & 0xffffu);
        } else {
#pragma unroll
            for (int e = 0; e < SPP; ++e) v[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < SPP; ++e) {
            if constexpr (QUANT) {
                tile[t][i0 + e] = (uint16_t)(__float_as_uint(v[e]) >> 16);  // a bf16 value: exact
            } else {
                tile[t][i0 + e] = v[e];
            }
        }
    }
    __syncthreads();

    // (slot, dim) of element number el of the tile in the pool's layout
    auto elem = [&](int el, int& t, int& i) {
        if (kind == 0) {  // K: 16-byte chunks of EPC consecutive dims, slot-minor
            const int ch = el / (16 * EPC);
            t = (el / EPC) % 16;
            i = ch * EPC + el % EPC;
        } else {          // V: transposed (int4: in runs of 8 tokens, see v_elem)
            v_elem<D, CB>(el, t, i);
        }
    };
    uint8_t* out = p.pool[kind] + ((size_t)phys * p.n_kv + kvh) * TILE;

    if constexpr (!QUANT) {
        for (int k = lane; k < TILE / 16; k += 64) {
            u32x4 w;
            int n_new = 0;
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                int t, i;
                elem(k * EPC + e, t, i);
                n_new += (t >= lo && t < hi);
            }
            if (n_new == 0) continue;
            if (n_new == EPC) {
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    int t, i;
                    elem(k * EPC + e, t, i);
                    const float x = tv(t, i);
                    if (SEB == 4) {
                        w[e] = __float_as_uint(x);
                    } else if (e % 2 == 0) {
                        w[e / 2] = __float_as_uint(x) >> 16;
                    } else {
                        w[e / 2] |= __float_as_uint(x) & 0xffff0000u;
                    }
                }
                *reinterpret_cast<u32x4*>(out + (size_t)k * 16) = w;
            } else {  // a chunk shared with slots not written now: its new elements one by one
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    int t, i;
                    elem(k * EPC + e, t, i);
                    if (t < lo || t >= hi) continue;
                    const float x = tv(t, i);
                    if (SEB == 4) {
                        reinterpret_cast<uint32_t*>(out)[k * EPC + e] = __float_as_uint(x);
                    } else {
                        reinterpret_cast<uint16_t*>(out)[k * EPC + e] = (uint16_t)(__float_as_uint(x) >> 16);
                    }
                }
            }
        }
    } else {
        float amax = 0.f;
        for (int e = lane; e < kBlock * D; e += 64) amax = fmaxf(amax, fabsf(tv(e / D, e % D)));
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
        uint16_t sbits;
        bool zero;
        const float sf = tile_scale<BITS>(amax, &sbits, &zero);
        const float rsf = __builtin_amdgcn_rcpf(sf);
        if (lane == 0) p.scales[kind][(size_t)phys * p.n_kv + kvh] = sbits;
        for (int k = lane; k < TILE / 16; k += 64) {
            u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                int t, i;
                elem(k * EPC + e, t, i);
                const uint32_t c = (uint32_t)quant_code<BITS>(tv(t, i), sf, rsf, zero) & ((1u << CB) - 1u);
                w[(e * CB) / 32] |= c << ((e * CB) % 32);
            }
            *reinterpret_cast<u32x4*>(out + (size_t)k * 16) = w;
        }
        // a block left partly filled keeps its new tokens for the next write
        if (j == (ctx - 1) / kBlock && ctx % kBlock != 0) {
            for (int c = lane; c < (hi - lo) * D / 8; c += 64) {
                const int t = lo + c / (D / 8);
                const int i0 = (c % (D / 8)) * 8;
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (uint32_t)tile[t][i0 + 2 * e] | ((uint32_t)tile[t][i0 + 2 * e + 1] << 16);
                *reinterpret_cast<u32x4*>(stage + t * D + i0) = w;
            }
        }
    }
}

template <int D, int FMT>
static hipError_t append_t(const AppendParams& p, int num_seqs, hipStream_t stream) {
    const long grid = (long)num_seqs * p.tiles_per_seq * p.n_kv * 2;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((kv_append_kernel<D, FMT>), dim3((unsigned)grid), dim3(64), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int32_t* cu_new, int max_new,
                            const int32_t* tables, int max_blocks, const int32_t* ctx, void* k_pool, void* v_pool,
                            uint16_t* k_scales, uint16_t* v_scales, void* k_stage, void* v_stage, int num_seqs,
                            int num_blocks, int n_kv, int d, int fmt, hipStream_t stream) {
    AppendParams p{};
    p.src[0] = static_cast<const uint8_t*>(k_new);
    p.src[1] = static_cast<const uint8_t*>(v_new);
    p.pool[0] = static_cast<uint8_t*>(k_pool);
    p.pool[1] = static_cast<uint8_t*>(v_pool);
    p.scales[0] = k_scales;
    p.scales[1] = v_scales;
    p.stage[0] = static_cast<uint16_t*>(k_stage);
    p.stage[1] = static_cast<uint16_t*>(v_stage);
    p.cu = cu_new;
    p.ctx = ctx;
    p.tables = tables;
    p.max_blocks = max_blocks;
    p.num_blocks = num_blocks;
    p.n_kv = n_kv;
    p.tiles_per_seq = (max_new + kBlock - 1) / kBlock + 1;
#define PA_A(DD, FF) \
    if (d == DD && fmt == FF) return append_t<DD, FF>(p, num_seqs, stream);
    PA_A(128, FMT_F32) PA_A(128, FMT_BF16) PA_A(128, FMT_I8) PA_A(128, FMT_I4) PA_A(128, FMT_F8)
    PA_A(64, FMT_F32) PA_A(64, FMT_BF16) PA_A(64, FMT_I8) PA_A(64, FMT_I4) PA_A(64, FMT_F8)
#undef PA_A
    return hipErrorInvalidValue;
}

}  // namespace pa

namespace pa {

// Copy-on-write block copies: workgroup i copies the n_kv tiles of block
// pairs[2i] to block pairs[2i+1] in both pools (bytes = n_kv * tile bytes,
// a multiple of 16) and, when given, the blocks' scales. Pairs naming a
// block outside [0, num_blocks) are skipped.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ kpool, uint8_t* __restrict__ vpool,
                                                         uint16_t* __restrict__ kscales,
                                                         uint16_t* __restrict__ vscales,
                                                         const int32_t* __restrict__ pairs, int num_blocks,
                                                         int n_kv, size_t block_bytes) {
    const int src = pairs[2 * blockIdx.x];
    const int dst = pairs[2 * blockIdx.x + 1];
    if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) return;
    const size_t n16 = block_bytes / 16;
    for (size_t i = threadIdx.x; i < n16; i += 256) {
        if (kpool) {
            reinterpret_cast<u32x4*>(kpool + (size_t)dst * block_bytes)[i] =
                reinterpret_cast<const u32x4*>(kpool + (size_t)src * block_bytes)[i];
        }
        if (vpool) {
            reinterpret_cast<u32x4*>(vpool + (size_t)dst * block_bytes)[i] =
                reinterpret_cast<const u32x4*>(vpool + (size_t)src * block_bytes)[i];
        }
    }
    for (int h = threadIdx.x; h < n_kv; h += 256) {
        if (kscales) kscales[(size_t)dst * n_kv + h] = kscales[(size_t)src * n_kv + h];
        if (vscales) vscales[(size_t)dst * n_kv + h] = vscales[(size_t)src * n_kv + h];
    }
}

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, uint16_t* k_scales, uint16_t* v_scales,
                              const int32_t* pairs, int n_pairs, int num_blocks, int n_kv, size_t block_bytes,
                              hipStream_t stream) {
    if (n_pairs == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n_pairs), dim3(256), 0, stream,
                       static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), k_scales, v_scales, pairs,
                       num_blocks, n_kv, block_bytes);
    return hipGetLastError();
}

}  // namespace pa

namespace pa {

// Read-bandwidth probe: workgroup w reads tiles w, w + grid, w + 2 grid, ...
// of n_tiles (tile t at byte offset (order ? order[t] : t) * tile_bytes,
// skipped unless that tile lies in the buf_tiles of the buffer; 16-byte
// nontemporal loads, kProbeDepth tiles in flight per thread) and writes the
// XOR of every 32-bit word it read to xor_out[w].
constexpr int kProbeDepth = 8;

__global__ __launch_bounds__(256) void read_probe_kernel(const uint8_t* __restrict__ buf, long buf_tiles,
                                                        long n_tiles, int tile_bytes,
                                                        const int32_t* __restrict__ order,
                                                        uint32_t* __restrict__ xor_out) {
    const int per_tile = tile_bytes / 16;  // 16-byte pieces per tile
    uint32_t acc = 0;
    const long stride = gridDim.x;
    for (long t0 = blockIdx.x; t0 < n_tiles; t0 += stride * kProbeDepth) {
        for (int e = threadIdx.x; e < per_tile; e += 256) {
            u32x4 v[kProbeDepth];
#pragma unroll
            for (int k = 0; k < kProbeDepth; ++k) {
                const long t = t0 + k * stride;
                v[k] = u32x4{0u, 0u, 0u, 0u};
                const long tile = t < n_tiles ? (order ? (long)order[t] : t) : -1;
                if (tile >= 0 && tile < buf_tiles) {
                    v[k] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4*>(buf + tile * (long)tile_bytes) + e);
                }
            }
#pragma unroll
            for (int k = 0; k < kProbeDepth; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
        }
    }
    __shared__ uint32_t red[4];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) xor_out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t take_bad_id_kvops(BadIdRecord* out) {
    const BadIdRecord zero{};
    hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_bad_ids), sizeof(BadIdRecord), 0, hipMemcpyDeviceToHost);
    if (e == hipSuccess && out->flag)
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_bad_ids), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
    return e;
}

hipError_t launch_read_probe(const void* buf, long buf_tiles, long n_tiles, int tile_bytes, const int32_t* order,
                             uint32_t* xor_out, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(buf), buf_tiles, n_tiles, tile_bytes, order, xor_out);
    return hipGetLastError();
}

}  // namespace pa
