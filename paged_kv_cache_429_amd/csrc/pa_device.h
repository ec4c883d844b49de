// Device-side helpers shared by the gfx950 kernels: vector types, bf16/fp16
// conversions, MFMA wrappers and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

// The first block-table entry outside [0, num_blocks) that a kernel of this
// source file met on this device since the host last took the record (the
// kernels read such an entry as block 0). Taken by take_bad_id_*.
static __device__ BadIdRecord g_bad_ids;

// Record entry `idx` of a block-table array holding the out-of-range id
// `id`, unless a record is already held. Runs only for such an entry.
__device__ __noinline__ void note_bad_id(long idx, int id) {
    if (atomicCAS(&g_bad_ids.flag, 0, 1) == 0) {
        g_bad_ids.idx_hi = (int)(idx >> 32);
        g_bad_ids.idx_lo = (unsigned)idx;
        g_bad_ids.id = id;
    }
}

// Block id `id` read from entry `idx` of the table array, or 0 (recorded)
// when it lies outside the pool.
__device__ __forceinline__ int checked_id(int id, long idx, int num_blocks) {
    if ((unsigned)id >= (unsigned)num_blocks) {
        note_bad_id(idx, id);
        id = 0;
    }
    return id;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;   // tokens per physical block
constexpr int kWave = 64;    // CDNA wavefront

enum KvFmt { FMT_F32 = 0, FMT_BF16 = 1, FMT_I8 = 2, FMT_I4 = 3, FMT_F8 = 4 };

template <int FMT> struct FmtBits;
template <> struct FmtBits<FMT_F32> { static constexpr int v = 32; };
template <> struct FmtBits<FMT_BF16> { static constexpr int v = 16; };
template <> struct FmtBits<FMT_I8> { static constexpr int v = 8; };
template <> struct FmtBits<FMT_I4> { static constexpr int v = 4; };
template <> struct FmtBits<FMT_F8> { static constexpr int v = 8; };

// Quantized formats: codes that share one fp16 scale per (block, KV head).
template <int FMT> constexpr bool is_quant() { return FMT == FMT_I8 || FMT == FMT_I4 || FMT == FMT_F8; }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bfloat16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bfloat16 pair (lo in the low half), round to nearest
// even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ float fp16_bits_to_f32(uint16_t h) {
    _Float16 x = __builtin_bit_cast(_Float16, h);
    return (float)x;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16 f32) += A(16x32 bf16) * B(32x16 bf16). Lane l supplies row l%16 of
// A and column l%16 of B, eight consecutive k each (k-slot group l/16); the
// result lane l holds rows 4*(l/16)+i, column l%16.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// D(32x32 f32) += A(32x16 bf16) * B(16x32 bf16). Lane l supplies row l%32
// of A and column l%32 of B, eight consecutive k each (k-slot group l/32);
// result register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Exact int8 -> bf16 of the four codes in a dword (|code| <= 128 fits bf16).
// OCP fp8 e4m3 -> bf16 of the four bytes of a dword (byte 0 first, in the
// low half of r[0]): two v_cvt_scalef32_pk_bf16_fp8 at scale 1. Every e4m3
// value (3 mantissa bits, exponents 2^-9 .. 2^8) is a bf16 value, so the
// conversion is exact.
__device__ __forceinline__ u32x2 f8x4_to_bf16x4(uint32_t w) {
    u32x2 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    return r;
}

__device__ __forceinline__ u32x2 i8x4_to_bf16x4(uint32_t w) {
    float f0 = (float)((int32_t)(w << 24) >> 24);
    float f1 = (float)((int32_t)(w << 16) >> 24);
    float f2 = (float)((int32_t)(w << 8) >> 24);
    float f3 = (float)((int32_t)w >> 24);
    u32x2 r;
    r[0] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
    r[1] = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xffff0000u);
    return r;
}

// int8 -> bf16 of the four bytes of a dword (byte 0 first), offset by +128:
// flipping a byte's sign bit gives v + 128 in [0, 255], converted by the
// unsigned-byte instructions to a float with at most 8 significant bits,
// whose upper half is then exactly its bf16.
__device__ __forceinline__ u32x2 i8x4_to_bf16x4_off128(uint32_t w) {
    const uint32_t x = w ^ 0x80808080u;
    const uint32_t f0 = __float_as_uint((float)(x & 0xffu));
    const uint32_t f1 = __float_as_uint((float)((x >> 8) & 0xffu));
    const uint32_t f2 = __float_as_uint((float)((x >> 16) & 0xffu));
    const uint32_t f3 = __float_as_uint((float)(x >> 24));
    u32x2 r;
    r[0] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);  // high halves of f0 (low) and f1 (high)
    r[1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
    return r;
}

// Exact int4 -> bf16 of the eight nibbles of a dword (low nibble first).
__device__ __forceinline__ u32x4 i4x8_to_bf16x8(uint32_t w) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float lo = (float)((int32_t)(w << (28 - 8 * k)) >> 28);
        float hi = (float)((int32_t)(w << (24 - 8 * k)) >> 28);
        r[k] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
    }
    return r;
}

// int4 -> bf16 of the eight nibbles of a dword (low nibble first), offset by
// +136: flipping a two's-complement nibble's sign bit gives v + 8 in [0, 15],
// and those four bits OR-ed into the mantissa of bf16 128 (0x4300) make
// exactly 136 + v. Byte k of the result pairs element 2k (low half) with
// element 2k + 1 (high half), like i4x8_to_bf16x8.
__device__ __forceinline__ u32x4 i4x8_to_bf16x8_off136(uint32_t w) {
    const uint32_t x = w ^ 0x88888888u;
    const uint32_t a = x & 0x0f0f0f0fu;         // elements 0, 2, 4, 6
    const uint32_t b = (x >> 4) & 0x0f0f0f0fu;  // elements 1, 3, 5, 7
    // v_perm_b32: selector bytes 0-3 pick bytes of the second operand (a),
    // 4-7 bytes of the first (b), 0x0c gives zero
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(b, a, 0x0c040c00u) | 0x43004300u;
    r[1] = __builtin_amdgcn_perm(b, a, 0x0c050c01u) | 0x43004300u;
    r[2] = __builtin_amdgcn_perm(b, a, 0x0c060c02u) | 0x43004300u;
    r[3] = __builtin_amdgcn_perm(b, a, 0x0c070c03u) | 0x43004300u;
    return r;
}

// The same values as i4x8_to_bf16x8_off136, elements in the order
// 0, 2, 4, 6, 1, 3, 5, 7 (dword j holds elements 2j, 2j + 2 for j < 2 and
// 2j - 3, 2j - 1 for j >= 2): each dword is one v_perm of the even or odd
// nibbles with bf16 128's high byte taken from a constant, so no OR is
// needed. The other MFMA operand takes the same order (bf16x8_even_odd).
__device__ __forceinline__ u32x4 i4x8_to_bf16x8_off136_eo(uint32_t w) {
    // each a three-input bitwise op (v_bitop3) of w or w >> 4
    const uint32_t a = (w ^ 0x88888888u) & 0x0f0f0f0fu;         // byte k: element 2k + 8
    const uint32_t b = ((w >> 4) ^ 0x08080808u) & 0x0f0f0f0fu;  // byte k: element 2k + 1 + 8
    const uint32_t hi = 0x43434343u;
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(hi, a, 0x04010400u);  // elements 0, 2
    r[1] = __builtin_amdgcn_perm(hi, a, 0x04030402u);  // elements 4, 6
    r[2] = __builtin_amdgcn_perm(hi, b, 0x04010400u);  // elements 1, 3
    r[3] = __builtin_amdgcn_perm(hi, b, 0x04030402u);  // elements 5, 7
    return r;
}

// Eight 16-bit values (dword j = elements 2j, 2j + 1) reordered to
// 0, 2, 4, 6, 1, 3, 5, 7, the order of i4x8_to_bf16x8_off136_eo.
__device__ __forceinline__ u32x4 bf16x8_even_odd(u32x4 v) {
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
    r[1] = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);
    r[2] = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
    r[3] = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);
    return r;
}

// Exact int4 -> bf16 of the four nibbles in the low 16 bits.
__device__ __forceinline__ u32x2 i4x4_to_bf16x4(uint32_t w) {
    u32x4 t = i4x8_to_bf16x8(w);
    u32x2 r;
    r[0] = t[0];
    r[1] = t[1];
    return r;
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask)); }

template <typename T>
__device__ __forceinline__ T readlane(T v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}

// Direct global-to-LDS load of 16 bytes per lane: lane i's bytes land at LDS
// byte address lds_base + 16 i (lds_base wave-uniform). It is issued as
// inline assembly so that the compiler does not make every later LDS read
// wait for it (it cannot tell which LDS bytes the load writes, and would
// otherwise drain all such loads before the next LDS read, which defeats
// multi-buffering); the caller orders it with lds_wait_barrier.
// M0 (which carries the LDS address) is saved and restored around it.
__device__ __forceinline__ void lds_dma16(const void* src, const void* lds_dst) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)lds_dst)));
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(base)
        : "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (loads complete in order, so every earlier direct-to-LDS load has landed),
// then a workgroup barrier. A compiler memory barrier as well: no memory
// access moves across it.
template <int N>
__device__ __forceinline__ void lds_wait_barrier() {
    static_assert(N >= 0 && N < 16, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

}  // namespace pa
