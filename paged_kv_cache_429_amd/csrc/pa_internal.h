// Host <-> kernel interface of the library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Context partitions of a sequence of nblk blocks (nblk >= 1) at pb blocks
// per partition. Partition p starts at block p * pb and holds pb blocks; the
// last one runs to the end of the sequence and absorbs a remainder of at
// most pb / 4 blocks instead of leaving it as a short partition of its own
// (a short partition's workgroup never fills its load pipeline). Partitions
// therefore hold up to 5 pb / 4 blocks. Depends only on the length, never on
// block ids.
constexpr int kAbsorbDiv = 4;
__host__ __device__ inline int num_parts(int nblk, int pb) {
    const int full = nblk / pb;
    const int rem = nblk - full * pb;
    const int thr = pb / kAbsorbDiv;
    const int n = full + (rem > thr ? 1 : 0);
    return n > 1 ? n : 1;
}
__host__ __device__ inline int part_end(int nblk, int pb, int part, int nparts) {
    return part + 1 == nparts ? nblk : (part + 1) * pb;
}

struct DecodeParams {
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const uint16_t* k_scales;
    const uint16_t* v_scales;
    const int32_t* tables;
    const int32_t* ctx;
    void* out;
    float* part_acc;    // [num_seqs][n_heads][pmax][d]   (unnormalised)
    float* part_ml;     // [num_seqs][n_heads][pmax][2]   (max, sum) in log2 units
    int* counters;      // [num_seqs][n_kv] partitions arrived (zero between calls)
    int max_blocks;     // table row stride
    int ctx_cap;        // min(max_context_len, 16 * max_blocks)
    int num_seqs;
    int num_blocks;
    int n_heads;
    int n_kv;
    int group;
    int pmax;           // num_parts() of a sequence at max_context_len
    int pb;             // blocks per partition (even)
    float scale_log2;   // log2(e) / sqrt(d)
    int share_n;        // sequences per shared-prefix group (0: no shared-prefix workgroups)
    int n_shared;       // shared-prefix workgroups, first in the grid: (S / share_n) * pmax * n_kv
};

// Bytes of the arrival-counter region at the start of a decode workspace:
// one int32 per (sequence, KV head), so num_seqs * n_kv_heads <= 262144.
constexpr size_t kCounterBytes = (size_t)1 << 20;
constexpr long kMaxCounterPairs = (long)(kCounterBytes / sizeof(int));

// Workspace bytes for the arrival counters and split-context partials (0
// when pmax == 1).
size_t decode_workspace_bytes(int num_seqs, int n_heads, int n_kv, int d, int pmax);
void decode_workspace_carve(void* ws, int num_seqs, int n_heads, int n_kv, int d, int pmax, float** part_acc,
                            float** part_ml, int** counters);

// fmt: 0 fp32, 1 bf16, 2 int8, 3 int4. Launches the decode kernel on
// `stream`.
hipError_t launch_decode(const DecodeParams& p, int d, int fmt, hipStream_t stream);

struct PrefillParams {
    const void* q;
    const int32_t* cu_q_lens;
    const void* k_pool;
    const void* v_pool;
    const uint16_t* k_scales;
    const uint16_t* v_scales;
    const int32_t* tables;
    const int32_t* ctx;
    void* out;
    int max_blocks;
    int ctx_cap;
    int num_seqs;
    int num_blocks;
    int n_heads;
    int n_kv;
    int group;
    int max_q_len;
    float scale_log2;
};

hipError_t launch_prefill(const PrefillParams& p, int d, int fmt, hipStream_t stream);

hipError_t launch_quantize(const void* src, void* codes, uint16_t* scales, const int32_t* block_ids, int n_ids,
                           int num_blocks, int n_kv, int d, int bits, int kind, hipStream_t stream);

hipError_t launch_kv_write(const void* k_src, const void* v_src, const int64_t* slots, int num_tokens,
                           void* k_pool, void* v_pool, int num_blocks, int n_kv, int d, int fmt,
                           hipStream_t stream);

}  // namespace pa
