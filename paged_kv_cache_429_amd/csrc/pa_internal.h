// Host <-> kernel interface of the library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Context partitions of a sequence of nblk blocks (nblk >= 1) at pb blocks
// per partition (pb <= 256). Partition p starts at block p * pb and holds pb
// blocks; the last one runs to the end of the sequence and absorbs a
// remainder of at most min(pb / 4, 256 - pb) blocks instead of leaving it as
// a short partition of its own (a short partition's workgroup never fills
// its load pipeline). Partitions therefore hold at most 256 blocks: each of
// the four waves keeps the ids of its 64 blocks in one register. Depends
// only on the length, never on block ids.
constexpr int kAbsorbDiv = 4;
constexpr int kMaxPartitionBlocks = 256;
__host__ __device__ inline int num_parts(int nblk, int pb) {
    const int full = nblk / pb;
    const int rem = nblk - full * pb;
    const int thr = pb / kAbsorbDiv < kMaxPartitionBlocks - pb ? pb / kAbsorbDiv : kMaxPartitionBlocks - pb;
    const int n = full + (rem > thr ? 1 : 0);
    return n > 1 ? n : 1;
}
__host__ __device__ inline int part_end(int nblk, int pb, int part, int nparts) {
    return part + 1 == nparts ? nblk : (part + 1) * pb;
}
// Most blocks a partition can hold at pb blocks per partition (the last
// partition's absorbed remainder included).
__host__ __device__ inline int max_partition_blocks(int pb) {
    const int thr = pb / kAbsorbDiv < kMaxPartitionBlocks - pb ? pb / kAbsorbDiv : kMaxPartitionBlocks - pb;
    return pb + thr;
}

// Prefix pass ("jovanaeducation" guide a2-inf-2, section "Prefix caching";
// "KV cache, GQA, paging and continuous batching", section
// "PagedAttention..."): the batch is cut into tiles of kPrefixRows / G
// consecutive sequences (kPrefixRows query rows per KV head). For each tile,
// the longest leading run of logical blocks that every member holds at the
// same physical ids, with at least one token of every member after it, is
// found and cut to whole key stages of kPrefixStageBlocks blocks (a masked
// partial stage would cost the pass more registers than the few blocks
// save); a run of kMinPrefixBlocks or more is attended by one MFMA
// contraction over all the tile's rows (bf16 pools, d_head 128), its
// stages split into prefix_parts() near-equal ranges that each leave a
// log-sum-exp partial. The decode workgroups then cover only the blocks
// after the run and merge with those partials.
constexpr int kPrefixRows = 256;
constexpr int kPrefixStageBlocks = 4;
constexpr int kMinPrefixBlocks = 16;
__host__ __device__ inline int prefix_parts(int run_blocks, int kpmax) {
    const int stages = run_blocks / kPrefixStageBlocks;
    return stages < kpmax ? stages : kpmax;
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
    float* part_acc;    // [num_seqs][n_heads][pslots][d]   (unnormalised)
    float* part_ml;     // [num_seqs][n_heads][pslots][2]   (max, sum) in log2 units
    unsigned long long* counters;  // [num_seqs][n_kv] arrival words: epoch << 32 | partitions arrived
    unsigned epoch;     // this call's epoch (never 0); a word of another epoch counts as 0 arrivals
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
    int share_n;        // sequences per shared-prefix group (0: no group check)
    int pslots;         // partial slots per (sequence, query head): kpmax + pmax
    int prefix_ts;      // sequences per prefix-pass tile (0: no prefix pass)
    int kpmax;          // prefix partitions per tile at most
    const int* plan;    // [tiles] run (blocks) the prefix pass covered, written by it
    int window;         // sliding window in tokens (0: none): the last `window` tokens are attended
};

// Bytes of the arrival-counter region at the start of a decode workspace:
// one 64-bit word per (sequence, KV head), so num_seqs * n_kv_heads <=
// 262144. A word holds the epoch of the call that last counted in it (high
// half) and the partitions of that call that have arrived (low half); every
// call has an epoch of its own, so whatever a word holds from an earlier
// call (one that completed, or one whose launch died midway) counts as zero
// arrivals, and the region needs no initialisation.
constexpr size_t kCounterBytes = (size_t)2 << 20;
constexpr long kMaxCounterPairs = (long)(kCounterBytes / sizeof(unsigned long long));

// A fresh epoch for a decode call (process-wide counter, skipping 0).
unsigned next_epoch();

// Workspace bytes for the arrival counters and split-context partials (0
// when pmax == 1).
size_t decode_workspace_bytes(int num_seqs, int n_heads, int n_kv, int d, int pmax, int kpmax);
void decode_workspace_carve(void* ws, int num_seqs, int n_heads, int n_kv, int d, int pmax, int kpmax,
                            float** part_acc, float** part_ml, unsigned long long** counters, int** plan);

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
    int window;         // sliding window in tokens (0: none): row at position p attends keys p - window + 1 .. p
    // prefix pass only (see kPrefixRows)
    float* part_acc;
    float* part_ml;
    int* plan;
    int pslots;
    int kpmax;
};

hipError_t launch_prefill(const PrefillParams& p, int d, int fmt, hipStream_t stream);

// The prefix pass of a decode step (bf16 pools, d_head 128, 32 % G == 0):
// num_seqs, tables, ctx, ctx_cap, q as for the decode; writes the tiles'
// plan entries and the prefix partials in slots 0 .. prefix_parts() - 1.
hipError_t launch_prefix(const PrefillParams& p, hipStream_t stream);

// Block-table entries outside [0, num_blocks) met by a kernel are read as
// block 0 and recorded: the first one per device and per source file, as
// (flag, table index high, table index low, id). read_*_bad_id copies the
// record of that file's kernels to the host and clears it (synchronous).
struct BadIdRecord {
    int flag;
    int idx_hi;
    unsigned idx_lo;
    int id;
};
hipError_t take_bad_id_decode(BadIdRecord* out);
hipError_t take_bad_id_prefill(BadIdRecord* out);
hipError_t take_bad_id_kvops(BadIdRecord* out);

hipError_t launch_quantize(const void* src, void* codes, uint16_t* scales, const int32_t* block_ids, int n_ids,
                           int num_blocks, int n_kv, int d, int bits, int kind, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, uint16_t* k_scales, uint16_t* v_scales,
                              const int32_t* pairs, int n_pairs, int num_blocks, int n_kv, size_t block_bytes,
                              hipStream_t stream);

hipError_t launch_read_probe(const void* buf, long buf_tiles, long n_tiles, int tile_bytes, const int32_t* order,
                             uint32_t* xor_out, int grid, hipStream_t stream);

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int32_t* cu_new, int max_new,
                            const int32_t* tables, int max_blocks, const int32_t* ctx, void* k_pool, void* v_pool,
                            uint16_t* k_scales, uint16_t* v_scales, void* k_stage, void* v_stage, int num_seqs,
                            int num_blocks, int n_kv, int d, int fmt, hipStream_t stream);

hipError_t launch_kv_write(const void* k_src, const void* v_src, const int64_t* slots, int num_tokens,
                           void* k_pool, void* v_pool, int num_blocks, int n_kv, int d, int fmt,
                           hipStream_t stream);

}  // namespace pa
