// C-ABI entry points: argument validation, split planning and launch.
// Every check runs on the host before any device work is enqueued.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cmath>

#include "../../include/paged_attn.h"
#include "pa_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
std::atomic<unsigned> g_epoch{0};

// Compute units of the current device (cached per device; 256 on MI355X).
int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
    return n;
}

// kv_bits codes the library knows: 32, 16, 8, 4 and PA_KV_FP8.
bool valid_kv_bits(int kv_bits) {
    return kv_bits == 32 || kv_bits == 16 || kv_bits == 8 || kv_bits == 4 || kv_bits == PA_KV_FP8;
}
// Bits of storage per element of a kv_bits code.
int storage_bits(int kv_bits) { return kv_bits == PA_KV_FP8 ? 8 : kv_bits; }
// Quantized formats carry one fp16 scale per (block, KV head).
bool quantized(int kv_bits) { return kv_bits == 8 || kv_bits == 4 || kv_bits == PA_KV_FP8; }

int fmt_of(int dtype, int kv_bits) {
    if (dtype == PA_F32 && kv_bits == 32) return 0;
    if (dtype == PA_BF16 && kv_bits == 16) return 1;
    if (dtype == PA_BF16 && kv_bits == 8) return 2;
    if (dtype == PA_BF16 && kv_bits == 4) return 3;
    if (dtype == PA_BF16 && kv_bits == PA_KV_FP8) return 4;
    return -1;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Blocks per partition. Depends only on host-side shape arguments (never on
// device data or physical block ids), so a given set of arguments always
// splits every sequence at the same logical positions. Large partitions
// amortise each workgroup's start and the merge of its partial, and a
// sequence that fits one partition needs no merge at all; but one workgroup
// streams its partition alone, so with few (sequence, KV head) pairs a
// ragged batch needs short partitions to balance. Hence, by pairs per
// compute unit:
//   more than two: 256 blocks while a batch at max_context_len still gives
//     four workgroups per compute unit;
//   at most one: 256 blocks while it still gives one per compute unit;
//   otherwise (or when those fail): 80 to 128 blocks, largest first, while
//     it gives six per compute unit (at most 80 with two pairs per unit or
//     fewer); then 64, halved until four workgroups per compute unit.
// On shapes the prefix pass applies to, 256 is taken only when a sequence at
// max_context_len still splits in two: unsplit, a batch that shares nothing
// still pays for the pass, and its cost is no longer hidden by a merge the
// split needs anyway (128 x U[512,4096], 32/8/128: 202 us unsplit against
// 197 us at 128 blocks).
int plan_prefix_parts(int num_seqs, int n_heads, int n_kv, int d, int ctx_cap);

int plan_partition_blocks(int num_seqs, int n_heads, int n_kv, int d, int max_context_len, int requested) {
    if (requested > 0) return requested;
    const int max_blocks = std::max(1, ceil_div(max_context_len, PA_BLOCK_SIZE));
    const long pairs = (long)num_seqs * n_kv;
    const long cus = cu_count();
    const int big = pa::kMaxPartitionBlocks;
    const int big_parts = pa::num_parts(max_blocks, big);
    const long big_units = pairs * big_parts;
    const bool big_ok = big_parts > 1 || plan_prefix_parts(num_seqs, n_heads, n_kv, d, max_context_len) == 0;
    if (big_ok && pairs > 2 * cus && big_units >= 4 * cus) return big;
    if (big_ok && pairs <= cus && big_units >= cus) return big;
    const int cap = pairs > 2 * cus ? 128 : 80;
    for (int pb : {128, 112, 96, 80}) {
        if (pb <= cap && pairs * pa::num_parts(max_blocks, pb) >= 6 * cus) return pb;
    }
    const long target = 4 * cus;  // workgroups wanted in flight
    int pb = 64;
    while (pb > 8) {
        const long units = pairs * ceil_div(max_blocks, pb);
        if (units >= target) break;
        pb /= 2;
    }
    return pb;
}

// Prefix partitions per tile (0: no prefix pass) for a decode of this shape.
// The pass runs for d_head 128 and G dividing 32 (one 32-row MFMA tile per
// wave) when the batch has at least two tiles' worth of query rows per KV
// head and the longest context leaves room for a run of kMinPrefixBlocks;
// the run is split so that the pass has about one workgroup per compute
// unit, each range holding at least kMinPrefixBlocks blocks. The element
// format is checked by the caller (bf16 pools only).
int plan_prefix_parts(int num_seqs, int n_heads, int n_kv, int d, int ctx_cap) {
    const int G = n_heads / n_kv;
    if (d != 128 || G <= 0 || 32 % G != 0) return 0;
    if ((long)num_seqs * G < 2L * pa::kPrefixRows) return 0;
    const int max_run = (ctx_cap - 1) / PA_BLOCK_SIZE;
    if (max_run < pa::kMinPrefixBlocks) return 0;
    const int ts = pa::kPrefixRows / G;
    const long tiles = ((long)num_seqs + ts - 1) / ts;
    const long want = ((long)cu_count() + tiles * n_kv - 1) / (tiles * n_kv);
    return (int)std::max(1L, std::min(want, (long)(max_run / pa::kMinPrefixBlocks)));
}

bool valid_common(int num_seqs, int num_blocks, int block_size, int n_heads, int n_kv_heads, int d_head) {
    if (num_seqs < 0 || num_blocks <= 0 || n_heads <= 0 || n_kv_heads <= 0 || d_head <= 0) return false;
    if (block_size != PA_BLOCK_SIZE) return false;
    if (n_heads % n_kv_heads != 0) return false;
    return true;
}

}  // namespace

namespace pa {
unsigned next_epoch() {
    unsigned e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    if (e == 0) e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    return e;
}
}  // namespace pa

extern "C" {

const char* pa_error_string(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID_ARG: return "invalid argument";
        case PA_ERR_UNSUPPORTED: return "unsupported shape or format";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_HIP: return "HIP runtime error";
        case -5: return "not enough free KV blocks";
        case -6: return "unknown (or already used) sequence id";
        case PA_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point holds";
        default: return "unknown status";
    }
}

size_t pa_tile_bytes(int d_head, int kv_bits) {
    if (d_head <= 0 || !valid_kv_bits(kv_bits)) return 0;
    return (size_t)PA_BLOCK_SIZE * d_head * storage_bits(kv_bits) / 8;
}

uint64_t pa_kv_bytes_per_token(int n_layers, int n_kv_heads, int d_head, int kv_bits) {
    if (n_layers <= 0 || n_kv_heads <= 0 || d_head <= 0 || kv_bits <= 0) return 0;
    return 2ull * n_layers * n_kv_heads * (uint64_t)d_head * storage_bits(kv_bits) / 8;
}

uint64_t pa_kv_cache_bytes(int n_layers, int n_kv_heads, int d_head, int kv_bits, int64_t n_tokens) {
    if (n_layers <= 0 || n_kv_heads <= 0 || d_head <= 0 || n_tokens < 0) return 0;
    if (!valid_kv_bits(kv_bits)) return 0;
    const uint64_t blocks = (uint64_t)((n_tokens + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE);
    const uint64_t tile = (uint64_t)PA_BLOCK_SIZE * d_head * storage_bits(kv_bits) / 8 + (quantized(kv_bits) ? 2 : 0);
    return 2ull * n_layers * blocks * n_kv_heads * tile;
}

size_t paged_attn_decode_workspace_size(int num_seqs, int n_heads, int n_kv_heads, int d_head,
                                        int max_context_len, int partition_blocks) {
    if (num_seqs <= 0 || n_heads <= 0 || n_kv_heads <= 0 || d_head <= 0 || max_context_len <= 0) return 0;
    if (partition_blocks < 0 || partition_blocks > pa::kMaxPartitionBlocks || (partition_blocks & 1)) return 0;
    if (n_heads % n_kv_heads != 0) return 0;
    const int pb = plan_partition_blocks(num_seqs, n_heads, n_kv_heads, d_head, max_context_len, partition_blocks);
    const int pmax = pa::num_parts(ceil_div(max_context_len, PA_BLOCK_SIZE), pb);
    const int kpmax = plan_prefix_parts(num_seqs, n_heads, n_kv_heads, d_head, max_context_len);
    return pa::decode_workspace_bytes(num_seqs, n_heads, n_kv_heads, d_head, pmax, kpmax);
}

}  // extern "C"

namespace {

// Both decode entry points; window 0 = none.
int decode_impl(const void* q, const void* k_pool, const void* v_pool, const uint16_t* k_scales,
                const uint16_t* v_scales, const int32_t* block_tables, int max_blocks_per_seq,
                const int32_t* context_lens, int max_context_len, int num_seqs, int num_blocks, int block_size,
                int n_heads, int n_kv_heads, int d_head, int dtype, int kv_bits, void* out, void* workspace,
                size_t workspace_bytes, int partition_blocks, int window, void* stream) {
    if (window < 0) return PA_ERR_INVALID_ARG;
    if (!valid_common(num_seqs, num_blocks, block_size, n_heads, n_kv_heads, d_head)) return PA_ERR_INVALID_ARG;
    if (max_blocks_per_seq <= 0 || max_context_len < 0) return PA_ERR_INVALID_ARG;
    if (partition_blocks < 0 || partition_blocks > pa::kMaxPartitionBlocks || (partition_blocks & 1)) return PA_ERR_INVALID_ARG;
    const int fmt = fmt_of(dtype, kv_bits);
    if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
    if (!valid_kv_bits(kv_bits)) return PA_ERR_INVALID_ARG;
    if (fmt < 0) return PA_ERR_UNSUPPORTED;
    if (d_head != 64 && d_head != 128) return PA_ERR_UNSUPPORTED;
    const int G = n_heads / n_kv_heads;
    if (G > PA_MAX_GROUP) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out) return PA_ERR_INVALID_ARG;
    if (quantized(kv_bits) && (!k_scales || !v_scales)) return PA_ERR_INVALID_ARG;
    if (max_context_len == 0) max_context_len = 1;  // every row is then 0 or 1 token

    pa::DecodeParams p{};
    p.q = q;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.k_scales = k_scales;
    p.v_scales = v_scales;
    p.tables = block_tables;
    p.ctx = context_lens;
    p.out = out;
    p.max_blocks = max_blocks_per_seq;
    p.ctx_cap = (int)std::min<long>((long)max_context_len, (long)PA_BLOCK_SIZE * max_blocks_per_seq);
    p.num_seqs = num_seqs;
    p.num_blocks = num_blocks;
    p.n_heads = n_heads;
    p.n_kv = n_kv_heads;
    p.group = G;
    // planned from max_context_len exactly as paged_attn_decode_workspace_size() does
    p.pb = plan_partition_blocks(num_seqs, n_heads, n_kv_heads, d_head, std::max(1, max_context_len), partition_blocks);
    p.pmax = pa::num_parts(ceil_div(std::max(1, p.ctx_cap), PA_BLOCK_SIZE), p.pb);
    p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d_head));
    p.window = window;

    // Shared-prefix groups (16/G consecutive sequences whose tables name the
    // same blocks fill the 16 MFMA columns, computed by the workgroup of the
    // group's first sequence) for the MFMA formats at G = 4 or 8, when the
    // batch holds a whole group.
    p.share_n = 0;
    // (bf16 keeps the group's ids for at most 128 blocks per partition, so it
    // takes groups only when no partition, an absorbed remainder included,
    // can exceed 128 blocks).
    if (fmt != 0 && window == 0 && (G == 4 || G == 8) && num_seqs >= 16 / G &&
        (fmt != 1 || pa::max_partition_blocks(p.pb) <= 128))
        p.share_n = 16 / G;
    // Prefix pass (bf16 pools): a launch before the decode that attends each
    // tile's common leading run of blocks for all its rows at once.
    p.kpmax = fmt == 1 && window == 0 ? plan_prefix_parts(num_seqs, n_heads, n_kv_heads, d_head, p.ctx_cap)
                                      : 0;
    p.pslots = p.pmax + p.kpmax;
    p.prefix_ts = p.kpmax > 0 ? pa::kPrefixRows / G : 0;
    const size_t need = pa::decode_workspace_bytes(num_seqs, n_heads, n_kv_heads, d_head, p.pmax, p.kpmax);
    int* plan = nullptr;
    if (need > 0) {
        if ((long)num_seqs * n_kv_heads > pa::kMaxCounterPairs) return PA_ERR_UNSUPPORTED;
        if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
        pa::decode_workspace_carve(workspace, num_seqs, n_heads, n_kv_heads, d_head, p.pmax, p.kpmax, &p.part_acc,
                                   &p.part_ml, &p.counters, &plan);
    }
    p.plan = plan;
    p.epoch = pa::next_epoch();
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.kpmax > 0) {
        pa::PrefillParams pp{};
        pp.q = q;
        pp.k_pool = k_pool;
        pp.v_pool = v_pool;
        pp.tables = block_tables;
        pp.ctx = context_lens;
        pp.max_blocks = max_blocks_per_seq;
        pp.ctx_cap = p.ctx_cap;
        pp.num_seqs = num_seqs;
        pp.num_blocks = num_blocks;
        pp.n_heads = n_heads;
        pp.n_kv = n_kv_heads;
        pp.group = G;
        pp.scale_log2 = p.scale_log2;
        pp.part_acc = p.part_acc;
        pp.part_ml = p.part_ml;
        pp.plan = plan;
        pp.pslots = p.pslots;
        pp.kpmax = p.kpmax;
        const hipError_t e = pa::launch_prefix(pp, st);
        if (e != hipSuccess) return PA_ERR_HIP;
    }
    const hipError_t e = pa::launch_decode(p, d_head, fmt, st);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

int paged_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                      const uint16_t* k_scales, const uint16_t* v_scales,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int max_context_len,
                      int num_seqs, int num_blocks, int block_size,
                      int n_heads, int n_kv_heads, int d_head, int dtype, int kv_bits,
                      void* out, void* workspace, size_t workspace_bytes,
                      int partition_blocks, void* stream) {
    return decode_impl(q, k_pool, v_pool, k_scales, v_scales, block_tables, max_blocks_per_seq, context_lens,
                       max_context_len, num_seqs, num_blocks, block_size, n_heads, n_kv_heads, d_head, dtype, kv_bits,
                       out, workspace, workspace_bytes, partition_blocks, 0, stream);
}

int paged_attn_decode_window(const void* q, const void* k_pool, const void* v_pool,
                             const uint16_t* k_scales, const uint16_t* v_scales,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len,
                             int num_seqs, int num_blocks, int block_size,
                             int n_heads, int n_kv_heads, int d_head, int dtype, int kv_bits,
                             void* out, void* workspace, size_t workspace_bytes,
                             int partition_blocks, int window_tokens, void* stream) {
    if (window_tokens <= 0) return PA_ERR_INVALID_ARG;
    return decode_impl(q, k_pool, v_pool, k_scales, v_scales, block_tables, max_blocks_per_seq, context_lens,
                       max_context_len, num_seqs, num_blocks, block_size, n_heads, n_kv_heads, d_head, dtype, kv_bits,
                       out, workspace, workspace_bytes, partition_blocks, window_tokens, stream);
}

}  // extern "C"

namespace {

// Both prefill entry points; window 0 = none.
int prefill_impl(const void* q, const int32_t* cu_q_lens, int total_q, int max_q_len, const void* k_pool,
                 const void* v_pool, const uint16_t* k_scales, const uint16_t* v_scales, const int32_t* block_tables,
                 int max_blocks_per_seq, const int32_t* context_lens, int max_context_len, int num_seqs,
                 int num_blocks, int block_size, int n_heads, int n_kv_heads, int d_head, int dtype, int kv_bits,
                 void* out, int window, void* stream) {
    if (window < 0) return PA_ERR_INVALID_ARG;
    if (!valid_common(num_seqs, num_blocks, block_size, n_heads, n_kv_heads, d_head)) return PA_ERR_INVALID_ARG;
    if (max_blocks_per_seq <= 0 || max_context_len < 0 || total_q < 0 || max_q_len < 0) return PA_ERR_INVALID_ARG;
    if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
    if (!valid_kv_bits(kv_bits)) return PA_ERR_INVALID_ARG;
    const int fmt = fmt_of(dtype, kv_bits);
    if (fmt < 0) return PA_ERR_UNSUPPORTED;
    if (d_head != 64 && d_head != 128) return PA_ERR_UNSUPPORTED;
    const int G = n_heads / n_kv_heads;
    if (G > PA_MAX_GROUP) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
    if (!q || !cu_q_lens || !k_pool || !v_pool || !block_tables || !context_lens || !out) return PA_ERR_INVALID_ARG;
    if (quantized(kv_bits) && (!k_scales || !v_scales)) return PA_ERR_INVALID_ARG;

    pa::PrefillParams p{};
    p.q = q;
    p.cu_q_lens = cu_q_lens;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.k_scales = k_scales;
    p.v_scales = v_scales;
    p.tables = block_tables;
    p.ctx = context_lens;
    p.out = out;
    p.max_blocks = max_blocks_per_seq;
    p.ctx_cap = (int)std::min<long>((long)max_context_len, (long)PA_BLOCK_SIZE * max_blocks_per_seq);
    p.num_seqs = num_seqs;
    p.num_blocks = num_blocks;
    p.n_heads = n_heads;
    p.n_kv = n_kv_heads;
    p.group = G;
    p.max_q_len = max_q_len;
    p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d_head));
    p.window = window;
    const hipError_t e = pa::launch_prefill(p, d_head, fmt, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

int paged_attn_prefill_chunk(const void* q, const int32_t* cu_q_lens, int total_q, int max_q_len,
                             const void* k_pool, const void* v_pool,
                             const uint16_t* k_scales, const uint16_t* v_scales,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len,
                             int num_seqs, int num_blocks, int block_size,
                             int n_heads, int n_kv_heads, int d_head, int dtype, int kv_bits,
                             void* out, void* stream) {
    return prefill_impl(q, cu_q_lens, total_q, max_q_len, k_pool, v_pool, k_scales, v_scales, block_tables,
                        max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_blocks, block_size, n_heads,
                        n_kv_heads, d_head, dtype, kv_bits, out, 0, stream);
}

int paged_attn_prefill_chunk_window(const void* q, const int32_t* cu_q_lens, int total_q, int max_q_len,
                                    const void* k_pool, const void* v_pool,
                                    const uint16_t* k_scales, const uint16_t* v_scales,
                                    const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* context_lens, int max_context_len,
                                    int num_seqs, int num_blocks, int block_size,
                                    int n_heads, int n_kv_heads, int d_head, int dtype, int kv_bits,
                                    void* out, int window_tokens, void* stream) {
    if (window_tokens <= 0) return PA_ERR_INVALID_ARG;
    return prefill_impl(q, cu_q_lens, total_q, max_q_len, k_pool, v_pool, k_scales, v_scales, block_tables,
                        max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_blocks, block_size, n_heads,
                        n_kv_heads, d_head, dtype, kv_bits, out, window_tokens, stream);
}

int kv_quantize(const void* src, void* codes, uint16_t* scales, const int32_t* block_ids, int n_ids,
                int num_blocks, int n_kv_heads, int block_size, int d_head, int bits, int kind, void* stream) {
    if (num_blocks <= 0 || n_kv_heads <= 0 || block_size != PA_BLOCK_SIZE || d_head <= 0) return PA_ERR_INVALID_ARG;
    if (bits != 8 && bits != 4 && bits != PA_KV_FP8) return PA_ERR_INVALID_ARG;
    if (kind != PA_KIND_K && kind != PA_KIND_V) return PA_ERR_INVALID_ARG;
    if (d_head != 64 && d_head != 128) return PA_ERR_UNSUPPORTED;
    if (block_ids && n_ids < 0) return PA_ERR_INVALID_ARG;
    const int n = block_ids ? n_ids : num_blocks;
    if (n == 0) return PA_OK;
    if (!src || !codes || !scales) return PA_ERR_INVALID_ARG;
    // the kernels take 0 for fp8 codes
    const hipError_t e = pa::launch_quantize(src, codes, scales, block_ids, n, num_blocks, n_kv_heads, d_head,
                                             bits == PA_KV_FP8 ? 0 : bits, kind, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_copy_blocks(void* k_pool, void* v_pool, uint16_t* k_scales, uint16_t* v_scales, const int32_t* pairs,
                   int n_pairs, int num_blocks, int n_kv_heads, int d_head, int kv_bits, void* stream) {
    if (n_pairs < 0 || num_blocks <= 0 || n_kv_heads <= 0 || d_head <= 0 || !valid_kv_bits(kv_bits))
        return PA_ERR_INVALID_ARG;
    if (d_head != 64 && d_head != 128) return PA_ERR_UNSUPPORTED;
    if (n_pairs == 0) return PA_OK;
    if (!pairs || n_pairs > 0x7fffffff) return PA_ERR_INVALID_ARG;
    if (!quantized(kv_bits) && (k_scales || v_scales)) return PA_ERR_INVALID_ARG;
    const size_t block_bytes = (size_t)n_kv_heads * PA_BLOCK_SIZE * d_head * storage_bits(kv_bits) / 8;
    const hipError_t e = pa::launch_copy_blocks(k_pool, v_pool, k_scales, v_scales, pairs, n_pairs, num_blocks,
                                                n_kv_heads, block_bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int paged_kv_append(const void* k_new, const void* v_new, const int32_t* cu_new, int total_new, int max_new,
                    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                    void* k_pool, void* v_pool, uint16_t* k_scales, uint16_t* v_scales, void* k_stage,
                    void* v_stage, int num_seqs, int num_blocks, int block_size, int n_kv_heads, int d_head,
                    int dtype, int kv_bits, void* stream) {
    if (num_seqs < 0 || num_blocks <= 0 || block_size != PA_BLOCK_SIZE || n_kv_heads <= 0 || d_head <= 0)
        return PA_ERR_INVALID_ARG;
    if (total_new < 0 || max_new < 0 || max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
    if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
    if (!valid_kv_bits(kv_bits)) return PA_ERR_INVALID_ARG;
    const int fmt = fmt_of(dtype, kv_bits);
    if (fmt < 0) return PA_ERR_UNSUPPORTED;
    if (d_head != 64 && d_head != 128) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || total_new == 0 || max_new == 0 || (!k_new && !v_new)) return PA_OK;
    if (!cu_new || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
    const bool q = quantized(kv_bits);
    if (k_new && (!k_pool || (q && (!k_scales || !k_stage)))) return PA_ERR_INVALID_ARG;
    if (v_new && (!v_pool || (q && (!v_scales || !v_stage)))) return PA_ERR_INVALID_ARG;
    const hipError_t e = pa::launch_kv_append(k_new, v_new, cu_new, max_new, block_tables, max_blocks_per_seq,
                                              context_lens, k_pool, v_pool, k_scales, v_scales, k_stage, v_stage,
                                              num_seqs, num_blocks, n_kv_heads, d_head, fmt,
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_take_block_id_error(int64_t* table_index, int32_t* block_id) {
    pa::BadIdRecord r[3] = {};
    if (pa::take_bad_id_decode(&r[0]) != hipSuccess || pa::take_bad_id_prefill(&r[1]) != hipSuccess ||
        pa::take_bad_id_kvops(&r[2]) != hipSuccess)
        return PA_ERR_HIP;
    for (const auto& x : r) {
        if (!x.flag) continue;
        if (table_index) *table_index = ((int64_t)x.idx_hi << 32) | (int64_t)x.idx_lo;
        if (block_id) *block_id = x.id;
        return 1;
    }
    return 0;
}

int pa_hbm_read_probe(const void* buf, int64_t buf_bytes, int tile_bytes, const int32_t* order, int64_t n_order,
                      uint32_t* xor_out, int grid, void* stream) {
    if (buf_bytes < 0 || n_order < 0 || tile_bytes < 16 || tile_bytes > 65536 || tile_bytes % 16 != 0)
        return PA_ERR_INVALID_ARG;
    if (grid <= 0 || grid > 65536 || !xor_out || (buf_bytes > 0 && !buf) || (n_order > 0 && !order))
        return PA_ERR_INVALID_ARG;
    const long buf_tiles = (long)(buf_bytes / tile_bytes);
    const long n_tiles = order ? (long)n_order : buf_tiles;
    const hipError_t e = pa::launch_read_probe(buf, buf_tiles, n_tiles, tile_bytes, order, xor_out, grid,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int paged_kv_write(const void* k_src, const void* v_src, const int64_t* slot_mapping, int num_tokens,
                   void* k_pool, void* v_pool, int num_blocks, int block_size,
                   int n_kv_heads, int d_head, int dtype, void* stream) {
    if (num_tokens < 0 || num_blocks <= 0 || block_size != PA_BLOCK_SIZE || n_kv_heads <= 0 || d_head <= 0)
        return PA_ERR_INVALID_ARG;
    if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
    if (d_head != 64 && d_head != 128) return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0 || (!k_src && !v_src)) return PA_OK;
    if (!slot_mapping) return PA_ERR_INVALID_ARG;
    if ((k_src && !k_pool) || (v_src && !v_pool)) return PA_ERR_INVALID_ARG;
    const hipError_t e = pa::launch_kv_write(k_src, v_src, slot_mapping, num_tokens, k_pool, v_pool, num_blocks,
                                             n_kv_heads, d_head, dtype == PA_F32 ? 0 : 1,
                                             static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
