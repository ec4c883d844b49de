/*
 * paged_attn.h -- paged-KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels:
 *   paged_attn_decode         single-query attention of a batch of sequences
 *   paged_attn_decode_window  the same over each sequence's last W tokens
 *   paged_attn_prefill_chunk  causal attention of a chunk of prompt tokens
 *   paged_attn_prefill_chunk_window  the same over each row's last W tokens
 *   kv_quantize               symmetric int8 / int4 codes + fp16 scales
 *   paged_kv_write            scatter new tokens' K/V into their cache slots
 *   paged_kv_append           append new tokens through the block table,
 *                             quantizing on write for int8 / int4 / fp8 pools
 * plus a few host-only helpers (sizes, error strings).
 *
 * Sources (three web pages on KV caching, cited by title and section):
 *   [TAI] "KV cache, continuous batching and paged attention"
 *   [IR]  "KV cache, GQA, paging and continuous batching"
 *   [JE]  jovanaeducation inference guide a2-inf-2
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ---------------------------------------------------------------------------
 * Memory. Every array argument is caller-owned device memory of the current
 * HIP device, unless stated otherwise; the library never allocates, frees or
 * retains a pointer after the call returns.
 *
 * Streams. `stream` is a hipStream_t passed as void* (NULL = the null
 * stream). Every call only enqueues work on that stream and returns; results
 * are ready once the stream reaches that point. The host never reads device
 * data, so no call synchronises.
 *
 * Errors. Each call returns PA_OK or a negative pa_status. Argument errors
 * are detected on the host before any device work is enqueued (nothing is
 * written). PA_ERR_HIP means a HIP launch call failed; a fault inside a
 * kernel surfaces as a HIP error at the caller's next synchronisation.
 * The only mutable global state is a per-device cache of the compute-unit
 * count (atomic); calls may be made from several host threads on different
 * streams.
 *
 * Paging ([TAI] "Paged attention"; [IR] "PagedAttention: why fragmentation
 * was eating most of the rest"). The cache of one layer is a pool of
 * `num_blocks` physical blocks of `block_size` = 16 token slots each. A
 * sequence's logical token t lives in slot t % 16 of physical block
 * block_tables[s * max_blocks_per_seq + t / 16]. Physical blocks may be
 * shared between sequences (common prefixes, [JE] "Prefix caching"); the
 * kernels follow the table and never write the pool. Only the entries
 * j < ceil(ctx_s / 16) of a row are used. Block ids outside [0, num_blocks)
 * are a caller error: the kernels replace them by block 0 (never reading out
 * of bounds), so results for that sequence are then meaningless, and record
 * the first such entry; pa_take_block_id_error() reports it.
 *
 * GQA ([IR] "What it is" and the table in "The memory equation"): query head
 * h reads KV head h / G, G = n_heads / n_kv_heads (contiguous groups);
 * n_kv_heads = n_heads is MHA, n_kv_heads = 1 is MQA. 1 <= G <= 16.
 *
 * Attention ([JE] the figure of attention as a soft query-key-value lookup;
 * [IR] "What it is"): o = softmax(q K^T / sqrt(d_head)) V with float32
 * accumulation. The pages lose the formula; the 1/sqrt(d_head) scale is the
 * standard reading and is not an argument.
 *
 * ---------------------------------------------------------------------------
 * Device layout of the K/V pools
 * ---------------------------------------------------------------------------
 * kv_bits gives the element format of the pools:
 *   32  float32            (requires dtype == PA_F32)
 *   16  bfloat16           (requires dtype == PA_BF16)
 *    8  int8 code  + fp16 scale per (block, KV head) (requires PA_BF16)
 *    4  int4 code  + fp16 scale per (block, KV head) (requires PA_BF16)
 *   PA_KV_FP8  OCP fp8 e4m3 code + fp16 scale per (block, KV head)
 *              (requires PA_BF16). One byte per element, laid
 *              out as int8; bit 7 sign, bits 6..3 exponent (bias 7), bits
 *              2..0 mantissa, exponent 0 subnormal, 0x7F / 0xFF NaN.
 * A pool is an array of tiles, one per (block b, KV head h), each holding the
 * 16 slots x d_head elements of that block and head, at byte offset
 *     ((size_t)b * n_kv_heads + h) * tile_bytes,  tile_bytes = 16*d_head*bits/8,
 * where bits is kv_bits, or 8 for PA_KV_FP8.
 * Inside a tile, element (slot t, dim i) is element number
 *     K pool:  ((i / x) * 16 + t) * x + i % x,   x = 128 / bits
 *              (16-byte chunks of x consecutive dims, slot-minor)
 *     V pool:  i * 16 + t                          (transposed: dim-major)
 *              for kv_bits 32, 16, 8 and PA_KV_FP8; for kv_bits 4
 *              (((i % 16) * 2 + t / 8) * (d_head / 16) + i / 16) * 8 + t % 8
 *              (runs of 8 consecutive slots of one dim; the d_head / 16 runs
 *              of dims i % 16 and slots t / 8 side by side)
 * of the tile, elements packed at kv_bits each, little-endian; for int4 the
 * even-numbered element of a pair is the low nibble. Integer codes are two's
 * complement. Scales are float16 bit patterns, k_scales / v_scales
 * [num_blocks][n_kv_heads]; value = code * scale (for fp8, the code's e4m3
 * value times the scale).
 * Supported d_head: 64 and 128.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = -1,  /* a pointer, size or shape is invalid            */
    PA_ERR_UNSUPPORTED = -2,  /* valid, but not a shape/format this build runs  */
    PA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required     */
    PA_ERR_HIP = -4,          /* a HIP runtime call failed                      */
    PA_ERR_SCRATCH = -7       /* paged_attn_decode_noalloc: the call needs more
                                 scratch than its fixed device array holds      */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;
typedef enum pa_kv_kind { PA_KIND_K = 0, PA_KIND_V = 1 } pa_kv_kind;

#define PA_BLOCK_SIZE 16
#define PA_MAX_GROUP 16
/* kv_bits code of OCP fp8 e4m3 pools (8 bits of storage per element). */
#define PA_KV_FP8 264
#define PA_DECODE_COUNTER_BYTES (2u << 20)
/* Bytes of the fixed per-device scratch of paged_attn_decode_noalloc. */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Human-readable text of a status code (static storage). */
const char* pa_error_string(int status);

/* Bytes of one (block, KV head) tile: 16 * d_head * kv_bits / 8; 0 if the
 * arguments are invalid. Host only. */
size_t pa_tile_bytes(int d_head, int kv_bits);

/* KV bytes per token, all layers: 2 (K and V) x n_layers x n_kv_heads x
 * d_head x kv_bits/8 ([TAI] "The KV cache"; [IR] "The memory equation").
 * Host only. */
uint64_t pa_kv_bytes_per_token(int n_layers, int n_kv_heads, int d_head, int kv_bits);

/* Bytes a paged cache holds for one sequence of n_tokens: whole 16-token
 * blocks of K and V in every layer, plus the two fp16 scales per (block, KV
 * head) of a quantized cache. Host only. */
uint64_t pa_kv_cache_bytes(int n_layers, int n_kv_heads, int d_head, int kv_bits, int64_t n_tokens);

/* ---------------------------------------------------------------------------
 * Decode ([TAI] "Paged attention": the attention kernel follows the block
 * table; [TAI] "The KV cache": each step attends over the cached K/V of all
 * earlier tokens).
 *
 * q            [num_seqs][n_heads][d_head] of dtype
 * k_pool/v_pool  pools in the layout above (read only)
 * k_scales/v_scales  fp16 [num_blocks][n_kv_heads]; NULL unless kv_bits is
 *              8, 4 or PA_KV_FP8
 * block_tables int32 [num_seqs][max_blocks_per_seq]
 * context_lens int32 [num_seqs]: tokens to attend, including the token being
 *              decoded (its K/V must already be in the pool). Values are
 *              clamped to min(max_context_len, 16 * max_blocks_per_seq); a
 *              value <= 0 yields a zero output row.
 * max_context_len  host-side upper bound of context_lens (plans the split)
 * out          [num_seqs][n_heads][d_head] of dtype (written)
 * workspace    device scratch of at least paged_attn_decode_workspace_size()
 *              bytes (may be NULL when that size is 0). It needs no
 *              initialisation. Its first PA_DECODE_COUNTER_BYTES hold
 *              arrival words, one 64-bit word per (sequence, KV head), so
 *              num_seqs * n_kv_heads may not exceed
 *              PA_DECODE_COUNTER_BYTES / 8 (else PA_ERR_UNSUPPORTED). Each
 *              call tags the words it counts in with an epoch of its own (a
 *              process-wide 32-bit counter), and a word of any other epoch
 *              counts as zero arrivals, so neither garbage nor the leftovers
 *              of a call whose launch died midway affect later calls. (A
 *              captured launch replays its epoch; it stays correct because
 *              each completed merge leaves its word at a count of zero.) The
 *              rest holds the partials of split sequences and of the prefix
 *              pass, and the prefix pass's per-tile runs. One workspace
 *              serves calls of any shape, but calls that share it must be
 *              ordered (same stream, or synchronised): overlapping calls
 *              race.
 * partition_blocks  blocks per context partition pb (even, 2..256), or 0 to
 *              let the library choose (from the arguments' values alone). Long contexts are split into
 *              partitions processed in parallel and merged by log-sum-exp
 *              within the same launch: the last partition of a (sequence,
 *              KV head) to finish merges them, in partition order. Partition
 *              p starts at block b0 + p * pb; the last one also takes a
 *              remainder of up to min(pb / 4, 256 - pb) blocks. b0 is 0
 *              unless the prefix pass below took a run of the sequence's
 *              first blocks (then b0 is the run's length). The split depends only on the
 *              arguments' values on the host, each sequence's length and
 *              that run.
 *              Shared prefixes ([JE] "Prefix caching"), two mechanisms:
 *              - Prefix pass. When the batch has at least 512 query rows
 *                per KV head (num_seqs * G >= 512) with bf16 pools, d_head
 *                128 and G dividing 32, a first launch takes tiles of
 *                256 / G consecutive sequences. In each, the longest
 *                leading run of blocks that every member holds at the same
 *                physical ids and that ends before every member's last
 *                token, cut to a multiple of 4 blocks, is attended, if it
 *                holds at least 16 blocks, for all the tile's query rows at
 *                once (one MFMA contraction, each shared block read once
 *                per tile and KV head); its log-sum-exp partials are merged
 *                with the decode's partitions of the blocks after the run.
 *                Such sequences agree with private copies of the same
 *                blocks to rounding, not bit for bit.
 *              - Shared groups. Elsewhere, consecutive sequences (16 / G
 *                of them, for G = 4 or 8) whose tables name the same
 *                physical blocks for a partition's first two blocks are
 *                processed together, by the workgroup of the group's first
 *                sequence, each shared block being read once for the group;
 *                results are bit-identical to those of private copies of
 *                the same blocks. With bf16 pools, only when no partition
 *                can exceed 128 blocks: pb + min(pb / 4, 256 - pb) <= 128.
 * ------------------------------------------------------------------------ */
size_t paged_attn_decode_workspace_size(int num_seqs, int n_heads, int n_kv_heads, int d_head,
                                        int max_context_len, int partition_blocks);

int paged_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                      const uint16_t* k_scales, const uint16_t* v_scales,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int max_context_len,
                      int num_seqs, int num_blocks, int block_size,
                      int n_heads, int n_kv_heads, int d_head, int dtype, int kv_bits,
                      void* out, void* workspace, size_t workspace_bytes,
                      int partition_blocks, void* stream);

/* ---------------------------------------------------------------------------
 * paged_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The call allocates nothing (no hipMalloc,
 * no hipFree, no allocating library routine): its scratch is a fixed
 * device array of PA_DECODE_NOALLOC_SCRATCH_BYTES (64 MiB) that the library
 * holds on each device it runs on until the process ends. Arguments and
 * results as for paged_attn_decode (the caller still passes the inputs and
 * the output). A call whose workspace, as paged_attn_decode_workspace_size()
 * gives it, exceeds the array returns PA_ERR_SCRATCH before any device work
 * (the 70B prefix-shared batch of 256 x 4500 tokens needs about 51 MiB).
 * The first call on a device takes the array's device address
 * (PA_ERR_HIP if that fails). The array keeps whatever the last call left;
 * nothing in it needs to start at zero (arrival words are epoch-tagged).
 * Every call on one device shares the array: calls that overlap on a device
 * (different streams, or host threads, without ordering) race.
 * ------------------------------------------------------------------------ */
int paged_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const uint16_t* k_scales, const uint16_t* v_scales,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, int max_context_len,
                              int num_seqs, int num_blocks, int block_size,
                              int n_heads, int n_kv_heads, int d_head, int dtype, int kv_bits,
                              void* out, int partition_blocks, void* stream);

/* ---------------------------------------------------------------------------
 * Sliding-window decode ([IR] "The memory equation": sliding-window attention
 * is one of the ways to shrink the cache; the pages give no formula). The
 * query of sequence s (its last token, position ctx_s - 1) attends only the
 * last window_tokens tokens, positions max(0, ctx_s - window_tokens) ..
 * ctx_s - 1; a window of at least ctx_s is full attention.
 * Arguments as for paged_attn_decode (same workspace size), plus
 * window_tokens >= 1 (else PA_ERR_INVALID_ARG). Only the blocks holding
 * attended tokens are read (table entries before them are not). The
 * shared-prefix mechanisms are not used: every sequence is computed on its
 * own.
 * ------------------------------------------------------------------------ */
int paged_attn_decode_window(const void* q, const void* k_pool, const void* v_pool,
                             const uint16_t* k_scales, const uint16_t* v_scales,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len,
                             int num_seqs, int num_blocks, int block_size,
                             int n_heads, int n_kv_heads, int d_head, int dtype, int kv_bits,
                             void* out, void* workspace, size_t workspace_bytes,
                             int partition_blocks, int window_tokens, void* stream);

/* ---------------------------------------------------------------------------
 * Causal prefill of a chunk ([JE] "Chunked prefill"; [TAI] "Scheduling
 * prefill and decode": a long prompt is split into chunks that run beside
 * decodes; each chunk is the same attention over the cache, split up).
 *
 * Sequence s contributes q_len_s = cu_q_lens[s+1] - cu_q_lens[s] query rows,
 * rows cu_q_lens[s] .. cu_q_lens[s+1]-1 of q. They are its last q_len_s
 * tokens: row i sits at absolute position context_lens[s] - q_len_s + i and
 * attends keys 0..that position (inclusive). The chunk's own K/V must already
 * be in the pool.
 * q, out        [total_q][n_heads][d_head] of dtype
 * cu_q_lens     int32 [num_seqs + 1] device prefix sums, cu_q_lens[0] = 0,
 *               cu_q_lens[num_seqs] = total_q, 0 <= q_len_s <= max_q_len,
 *               q_len_s <= context_lens[s]
 * other arguments as for paged_attn_decode (every pool format, fp8
 * included). No workspace: each chunk row is computed whole by one
 * workgroup.
 * ------------------------------------------------------------------------ */
int paged_attn_prefill_chunk(const void* q, const int32_t* cu_q_lens, int total_q, int max_q_len,
                             const void* k_pool, const void* v_pool,
                             const uint16_t* k_scales, const uint16_t* v_scales,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len,
                             int num_seqs, int num_blocks, int block_size,
                             int n_heads, int n_kv_heads, int d_head, int dtype, int kv_bits,
                             void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Sliding-window causal prefill of a chunk ([IR] "The memory equation":
 * sliding-window attention; [TAI] "The KV cache": sliding-window layers). As
 * paged_attn_prefill_chunk, but the row at absolute position p attends only
 * keys max(0, p - window_tokens + 1) .. p, the decode window's rule applied
 * to every row; window_tokens >= 1 (else PA_ERR_INVALID_ARG), and a window
 * reaching back past key 0 is the full causal prefill. Blocks wholly before
 * every row's window are not read.
 * ------------------------------------------------------------------------ */
int paged_attn_prefill_chunk_window(const void* q, const int32_t* cu_q_lens, int total_q, int max_q_len,
                                    const void* k_pool, const void* v_pool,
                                    const uint16_t* k_scales, const uint16_t* v_scales,
                                    const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* context_lens, int max_context_len,
                                    int num_seqs, int num_blocks, int block_size,
                                    int n_heads, int n_kv_heads, int d_head, int dtype, int kv_bits,
                                    void* out, int window_tokens, void* stream);

/* ---------------------------------------------------------------------------
 * Symmetric b-bit quantization of a bf16 pool ([JE] "KV-cache quantization":
 * each key/value becomes an integer sharing one scale s with its group).
 * Group = one (block, KV head) tile, 16 slots x d_head:
 *   s    = float16_rne( float32(amax |x|) / qmax ),  qmax = 127 (8 bit), 7 (4 bit)
 *   code = clamp( rint_half_even( x / float32(s) ), -qmax, qmax ), 0 if s == 0
 * (float32 IEEE division). src must be finite; a scale that overflows fp16
 * is stored as +inf with all codes 0.
 * bits = PA_KV_FP8 (fp8, the format the pages name as the usual cache
 * quantization: [TAI] "The KV cache"; [IR] "The debate"): qmax = 448, the
 * largest finite e4m3 value, and the code is the e4m3 value nearest
 * x / float32(s), ties to the even code, magnitudes past 448 saturating to
 * 448, the sign of x kept (-0 is 0x80); all codes 0x00 when s is 0 or +inf.
 * NaN codes are never written.
 * src     bf16 pool of `kind` (K or V layout, kv_bits = 16)
 * codes   pool of the same kind with kv_bits = bits (written)
 * scales  fp16 [num_blocks][n_kv_heads] (written for the processed blocks)
 * block_ids  int32 [n_ids] blocks to process, or NULL for all num_blocks
 *            (ids outside [0, num_blocks) are skipped)
 * ------------------------------------------------------------------------ */
int kv_quantize(const void* src, void* codes, uint16_t* scales,
                const int32_t* block_ids, int n_ids,
                int num_blocks, int n_kv_heads, int block_size, int d_head,
                int bits, int kind, void* stream);

/* ---------------------------------------------------------------------------
 * Write new tokens' keys/values into their slots ([TAI] "The KV cache":
 * each step computes K/V only for the new token and caches them; [IR]
 * "PagedAttention...": a table maps logical positions to physical slots).
 * k_src, v_src  [num_tokens][n_kv_heads][d_head] of dtype (either may be NULL)
 * slot_mapping  int64 [num_tokens]: slot = block * 16 + offset; a negative
 *               slot skips the token; slots >= num_blocks*16 are skipped.
 *               Slots should be distinct: where two tokens name one slot,
 *               which of them the slot ends up holding is unspecified.
 * k_pool, v_pool  pools with kv_bits = 32 (PA_F32) or 16 (PA_BF16), written
 *               only at the listed slots (other slots keep their bytes)
 * Speed: a block whose 16 slots are listed in order by 16 consecutive tokens
 * is written as whole K and V tiles; any other token costs one scattered
 * store per V element.
 * ------------------------------------------------------------------------ */
int paged_kv_write(const void* k_src, const void* v_src, const int64_t* slot_mapping, int num_tokens,
                   void* k_pool, void* v_pool, int num_blocks, int block_size,
                   int n_kv_heads, int d_head, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Append new tokens' keys/values through the block table ([TAI] "The KV
 * cache": each step computes K/V only for the new tokens and appends them;
 * [IR] "PagedAttention...": the table maps logical positions to physical
 * blocks). Sequence s appends n_s = cu_new[s+1] - cu_new[s] tokens, rows
 * cu_new[s] .. cu_new[s+1]-1 of k_new / v_new; they are its positions
 * context_lens[s] - n_s .. context_lens[s] - 1 (context_lens holds the
 * lengths after the append, as the decode takes them), and position t goes
 * to slot t % 16 of block block_tables[s * max_blocks_per_seq + t / 16]. A
 * decode step appends one token per sequence; a prefill chunk its tokens.
 * k_new, v_new  [total_new][n_kv_heads][d_head] of dtype (either may be NULL)
 * cu_new        int32 [num_seqs + 1] device prefix sums, 0 <= n_s <= max_new,
 *               n_s <= context_lens[s]
 * k_pool, v_pool  pools of kv_bits (written): 32 needs PA_F32, the others
 *               PA_BF16. For 32 / 16 only the new tokens' elements are
 *               written.
 * Quantized pools (kv_bits 8, 4, PA_KV_FP8; [JE] "KV-cache quantization"):
 * every block a call writes into gets the codes and fp16 scale that
 * kv_quantize would give for the tokens written into it so far, the slots
 * past the sequence's end counting as 0; so the block's scale is recomputed
 * with every write and is final once the block holds 16 tokens. The earlier
 * tokens of a partly filled block come from the sequence's staging tile:
 * k_stage, v_stage  bf16 [num_seqs][n_kv_heads][16][d_head] (read and
 *               written; NULL for 32 / 16). Row s holds, in slots
 *               0 .. (context_lens[s] - n_s) % 16 - 1, the earlier tokens of
 *               the block position context_lens[s] - n_s falls in; the call
 *               leaves in it the tokens of the block position
 *               context_lens[s] - 1 falls in, when that block is not full. The
 *               caller keeps a sequence's row across calls (copying it with
 *               the block on copy-on-write) and fills it for a sequence whose
 *               cache was quantized by kv_quantize with a partly filled last
 *               block.
 * k_scales, v_scales  fp16 [num_blocks][n_kv_heads] (written; quantized only)
 * Blocks a call writes must not be shared with another sequence of the same
 * call (copy them on write first). Table entries outside [0, num_blocks) are
 * recorded (pa_take_block_id_error) and nothing is written through them.
 * ------------------------------------------------------------------------ */
int paged_kv_append(const void* k_new, const void* v_new, const int32_t* cu_new, int total_new, int max_new,
                    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                    void* k_pool, void* v_pool, uint16_t* k_scales, uint16_t* v_scales,
                    void* k_stage, void* v_stage, int num_seqs, int num_blocks, int block_size,
                    int n_kv_heads, int d_head, int dtype, int kv_bits, void* stream);

/* ---------------------------------------------------------------------------
 * Copy whole blocks ([IR] "PagedAttention...": shared blocks are copied on
 * write when sequences diverge; the host block manager of
 * pa_block_manager.h reports the (source, destination) pairs).
 * For each of the n_pairs pairs in `pairs` (device int32 [n_pairs][2]:
 * source block, destination block), the block's tiles of every KV head are
 * copied in k_pool and in v_pool (either may be NULL), and for quantized
 * pools its fp16 scales in k_scales / v_scales (either may be NULL; both
 * must be NULL for kv_bits 32 or 16). Pairs naming a block outside
 * [0, num_blocks) are skipped. No destination may also appear as a source
 * in the same call (the copies run in parallel).
 * ------------------------------------------------------------------------ */
int pa_copy_blocks(void* k_pool, void* v_pool, uint16_t* k_scales, uint16_t* v_scales,
                   const int32_t* pairs, int n_pairs, int num_blocks, int n_kv_heads, int d_head,
                   int kv_bits, void* stream);

/* ---------------------------------------------------------------------------
 * HBM read probe: the read bandwidth this device reaches on the decode's
 * access pattern, the measured ceiling that the decode's bandwidth is
 * reported against beside the spec peak ([JE] "KV-cache quantization":
 * decode is bound by the bytes moved per step). buf holds buf_bytes / tile_bytes
 * tiles of tile_bytes (a multiple of 16, at most 65536). The tiles read are
 * order[0 .. n_order) (device int32 tile numbers; entries outside the
 * buffer are skipped), or with order NULL every tile of buf in turn.
 * Workgroup w of the grid (1..65536 workgroups of 256 threads) reads the
 * w-th, (w + grid)-th, (w + 2 grid)-th, ... of them with nontemporal
 * 16-byte loads and writes the XOR of every 32-bit word it read to
 * xor_out[w] (device uint32 [grid]). Nothing else is written.
 * ------------------------------------------------------------------------ */
/* ---------------------------------------------------------------------------
 * Block-table check ([IR] "PagedAttention: why fragmentation was eating most
 * of the rest": the table maps each logical block to a physical block of the
 * pool). Every kernel that follows a block table checks each entry it uses
 * against [0, num_blocks); an entry outside it is read as block 0 and the
 * first such entry per device is recorded (the check costs nothing while
 * every entry is valid). This takes the record of the current device:
 * returns 1 and sets *table_index (the entry's index in the block_tables
 * array of the call that met it: sequence * max_blocks_per_seq + logical
 * block) and *block_id (either pointer may be NULL), then clears it; returns
 * 0 if nothing was recorded since the last take; PA_ERR_HIP if the device
 * could not be read. Host; synchronous. Call it once the kernels of interest
 * have completed and while no call of this library runs on the device.
 * ------------------------------------------------------------------------ */
int pa_take_block_id_error(int64_t* table_index, int32_t* block_id);

int pa_hbm_read_probe(const void* buf, int64_t buf_bytes, int tile_bytes, const int32_t* order, int64_t n_order,
                      uint32_t* xor_out, int grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
