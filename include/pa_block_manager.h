/* Host-side block manager and scheduler step for a paged KV cache.
 *
 * CPU only: these calls allocate host memory for their own bookkeeping and
 * never touch the GPU. They produce the block tables, slot numbers and
 * copy-on-write pairs that the device entry points of paged_attn.h consume.
 *
 * What it implements ("KV cache, GQA, paging and continuous batching",
 * sections "PagedAttention: why fragmentation was eating most of the rest",
 * "Prefix caching: the biggest single lever most teams have" and "The
 * scheduler, and preemption"; "KV cache, continuous batching and paged
 * attention", sections "Paged attention" and "Prefix caching"):
 *   - a pool of num_blocks blocks of 16 tokens; each sequence has a block
 *     table, grown one block at a time as its tokens arrive, so at most its
 *     last block is partly filled;
 *   - forked sequences share blocks (reference counts); writing into a shared,
 *     partly filled last block first moves the writer to a fresh copy
 *     (copy-on-write: the caller copies the block's K/V, see pa_copy_blocks);
 *   - a prefix cache: every full block of a prompt is entered under the
 *     prompt's exact tokens up to the block's end (a trie of 16-token
 *     blocks, compared token by token, so different prefixes never share an
 *     entry); a later prompt reuses the blocks of its longest cached prefix
 *     of whole blocks;
 *   - a scheduler step that admits waiting requests while their prompts fit
 *     in free blocks and preempts the newest running sequence when another
 *     cannot get a block.
 * Rules where the pages are silent:
 *   - free blocks are a FIFO queue, initially 0 .. num_blocks-1; allocation
 *     takes the front; released blocks go to the back, a sequence's blocks
 *     last block first;
 *   - a cached block whose last reference goes away stays cached and becomes
 *     evictable (LRU order); allocation takes free blocks first, then evicts
 *     the least recently released cached block; a cache hit on an evictable
 *     block takes it back. Blocks of generated tokens are never cached;
 *   - an operation that cannot get the blocks it needs returns
 *     PA_ERR_NO_BLOCKS and changes nothing.
 * Handles are not thread-safe: one thread at a time per handle.
 * Sequence ids are caller-chosen int64 values.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#include "paged_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ERR_NO_BLOCKS (-5)   /* not enough free blocks; nothing changed      */
#define PA_ERR_NO_SEQUENCE (-6) /* unknown sequence id (or, for add/fork, taken) */

typedef struct pa_block_manager pa_block_manager;
typedef struct pa_scheduler pa_scheduler;

/* A manager of num_blocks (> 0) blocks; prefix_cache 0 or 1. NULL on invalid
 * arguments or host allocation failure. */
pa_block_manager* pa_bm_create(int num_blocks, int prefix_cache);
void pa_bm_destroy(pa_block_manager* bm);

/* Free blocks plus evictable cached blocks. */
int pa_bm_num_free(const pa_block_manager* bm);

/* Reference count of a block (0 when free or evictable); -1 if out of range. */
int pa_bm_ref_count(const pa_block_manager* bm, int block);

/* New sequence `seq` holding the n_tokens >= 0 prompt tokens `tokens`
 * (may be NULL when n_tokens is 0): ceil(n_tokens / 16) blocks, the leading
 * ones from the prefix cache where they match. *cached_tokens (may be NULL)
 * receives how many prompt tokens the cache held (a multiple of 16). */
int pa_bm_add(pa_block_manager* bm, int64_t seq, const int64_t* tokens, int n_tokens, int* cached_tokens);

/* Room for one more token of `seq`: a new block when its length is a
 * multiple of 16; if its last block is partly filled and shared, a fresh
 * block replaces it and *cow_src / *cow_dst (both required) name the block
 * to copy from and to, else both are -1. */
int pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t* cow_src, int32_t* cow_dst);

/* `child` (a new id) shares every block of `parent`. */
int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* Drop `seq` and its references. */
int pa_bm_release(pa_block_manager* bm, int64_t seq);

/* Tokens of `seq`, or a negative status. */
int pa_bm_num_tokens(const pa_block_manager* bm, int64_t seq);

/* Block table of `seq`: writes min(n, max_blocks) ids to row (may be NULL
 * when max_blocks is 0) and returns n, the number of blocks; or a negative
 * status. The KV slot of token position p is row[p / 16] * 16 + p % 16. */
int pa_bm_table(const pa_block_manager* bm, int64_t seq, int32_t* row, int max_blocks);

/* Scheduler over a manager (which must outlive it). NULL on failure. */
pa_scheduler* pa_sched_create(pa_block_manager* bm);
void pa_sched_destroy(pa_scheduler* s);

/* Queue request `seq` with its n_prompt >= 0 prompt tokens. */
int pa_sched_submit(pa_scheduler* s, int64_t seq, const int64_t* prompt, int n_prompt);

/* Submitted and not finished requests. */
int pa_sched_num_live(const pa_scheduler* s);

/* One step. First, waiting requests are admitted in order while
 * pa_bm_add succeeds for their tokens (the prompt plus tokens recorded
 * before a preemption); the first that does not fit stops admission. Then
 * every running sequence, oldest first, gets room for its next token
 * (pa_bm_append). When a block is missing, the newest running sequence is
 * preempted (released, and queued first among the waiting, to be recomputed)
 * and the append is tried again; the sequence needing the block may itself
 * be the newest. The only running sequence is never preempted: it is
 * reported as stalled and gets no room.
 * Outputs, each of capacity cap >= pa_sched_num_live(s) entries:
 *   running    ids that got room, oldest first (*n_running)
 *   preempted  ids preempted in this step, in order (*n_preempted)
 *   cow        copy-on-write pairs, cow[2i] = src, cow[2i+1] = dst (*n_cow;
 *              capacity 2 * cap int32 values)
 *   *n_stalled  0 or 1; the stalled id, if any, is not in running
 * Returns PA_ERR_INVALID_ARG (nothing done) if cap is too small. */
int pa_sched_step(pa_scheduler* s, int cap, int64_t* running, int* n_running, int64_t* preempted, int* n_preempted,
                  int32_t* cow, int* n_cow, int* n_stalled);

/* The token that running sequence `seq` produced at its newest position
 * (kept so that a preempted request is recomputed with it). */
int pa_sched_record(pa_scheduler* s, int64_t seq, int64_t token);

/* `seq` is done: removed from the running set, its blocks released. */
int pa_sched_finish(pa_scheduler* s, int64_t seq);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
