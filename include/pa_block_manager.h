/*
 * pa_block_manager.h - C ABI of the host-side KV block manager in libpa.so.
 *
 * The manager is the bookkeeping that produces what the kernels consume: block tables,
 * the slot of every new token, and copy-on-write (src, dst) pairs. It follows the pages:
 *   - a free list of physical blocks; a sequence gets a new block only when its last one
 *     is full (vLLM-PagedAttention与连续批处理技术拆解, section 3.2; the intelliparadigm
 *     article, section 3.1), so the only waste is the unfilled tail of each sequence's
 *     last block (serving-engine article, section 2);
 *   - reference counts for blocks shared between sequences (parallel sampling, beam
 *     search); a shared block is read-only and a sequence that must write into it copies
 *     it first (copy-on-write: vLLM-PagedAttention与连续批处理技术拆解, section 3.4;
 *     serving-engine article, section 2);
 *   - prefix caching (serving-engine article, section 4): every FULL block gets a key
 *     chained from the previous block's key, the block's token ids and extra data (a
 *     salt), so one key stands for the whole prefix up to that block; a new sequence
 *     whose prompt blocks match cached keys reuses those blocks instead of prefilling
 *     them; released cached blocks keep their contents in an evictable queue and are
 *     evicted least-recently-used first, a finished sequence's blocks entering tail first.
 *
 * Policy details (the pages leave them open; the oracle implements the same):
 *   - The free list starts as 0, 1, ..., N-1 and is first-in first-out: allocation takes
 *     its head, blocks freed without a cache key go to its tail.
 *   - Allocation uses the free list first, then evicts the head of the evictable queue
 *     (dropping its key). With neither, the call fails with PA_ERR_NO_BLOCKS and changes
 *     nothing.
 *   - Block key: FNV-1a 64-bit over the bytes prev_key (8, little-endian), salt (8, LE),
 *     then the block_size token ids (4 bytes each, LE); prev_key = 0 for a sequence's
 *     first block. A hit also requires the cached block's token ids to be equal, so a
 *     hash collision can never alias two prefixes. When a full block's key is already
 *     cached by another block, the first one stays cached and the new one is not.
 *   - Keys are registered when a block becomes full: the full prompt blocks when a
 *     sequence is added, later blocks when an appended token fills them. The caller
 *     writes the K/V of every non-cached token (prompt or appended) at the slots the
 *     manager reports, before any later call can hand those blocks out.
 *   - Releasing a sequence decrements its blocks' counts from the last block to the
 *     first; a block reaching zero goes to the tail of the evictable queue if it is
 *     cached, else to the tail of the free list. Reusing an evictable block (a cache hit)
 *     removes it from the queue.
 *
 * Conventions: all pointers are HOST pointers; the handle is not thread-safe (one caller
 * at a time); nothing touches the GPU. Errors are pa_status_t return codes (see
 * paged_attention.h) plus the three below; a failing call changes no state (except
 * PA_ERR_NO_MEMORY).
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ERR_NO_BLOCKS (-8)    /* not enough free or evictable blocks */
#define PA_ERR_UNKNOWN_SEQ (-9)  /* no such sequence id, or the id is already in use */
#define PA_ERR_NO_MEMORY (-10)   /* host memory ran out inside the manager; its state is then
                                    unspecified and the handle should only be destroyed */

typedef struct pa_block_manager pa_block_manager_t;

/* New manager over num_blocks physical blocks of block_size tokens (block_size in
 * [1, 1024], num_blocks in [1, 2^30]); prefix caching on when enable_prefix_cache != 0.
 * Returns NULL on bad arguments or allocation failure. */
pa_block_manager_t* pa_bm_create(int32_t num_blocks, int32_t block_size,
                                 int32_t enable_prefix_cache);
void pa_bm_destroy(pa_block_manager_t* bm);

/* Add sequence seq_id (must be new) with its prompt tokens[0..n) (n >= 0) and cache salt.
 * Full prompt blocks found in the prefix cache are reused (refcount + 1); the rest are
 * allocated. *num_cached (may be NULL) receives the number of leading prompt tokens whose
 * K/V are already in the cache (a multiple of block_size): only tokens from there on need
 * computing and writing. */
int32_t pa_bm_add(pa_block_manager_t* bm, int64_t seq_id, const int32_t* tokens, int32_t n,
                  uint64_t salt, int32_t* num_cached);

/* Append one token to seq_id. Allocates a block when the last one is full (or there is
 * none); copies on write when the last block is partial and shared: a new block is
 * allocated, the old one's count drops, and (*cow_src, *cow_dst) receive the pair for
 * pa_block_copy (else both -1). *slot receives the token's slot (block * block_size +
 * offset) for pa_cache_write. Output pointers may be NULL. */
int32_t pa_bm_append(pa_block_manager_t* bm, int64_t seq_id, int32_t token, int64_t* slot,
                     int64_t* cow_src, int64_t* cow_dst);

/* One decode step's appends in a single call: token tokens[i] to sequence seq_ids[i], in
 * order, exactly as n calls of pa_bm_append. slots[i] receives each token's slot; the
 * copy-on-write pairs are packed into cow_pairs[2 * k] (src, dst), k = *num_cow (at most n),
 * ready for one pa_block_copy before the step's pa_cache_write. Stops at the first failing
 * append: *done (required) receives the number applied, which stay applied, and the
 * failure's code is returned (PA_OK when all n are done). */
int32_t pa_bm_append_batch(pa_block_manager_t* bm, const int64_t* seq_ids,
                           const int32_t* tokens, int32_t n, int64_t* slots, int64_t* cow_pairs,
                           int32_t* num_cow, int32_t* done);

/* New sequence child sharing every block of parent (each count + 1): parallel sampling
 * and beam-search forks. */
int32_t pa_bm_fork(pa_block_manager_t* bm, int64_t parent_id, int64_t child_id);

/* Release seq_id (see the policy above). */
int32_t pa_bm_free(pa_block_manager_t* bm, int64_t seq_id);

/* Slots of token positions [first, first + count) of seq_id into slots[count]. */
int32_t pa_bm_slots(const pa_block_manager_t* bm, int64_t seq_id, int32_t first,
                    int32_t count, int64_t* slots);

/* Block table row of seq_id: its blocks in order, then -1 up to width. Returns the number
 * of blocks, or PA_ERR_SHAPE if width is smaller. */
int32_t pa_bm_block_table(const pa_block_manager_t* bm, int64_t seq_id, int32_t* row,
                          int32_t width);

/* Block tables [n, width] and context lengths [n] of n sequences (the kernels' inputs). */
int32_t pa_bm_tables(const pa_block_manager_t* bm, const int64_t* seq_ids, int32_t n,
                     int32_t* tables, int32_t width, int32_t* context_lens);

/* Tokens held by seq_id, or PA_ERR_UNKNOWN_SEQ. */
int32_t pa_bm_seq_len(const pa_block_manager_t* bm, int64_t seq_id);

/* Reference count of a physical block (0 for free or evictable blocks), or PA_ERR_SHAPE. */
int32_t pa_bm_refcount(const pa_block_manager_t* bm, int32_t block);

/* Cache key of block j of seq_id into *key; PA_ERR_SHAPE if that block is not full. */
int32_t pa_bm_block_key(const pa_block_manager_t* bm, int64_t seq_id, int32_t j,
                        uint64_t* key);

/* Counts: blocks on the free list, in the evictable queue, and holding a cache key. */
int32_t pa_bm_stats(const pa_block_manager_t* bm, int32_t* num_free, int32_t* num_evictable,
                    int32_t* num_cached);

/* Physical blocks in eviction order (head first) into out[cap]; returns the count. */
int32_t pa_bm_evictable(const pa_block_manager_t* bm, int32_t* out, int32_t cap);

/* Preemption by swapping (vLLM-PagedAttention与连续批处理技术拆解, section 4.3): a victim's
 * blocks move to host memory and come back when device blocks are free again. The host pool
 * has host_blocks blocks with its own FIFO free list (0 .. host_blocks-1); call this once,
 * before any swap (PA_ERR_SHAPE if called twice or host_blocks < 1). */
int32_t pa_bm_set_host_blocks(pa_block_manager_t* bm, int32_t host_blocks);

/* Swap seq_id out: every block gets a host block (in order, from the host free list), the
 * (device block, host block) pairs go to pairs[2 * nb] for pa_block_swap(host pool <- device
 * pool), and the device blocks are released as pa_bm_free releases them (a cached block stays
 * findable until evicted). The sequence keeps its tokens and keys but has no device blocks
 * until swapped in; append and fork fail on it (PA_ERR_UNSUPPORTED), as does swapping out a
 * sequence with a shared block (count > 1): sharing sequences are preempted together by
 * recomputation instead. Returns nb, PA_ERR_NO_BLOCKS if the host pool is short, or
 * PA_ERR_SHAPE if cap < nb. */
int32_t pa_bm_swap_out(pa_block_manager_t* bm, int64_t seq_id, int64_t* pairs, int32_t cap);

/* Swap seq_id back in: fresh device blocks (allocated as usual), the (host block, device
 * block) pairs into pairs[2 * nb] for pa_block_swap(device pool <- host pool), host blocks
 * back to the tail of the host free list, and full blocks registered in the prefix cache
 * under their keys when those are free. Returns nb or an error (nothing changed). */
int32_t pa_bm_swap_in(pa_block_manager_t* bm, int64_t seq_id, int64_t* pairs, int32_t cap);

/* Blocks on the host free list. */
int32_t pa_bm_host_free(const pa_block_manager_t* bm);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
