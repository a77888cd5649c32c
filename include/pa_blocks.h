/*
 * pa_blocks.h — host-side block manager with a prefix cache (C ABI).
 *
 * Pages (cited by title and section):
 *   [datawhale] "17. vLLM PagedAttention" (datawhalechina), Step 4 and the
 *               reference solution: a free list of physical blocks,
 *               ceil(len / block_size) blocks per prompt, one more block when
 *               a sequence crosses a block boundary, OOM when the free list
 *               runs short.
 *   [ybb]       "vLLM 与 LLM 推理部署实战" (ybb.press), §2.2: reference
 *               counts, copy-on-write of a shared block, reuse of cached
 *               blocks whose prefix hash matches (prefix caching).
 *   [bogosort]  "五十三：vLLM-PagedAttention", §16 Prefix Caching (the cache
 *               key is a hash; tenants are isolated; blocks are reference
 *               counted) and §17 Parallel Sampling (forks share prompt blocks
 *               and write into their own after the fork).
 *
 * This is host code: no call touches the GPU.  The block ids it hands out
 * index the device pools of pa.h; copy-on-write returns the (src, dst) pair
 * that pa_copy_blocks (or pa_copy_blocks_partial) must then perform.
 *
 * Rules (deterministic, so that a plain re-implementation gives the same ids):
 *  - free blocks leave from the front of a FIFO free list and return to its
 *    back; its initial order is `order` (a permutation of 0..num_blocks-1)
 *    or 0, 1, 2, ... when `order` is NULL;
 *  - full blocks of a prompt are keyed by FNV-1a-64 over the little-endian
 *    bytes of (parent key: uint64, namespace: uint64, the block's token ids:
 *    int32 each), the parent key of a prompt's first block being 0;
 *  - pa_bm_allocate_prompt reuses the longest chain of leading full blocks
 *    that are cached under the same keys with the same namespace, parent key
 *    and tokens, then hands out fresh blocks; each fresh full block is
 *    cached under its key unless that key is taken; a partial last block is
 *    not cached (pa_bm_register_blocks caches blocks once decode steps have
 *    filled them);
 *  - a cached block whose count drops to zero stays cached on an LRU list; a
 *    fresh block is taken from the free list, else by evicting the LRU front
 *    (it leaves the cache);
 *  - pa_bm_release drops a table's blocks last first (a prompt's tail is
 *    evicted before its head);
 *  - a call that returns PA_ERR_OUT_OF_BLOCKS or PA_ERR_INVALID_ARG changes
 *    nothing.
 * A handle is not thread safe; one thread at a time may use it.
 */
#ifndef PA_BLOCKS_H_
#define PA_BLOCKS_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* New manager over num_blocks blocks of block_size tokens (1..4096); `order`
 * (num_blocks entries, may be NULL) is the initial free-list order.  *out
 * receives the handle (NULL on error). */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* order,
                       pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* m);

/* Counters: blocks on the free list; cached blocks with no user (evictable);
 * cached blocks in all; the reference count of one block.  -1 on a bad
 * handle or block id. */
int32_t pa_bm_num_free(const pa_block_manager* m);
int32_t pa_bm_num_evictable(const pa_block_manager* m);
int32_t pa_bm_num_cached(const pa_block_manager* m);
int32_t pa_bm_ref_count(const pa_block_manager* m, int32_t block);

/* Blocks for a new prompt of num_tokens token ids: ceil(num_tokens /
 * block_size) ids written to blocks_out (capacity entries), of which the
 * first *num_cached_blocks_out (may be NULL) are prefix-cache hits whose K/V
 * are already in the pools; the caller prefills only the tokens after them. */
pa_status pa_bm_allocate_prompt(pa_block_manager* m, uint64_t namespace_id, const int32_t* tokens,
                                int32_t num_tokens, int32_t* blocks_out, int32_t capacity,
                                int32_t* num_blocks_out, int32_t* num_cached_blocks_out);

/* Cache the full blocks a sequence has filled since its prompt (multi-turn
 * prefix sharing, [intelli] §6.2): for each full block i of `tokens` (the
 * sequence's token ids so far), block table[i] is cached under the key of
 * tokens[0 .. (i+1) * block_size) in `namespace_id`, unless that block is
 * already cached or the key is taken.  Blocks must be in use; the caller
 * guarantees that the pools hold the K/V of these tokens.
 * *num_registered_out (may be NULL) receives the number of blocks added. */
pa_status pa_bm_register_blocks(pa_block_manager* m, uint64_t namespace_id, const int32_t* tokens,
                                int32_t num_tokens, const int32_t* table, int32_t num_blocks,
                                int32_t* num_registered_out);

/* Grow a table of num_blocks ids (array of capacity entries) so that it
 * covers new_len tokens; *num_blocks_out receives the new length.  Blocks
 * filled this way are not cached. */
pa_status pa_bm_append(pa_block_manager* m, int32_t* table, int32_t num_blocks, int32_t capacity,
                       int32_t new_len, int32_t* num_blocks_out);

/* A new sequence sharing every block of `table`: each count + 1. */
pa_status pa_bm_fork(pa_block_manager* m, const int32_t* table, int32_t num_blocks);

/* Before writing into logical block `logical` of `table`: if that block is
 * shared (count > 1), a fresh block replaces it in `table`, the old count
 * drops by one, and pair_out = {src, dst} names the copy the device must do;
 * otherwise pair_out = {-1, -1}. */
pa_status pa_bm_copy_on_write(pa_block_manager* m, int32_t* table, int32_t num_blocks,
                              int32_t logical, int64_t* pair_out);

/* A finished sequence: each block's count - 1 (see the rules above). */
pa_status pa_bm_release(pa_block_manager* m, const int32_t* table, int32_t num_blocks);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H_ */
