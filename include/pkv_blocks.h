/*
 * pkv_blocks.h -- C ABI of the host-side KV block manager in libpkv.so.
 *
 * It owns the bookkeeping of a physical block pool of 16-token blocks and
 * emits what the device entry points of pkv.h consume: block tables, slot
 * mappings, prefix groups for pkv_paged_attention_decode_shared_prefix, and
 * block copies for copy-on-write (pkv_copy_blocks). It is plain host C++:
 * no call touches the GPU.
 *
 * What it follows ([ttlab] = "Basics of LLM Inference and vLLM Internals:
 * KV Cache, PagedAttention, and Scheduler"):
 *  - [ttlab] section 4: each request maps its logical blocks to physical
 *    blocks through a block table, taking physical blocks one at a time as it
 *    grows; waste is only the empty rows of its last block; identical
 *    prefixes share one physical block by reference counting, with
 *    copy-on-write; the pool keeps its free blocks in a doubly linked queue
 *    and reserves block 0 as the null block (1,345 blocks -> 1,344 usable).
 *  - [ttlab] section 5: a cached block is named by a hash chained from its
 *    parent block's hash, its own tokens and extra keys; only full blocks are
 *    cached, so only prefixes hit, in multiples of 16 tokens, and the last
 *    prompt token is always recomputed; a finished request's blocks keep
 *    their hashes in the free queue, which is consumed from the front, and
 *    are returned tail block first, so tail blocks are evicted first.
 *  - [ttlab] sections 9 and 10: the block LRU model whose three passes over
 *    ten 5,033-token documents in 1,344 usable blocks give 0, 0 and 21,488
 *    cached tokens. Its reading that a free block holding no cached hash
 *    (never used, or a request's partial last block) is reused before any
 *    cached block is evicted is taken here: such blocks enter the free queue
 *    at its front.
 *
 * Conventions: functions return PKV_OK or a negative PKV_ERR_* (pkv.h) unless
 * stated. All pointers are host memory. A manager is not thread-safe: one
 * thread at a time per manager. Request ids are caller-chosen int64 values.
 */
#ifndef PKV_BLOCKS_H
#define PKV_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

/* A manager over physical blocks 0 .. num_blocks - 1 of 16 tokens (block 0 is
 * the null block and never handed out; num_blocks >= 2). prefix_caching != 0
 * enables the hash-chain prefix cache. NULL for invalid sizes. */
pkv_block_manager *pkv_bm_create(int32_t num_blocks, int32_t prefix_caching);
void pkv_bm_destroy(pkv_block_manager *bm);

/* Blocks that can be handed out now: the free queue's length (never-used
 * blocks and cached blocks no request holds). num_blocks - 1 on a fresh
 * manager. */
int32_t pkv_bm_num_free_blocks(const pkv_block_manager *bm);

/* Register a request with its prompt tokens (host array of num_tokens >= 1
 * int64 token ids) and an optional extra key (a salt or adapter id that
 * enters every block hash; 0 for none). With prefix caching, the longest
 * chain of cached full blocks covering at most num_tokens - 1 tokens is
 * taken (reference counts raised, free ones leave the free queue) and becomes
 * the start of the request's block table; *num_cached_tokens gets its length
 * (a multiple of 16). The rest of the prompt still needs pkv_bm_append.
 * Errors: INVALID_ARG (bad pointer or size, id already present). */
int pkv_bm_add_request(pkv_block_manager *bm, int64_t request_id, const int64_t *prompt_tokens,
                       int32_t num_tokens, uint64_t extra_key, int32_t *num_cached_tokens);

/* Admission check: can the request's next n tokens get their slots now
 * (new blocks, plus one for copy-on-write of a shared partial last block)?
 * Returns 1 or 0; 0 also for an unknown request or n < 0. */
int pkv_bm_can_append(const pkv_block_manager *bm, int64_t request_id, int32_t n);

/* Give the request's next n tokens KV slots. The tokens are the next n of its
 * prompt while any are left, then the n ids in new_tokens (generated tokens;
 * new_tokens may be NULL while the prompt is not exhausted). Writes
 * slot_mapping[0..n) (block * 16 + row, for pkv_kv_append). Blocks are taken
 * from the front of the free queue; a cached block taken that way loses its
 * hash (eviction). If the request's last block is shared and not full, it is
 * first replaced by a new block: *num_copies = 1 and copies[0] = {src, dst}
 * must be copied on the device (pkv_copy_blocks) before the append; else
 * *num_copies = 0. Full blocks are registered in the prefix cache as they
 * fill. Errors: INVALID_ARG (unknown request, n < 0, tokens missing),
 * WORKSPACE (not enough free blocks: nothing changes). */
int pkv_bm_append(pkv_block_manager *bm, int64_t request_id, int32_t n, const int64_t *new_tokens,
                  int64_t *slot_mapping, int32_t copies[][2], int32_t *num_copies);

/* New request child_id sharing every block of parent_id (reference counts
 * raised; parallel sampling). The next append to either into a shared
 * partial block copies it first. Errors: INVALID_ARG. */
int pkv_bm_fork(pkv_block_manager *bm, int64_t parent_id, int64_t child_id);

/* Drop a request: its blocks are released last block first; a block whose
 * count reaches zero enters the free queue at the back if it holds a cached
 * hash (evicted last), at the front if not. Errors: INVALID_ARG. */
int pkv_bm_free_request(pkv_block_manager *bm, int64_t request_id);

/* Tokens with slots (context length) and blocks of a request; -1 if unknown. */
int32_t pkv_bm_num_tokens(const pkv_block_manager *bm, int64_t request_id);
int32_t pkv_bm_num_blocks(const pkv_block_manager *bm, int64_t request_id);

/* Reference count of physical block `block` (0 for free or null). */
int32_t pkv_bm_ref_count(const pkv_block_manager *bm, int32_t block);

/* Block tables of n requests as int32 [n][max_blocks], rows padded with the
 * null block 0, and their context lengths (int32 [n], may be NULL). Errors:
 * INVALID_ARG (unknown request), UNSUPPORTED (a request has more than
 * max_blocks blocks). */
int pkv_bm_block_tables(const pkv_block_manager *bm, const int64_t *request_ids, int32_t n,
                        int32_t max_blocks, int32_t *block_tables, int32_t *context_lens);

/* Prefix groups of a batch in the given order, for
 * pkv_paged_attention_decode_shared_prefix: maximal runs of adjacent
 * requests whose first block is the same physical block; a run's shared
 * count is the number of leading blocks all its members hold in common and
 * full (0 for runs of one). group_starts gets num_groups + 1 entries (at most
 * n + 1) and group_prefix_blocks num_groups (at most n); *num_groups is set.
 * Errors: INVALID_ARG. */
int pkv_bm_prefix_groups(const pkv_block_manager *bm, const int64_t *request_ids, int32_t n,
                         int32_t *group_starts, int32_t *group_prefix_blocks,
                         int32_t *num_groups);

/* Prefix-cache counters since creation: tokens looked up (prompt tokens of
 * added requests) and tokens hit. */
void pkv_bm_prefix_cache_stats(const pkv_block_manager *bm, int64_t *queried_tokens,
                               int64_t *hit_tokens);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCKS_H */
