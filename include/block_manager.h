/*
 * block_manager.h -- C ABI of the host-side KV block manager: which
 * physical block of the pool holds which tokens of which sequence.
 *
 * The manager decides slots and block tables; the device library
 * (pagedkv.h) moves the bytes.  It follows the pages' block manager:
 *
 *   - a preallocated pool of equal blocks, handed out only when a token
 *     needs a slot, and returned as soon as nothing uses it ("vLLM 与 KV
 *     Cache", how-it-works points 1-4; "vLLM KV Cache 实现机制" §3.2 step 1
 *     and §4.1 pool diagram);
 *   - a block record with a reference count and a last-access stamp; blocks
 *     shared by several sequences (forked candidates, cached prefixes) are
 *     copied before the first write into them (copy-on-write) and are never
 *     evicted while referenced ("vLLM KV Cache 实现机制" §3.1 data structures
 *     and §3.2 point 3; "vLLM — 把操作系统的分页搬进 GPU KV cache", core
 *     mechanism 3 and case 2);
 *   - prefix caching: a full block is identified by its parent block, its
 *     exact tokens and an extra per-request hash (multimodal inputs); a new
 *     sequence whose leading full blocks match reuses them instead of
 *     recomputing their KV ("vLLM KV Cache 实现机制" §4.2, the three inputs of
 *     the hash match);
 *   - LRU eviction of cached blocks that no sequence references, when no
 *     plain free block is left (§3.2, LRU + RefCount);
 *   - the free-block count the pages watch during generation ("vLLM — 把操作
 *     系统的分页搬进 GPU KV cache", case 2, get_num_free_blocks).
 *
 * Policy where the pages leave a choice open:
 *   - Plain free blocks (holding no cached prefix) leave from the front of
 *     the free list in its initial order and return at its back.  Only when
 *     none is left is a cached, unreferenced block evicted, least recently
 *     used first.
 *   - A freed sequence releases its blocks from the last to the first, so a
 *     prefix's deeper blocks are evicted before the blocks they extend.
 *   - A block's prefix identity is the registration of its parent block (not
 *     a hash value alone): a lookup matches only if the parent registration,
 *     the extra hash and every token are equal, so hash collisions cannot
 *     produce a false hit, and a block whose parent was evicted is unreachable.
 *   - Full blocks are registered when their last slot is reserved, and only
 *     when the sequence's tokens are known and its previous block is
 *     registered.  Partial blocks are never shared through the cache.
 *   - Every matching full block is reused, including a prompt's last one.
 *
 * A manager is not thread-safe: one owner thread drives it.  Sequence ids
 * are caller-chosen int64 values.  Every call either succeeds or leaves the
 * manager unchanged (checked before any state is modified).
 */
#ifndef BLOCK_MANAGER_H_
#define BLOCK_MANAGER_H_

#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bm_manager bm_manager_t;  /* opaque, host memory */

typedef struct {
  int64_t num_blocks;
  int64_t free_blocks;     /* unreferenced, holding no cached prefix */
  int64_t cached_blocks;   /* unreferenced, holding a cached prefix (evictable) */
  int64_t used_blocks;     /* referenced by at least one sequence */
  int64_t num_sequences;
  int64_t tokens;          /* sum of sequence lengths */
  int64_t table_entries;   /* sum of sequence table lengths (a shared block counts once per sequence) */
  int64_t prefix_queries;  /* full blocks looked up by bm_add_sequence */
  int64_t prefix_hits;     /* of which found in the cache and reused */
  int64_t evictions;       /* cached blocks evicted to make room */
  int64_t cow_copies;      /* copy-on-write pairs handed out */
  int64_t allocations;     /* blocks taken from the free list or by eviction */
} bm_stats_t;

/* Create a manager for a pool of num_blocks blocks of block_size tokens.
 * free_order (num_blocks ids, a permutation of 0..num_blocks-1) sets the
 * initial free list; NULL means 0, 1, 2, ...  prefix_caching != 0 enables
 * the prefix cache.  KV_ERR_INVALID_ARG on bad sizes or a free_order that is
 * not a permutation; KV_ERR_OOM if host memory runs out. */
kv_status_t bm_create(int64_t num_blocks, int32_t block_size, const int32_t* free_order, int32_t prefix_caching,
                      bm_manager_t** out);
void bm_destroy(bm_manager_t* bm);

/* Register sequence `seq` with its first num_tokens tokens and reserve their
 * slots: slots[i] = block * block_size + offset of token i (caller-owned,
 * num_tokens int64 entries).  tokens (may be NULL: no prefix caching for
 * this sequence) are the token ids; extra_hash distinguishes requests whose
 * tokens agree but whose other inputs differ.  *num_cached (may be NULL)
 * receives how many leading tokens were found in the prefix cache: their KV
 * is already in the pool and need not be written again.
 * KV_ERR_INVALID_ARG: seq exists, num_tokens < 0 or a NULL slots with
 * num_tokens > 0.  KV_ERR_NO_BLOCKS: not enough free or evictable blocks
 * (nothing changes; the caller preempts a sequence). */
kv_status_t bm_add_sequence(bm_manager_t* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                            uint64_t extra_hash, int64_t* slots, int32_t* num_cached);

/* Each child starts as a copy of the parent's table and shares its blocks
 * (reference counts rise by one per child).  KV_ERR_INVALID_ARG if the parent
 * is unknown, a child exists or repeats. */
kv_status_t bm_fork(bm_manager_t* bm, int64_t parent, const int64_t* children, int32_t num_children);

/* Reserve the slots of the sequence's next `count` tokens (slots: count
 * int64 entries).  If the last block is shared, the first new token gets a
 * fresh block and the pair (shared, fresh) is written to copy_pairs (caller
 * capacity: 2 int32 entries; *num_pairs = 0 or 1): the device must copy it
 * (copy_blocks) before the new tokens are written.  tokens may be NULL (the
 * sequence's blocks from here on are not registered in the prefix cache).
 * KV_ERR_NO_BLOCKS leaves everything unchanged. */
kv_status_t bm_append_slots(bm_manager_t* bm, int64_t seq, const int32_t* tokens, int32_t count, int64_t* slots,
                            int32_t* copy_pairs, int32_t* num_pairs);

/* One step for a batch: reserve counts[i] slots for sequence seqs[i], in
 * list order, as bm_append_slots would one by one (a block shared by several
 * listed sequences is copied by each writer but the last).  slots receives
 * sum(counts) entries in list order; copy_pairs (capacity 2 * n int32) the
 * copy pairs in the order they arise.  tokens (may be NULL) holds sum(counts)
 * ids in the same order.  All or nothing: KV_ERR_NO_BLOCKS if the whole batch
 * does not fit, with nothing changed.  KV_ERR_INVALID_ARG for an unknown or
 * repeated sequence or a negative count. */
kv_status_t bm_append_batch(bm_manager_t* bm, const int64_t* seqs, const int32_t* counts, int32_t n,
                            const int32_t* tokens, int64_t* slots, int32_t* copy_pairs, int32_t* num_pairs);

/* Release the sequence: each block's count drops by one; a block reaching
 * zero goes back to the free list, or to the LRU list if it holds a cached
 * prefix. */
kv_status_t bm_free(bm_manager_t* bm, int64_t seq);

/* Blocks that can be handed out without preempting: free + cached. */
kv_status_t bm_num_free_blocks(const bm_manager_t* bm, int64_t* n);

kv_status_t bm_sequence_info(const bm_manager_t* bm, int64_t seq, int32_t* length, int32_t* num_blocks);

/* The sequence's table (physical block of each logical block) into out
 * (capacity entries; KV_ERR_INVALID_ARG if it has more blocks). */
kv_status_t bm_block_table(const bm_manager_t* bm, int64_t seq, int32_t* out, int32_t capacity);

/* Device-ready views for n sequences: out [n][max_blocks] int32 padded with
 * -1, and context_lens [n] (may be NULL).  KV_ERR_INVALID_ARG if a sequence
 * is unknown or has more than max_blocks blocks. */
kv_status_t bm_block_tables(const bm_manager_t* bm, const int64_t* seqs, int32_t n, int32_t max_blocks, int32_t* out,
                            int32_t* context_lens);

kv_status_t bm_ref_count(const bm_manager_t* bm, int32_t block, int32_t* ref);
kv_status_t bm_stats(const bm_manager_t* bm, bm_stats_t* out);

#ifdef __cplusplus
}
#endif

#endif /* BLOCK_MANAGER_H_ */
