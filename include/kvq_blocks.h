/*
 * kvq_blocks.h -- host-side block manager for the paged pools of kvq.h.
 *
 * Hands out the block ids that kvq_reshape_and_cache's slot_mapping and
 * kvq_paged_decode's block_tables refer to.  One block id addresses the
 * same block in every pool built from it: every layer's K and V pools, each
 * laid out by its own kvq_layout (per-layer formats and dims), hold
 * num_blocks blocks.
 *
 * Sources (web pages, cited by title and item):
 *   [kv_cache.rs]  "spark_runtime/kv_cache.rs" -- PagedKvCache: free_blocks,
 *                  block_ref_counts (a count per block so that blocks can be
 *                  shared, e.g. by a common prefix; 1 when handed out, back to
 *                  the free list when it drops to 0), per-layer dtypes and
 *                  (num_kv_heads, head_dim) in KvCacheConfig; release clears
 *                  the bookkeeping with the pools.
 *   [kv.rs]        "combs_models/kv.rs" -- PageAllocator (a stack of free page
 *                  ids, filled so that page 0 is handed out first), the paged
 *                  cache's ensure_pages (pages appended until the table covers
 *                  the length; an exhausted allocator is an error), popn (drop
 *                  the last n tokens and free the trailing pages no longer
 *                  used; returns how many were dropped), reset, pages_used.
 *
 * Host memory only: the manager allocates its own host bookkeeping (freed by
 * kvq_blocks_destroy) and never touches device memory.  Every call is
 * serialized by a lock inside the manager.  A call that fails returns a
 * negative kvq_status and leaves the manager unchanged.
 *
 * Shared blocks: kvq_blocks_fork gives a new sequence the parent's blocks
 * (their counts go up).  Appending to a sequence whose last block is shared
 * and partly filled would overwrite the other owners' rows, so the append
 * first moves the sequence onto a fresh block (copy on write) and reports the
 * pair: the caller copies block *cow_src to block *cow_dst in every pool
 * (k and v, every layer; block_stride bytes each) before writing the new rows.
 */
#ifndef KVQ_BLOCKS_H
#define KVQ_BLOCKS_H

#include <stdint.h>

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvq_blocks kvq_blocks;  /* opaque */

/* Any call that needs host memory it cannot get returns KVQ_ERR_HOST_MEMORY
 * and leaves the manager as it was. */

/* A manager of num_blocks blocks (1 <= num_blocks <= 2^31 - 1) of block_size
 * positions (>= 1).  *out receives the handle.  KVQ_ERR_INVALID_ARG on a bad
 * size or out == NULL. */
int kvq_blocks_create(uint32_t num_blocks, uint32_t block_size, kvq_blocks** out);

/* Frees the manager (NULL is a no-op). */
void kvq_blocks_destroy(kvq_blocks* bm);

/* Drops every sequence; every block is free again, handed out from block 0. */
int kvq_blocks_reset(kvq_blocks* bm);

/* Free blocks; the count of one block (0 when free). */
int kvq_blocks_num_free(kvq_blocks* bm, uint32_t* num_free);
int kvq_blocks_ref_count(kvq_blocks* bm, uint32_t block, uint32_t* count);

/* A new, empty sequence; *seq is the lowest id not in use. */
int kvq_blocks_seq_new(kvq_blocks* bm, uint32_t* seq);

/* A new sequence (lowest free id) that shares all of `parent`'s blocks and
 * has its length. */
int kvq_blocks_seq_fork(kvq_blocks* bm, uint32_t parent, uint32_t* child);

/* Releases the sequence's blocks, last block first, and retires its id. */
int kvq_blocks_seq_free(kvq_blocks* bm, uint32_t seq);

/* Length in positions and number of blocks (pages_used) of a sequence. */
int kvq_blocks_seq_len(kvq_blocks* bm, uint32_t seq, uint32_t* len, uint32_t* num_blocks);

/* Appends n positions to `seq`: blocks are taken from the free stack until
 * the table covers len + n positions (after the copy on write described
 * above, if the last block needs it).  slots (host, int64[n]) receives
 * block * block_size + offset of positions len .. len + n - 1, ready for
 * kvq_reshape_and_cache.  *cow_src / *cow_dst (host) receive the block pair to
 * copy, or -1 / -1.  KVQ_ERR_EXHAUSTED (nothing changed) if the free blocks
 * do not suffice; KVQ_ERR_INVALID_ARG for an unknown sequence, a NULL pointer
 * or a length past 2^31 - 1. */
int kvq_blocks_append(kvq_blocks* bm, uint32_t seq, uint32_t n, int64_t* slots, int32_t* cow_src,
                      int32_t* cow_dst);

/* One decode or prefill step for many sequences in one call: appends
 * counts[i] positions to seqs[i] (distinct ids), in list order, as
 * kvq_blocks_append would.  slots (host, int64[sum of counts]) receives the
 * slots of seqs[0]'s new positions, then seqs[1]'s, ...; cow (host,
 * int32[2 * num_seqs]) the copy pair of each sequence, or -1 / -1.  The free
 * blocks are checked first against every sequence's own need (its new blocks,
 * plus one if its last block is shared and partly filled): KVQ_ERR_EXHAUSTED,
 * nothing changed, if they fall short.  KVQ_ERR_INVALID_ARG for an unknown or
 * repeated id or a NULL pointer. */
int kvq_blocks_append_many(kvq_blocks* bm, const uint32_t* seqs, const uint32_t* counts, uint32_t num_seqs,
                           int64_t* slots, int32_t* cow);

/* Rolls back the last min(n, len) positions; blocks past the new last one
 * are released, last first.  *popped (host) receives the count. */
int kvq_blocks_popn(kvq_blocks* bm, uint32_t seq, uint32_t n, uint32_t* popped);

/* Block tables and lengths for kvq_paged_decode: row i of block_tables (host,
 * int32[num_seqs][max_blocks_per_seq]) holds seqs[i]'s blocks, then -1;
 * seq_lens (host, int32[num_seqs]) their lengths.  KVQ_ERR_INVALID_ARG
 * (nothing written) if a sequence is unknown or has more blocks than
 * max_blocks_per_seq. */
int kvq_blocks_table(kvq_blocks* bm, const uint32_t* seqs, uint32_t num_seqs, uint32_t max_blocks_per_seq,
                     int32_t* block_tables, int32_t* seq_lens);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_BLOCKS_H */
