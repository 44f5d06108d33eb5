/*
 * pa_blocks.h — host-side KV block manager: the pool of cache blocks, per-
 * sequence block tables and prefix reuse by token-block hashing, producing
 * the block_tables / slot_mapping / context_lens / cu_seqlens arrays that the
 * kernels of pa.h consume.
 *
 * Page "nano-vLLM 最小化vLLM重新实现", section 3 "块管理器": fixed-size KV
 * blocks are handed out from a pool; each block tracks a reference count and
 * a hash; allocation looks up cached prefix blocks by hash and allocates only
 * the remainder; token blocks are hashed (xxhash) for automatic prefix
 * caching; preemption releases a sequence's blocks. Page at
 * hotelren.com/news/2273631, section 2.2: a sequence's block list is its page
 * table; section 4.4: a cached prefix is reused and only the rest computed.
 *
 * Policy (where the pages are silent):
 *  - A full block's hash chains through its prefix: h_i = XXH64(token ids of
 *    block i as little-endian int32, seed h_{i-1}), h_{-1} = 0 (XXH64 as
 *    published by its author, implemented here). Only full blocks are hashed;
 *    a hit also compares the token ids; matching stops at the first miss; at
 *    most (n - 1) / block_size blocks of an n-token prompt come from the cache.
 *  - The free list is a queue: blocks are taken from its front; a released
 *    sequence's blocks go to its back, last block first. A released block keeps
 *    its hash (a later prompt can still hit it) until it is taken for new
 *    content. A hash is registered only if not already present.
 *  - A call that lacks blocks returns PA_ERR_NO_BLOCKS and changes nothing.
 *
 * All arrays are host memory owned by the caller. A manager is not thread
 * safe: one caller at a time. Status codes are those of pa.h.
 */
#ifndef PA_BLOCKS_H_
#define PA_BLOCKS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* XXH64 of len bytes with the given seed (the published 64-bit xxHash). */
uint64_t pa_xxh64(const void* data, size_t len, uint64_t seed);

/*
 * New manager over blocks 0 .. num_blocks - 1 of block_size tokens. order
 * (optional, num_blocks entries, a permutation) is the initial free-list
 * order; NULL means ascending. *out receives the manager (NULL on error).
 */
int pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* order, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/*
 * Blocks for a new sequence's prompt of num_tokens token ids. *num_cached
 * receives how many leading prompt tokens sit in blocks reused from the cache
 * (a multiple of block_size; their K/V need not be computed or stored).
 * Errors: unknown manager or negative size (PA_ERR_INVALID_ARGUMENT), seq_id
 * already live (PA_ERR_INVALID_ARGUMENT), too few free blocks
 * (PA_ERR_NO_BLOCKS).
 */
int pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                   int32_t* num_cached);

/* One more token for a live sequence (decode); takes a block when the last one
 * is full (PA_ERR_NO_BLOCKS if none is free). Unknown seq_id: PA_ERR_NOT_FOUND. */
int pa_bm_append(pa_block_manager* bm, int64_t seq_id, int32_t token);

/* One decode step for many sequences: appends tokens[i] to seq_ids[i] in order
 * and stops at the first failure, returning its status; *num_done receives how
 * many appends were made (those stay made). */
int pa_bm_append_batch(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* tokens, int32_t count,
                       int32_t* num_done);

/* Release a finished or preempted sequence (PA_ERR_NOT_FOUND if unknown). */
int pa_bm_free(pa_block_manager* bm, int64_t seq_id);

/* Number of free blocks; tokens held by a sequence (-1 if unknown). */
int32_t pa_bm_num_free(const pa_block_manager* bm);
int32_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq_id);

/* The sequence's block table: its ceil(len / block_size) block ids in order
 * (*num_blocks receives the count; PA_ERR_INVALID_ARGUMENT if capacity is too small). */
int pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out, int32_t capacity,
                      int32_t* num_blocks);

/* The free list in order, and a block's reference count (-1 if out of range). */
int pa_bm_free_list(const pa_block_manager* bm, int32_t* out, int32_t capacity, int32_t* count);
int32_t pa_bm_block_ref(const pa_block_manager* bm, int32_t block);

/*
 * Decode-step metadata for num_seqs live sequences: block_tables
 * [num_seqs, width] (entries past a table padded with -1), context_lens
 * [num_seqs] (each sequence's length, counting its newest token) and
 * slot_mapping [num_seqs] (the slot of each sequence's newest token,
 * position len - 1; -1 for an empty sequence). width must cover every table.
 */
int pa_bm_decode_metadata(const pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs, int32_t width,
                          int32_t* block_tables, int32_t* context_lens, int32_t* slot_mapping);

/*
 * Prefill metadata: sequence i computes its positions num_cached[i] .. len - 1
 * (0 <= num_cached[i] <= len). Writes block_tables [num_seqs, width] (-1
 * padded), cu_seqlens_q and cu_seqlens_k [num_seqs + 1] (query and key counts
 * len - num_cached[i] and len), and slot_mapping [total query tokens] (the
 * slot of every computed position, in sequence order); slot_capacity must be
 * at least that total.
 */
int pa_bm_prefill_metadata(const pa_block_manager* bm, const int64_t* seq_ids, const int32_t* num_cached,
                           int32_t num_seqs, int32_t width, int32_t* block_tables, int32_t* cu_seqlens_q,
                           int32_t* cu_seqlens_k, int32_t* slot_mapping, int64_t slot_capacity);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H_ */
