/*
 * pa_block_manager.h -- C ABI of the host-side block manager of the paged KV
 * cache: a pool of fixed-size blocks, per-request block tables, reference
 * counts with copy-on-write, and prefix caching by chained block keys with a
 * least-recently-used free queue.  It produces the arrays the device entry
 * points of pa.h consume: block tables, context lengths, slot mappings and
 * copy-on-write pairs.  Host memory only; nothing here touches a GPU.
 *
 * Sources (web pages, by title and section):
 *   [AQ] "PagedAttention and Continuous Batching Explained (2026)":
 *        "PagedAttention: a block table for the KV cache" (16-token blocks,
 *        a table per request, one block taken at a time as a sequence grows,
 *        copy-on-write of shared blocks, freed blocks reusable at once) and
 *        "Prefix caching" (a full block's key hashes its parent's key, its
 *        tokens and extra keys such as a LoRA id or a cache salt; lookup by
 *        key; LRU eviction of unreferenced blocks; only full blocks cached;
 *        sha256 by default).
 *   [TT] "KV Cache in Serving Engines", section 2 "Blocks and Block Tables",
 *        "Sharing Blocks" (reference counts, copy when a holder appends) and
 *        section 4 "Prefix Caching" (finished requests' blocks keep their
 *        contents in a queue, oldest evicted first, entering it from the
 *        request's back so that its tail is evicted first).
 *
 * Behaviour (readings where the pages leave a step open):
 *  - Key of full block j = Hash(key of block j-1, its token ids, extra),
 *    block 0 chaining from 32 zero bytes; hashed bytes: parent key, then the
 *    tokens as little-endian int32, then the request's extra bytes.
 *    PA_BM_HASH_SHA256 (FIPS 180-4) or PA_BM_HASH_FNV1A64 (64-bit FNV-1a,
 *    written little-endian into the first 8 key bytes, the rest zero).
 *  - The free queue starts in pool order (or free_order).  Taking a block
 *    pops the queue's front and drops any key the block still holds.  A
 *    cache hit on a queued block takes it out of the queue.
 *  - Admitting a prompt reuses its leading full blocks while their keys hit
 *    (the first miss ends the shared part) and takes fresh blocks for the
 *    rest; fresh full blocks are registered under their keys unless the key
 *    is held already.  A block filled by appended tokens is registered too.
 *  - Appending takes a new block only when the last one is full; a shared,
 *    partly filled last block is first copied (copy-on-write).
 *  - Freeing a request visits its blocks last to first; a block whose count
 *    drops to zero goes to the back of the free queue.
 *  - An operation that runs out of blocks fails with PA_BM_ERR_NO_BLOCKS
 *    and leaves the state unchanged.
 *
 * Not thread-safe: one manager per thread, or the caller serialises calls.
 * Return codes: 0 on success or a negative code (below, or PA_ERR_INVALID_ARG
 * = -1 from pa.h for a null pointer or a bad size).
 */
#ifndef PAGED_KV_PA_BLOCK_MANAGER_H
#define PAGED_KV_PA_BLOCK_MANAGER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_BM_HASH_SHA256 = 0,
  PA_BM_HASH_FNV1A64 = 1,
};

enum {
  PA_BM_ERR_NO_BLOCKS = -5, /* the pool has too few free blocks            */
  PA_BM_ERR_REQUEST = -6,   /* unknown request id, or an id already in use  */
};

typedef struct pa_block_manager pa_block_manager;

/* A manager over num_blocks blocks of block_size token slots.  free_order
 * (num_blocks distinct ids, or NULL for 0..num_blocks-1) is the initial
 * order of the free queue.  Returns NULL on a bad argument. */
pa_block_manager* pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t hash_kind,
                               const int32_t* free_order);
void pa_bm_destroy(pa_block_manager* bm);

/* Admit request req with its prompt tokens[0..num_tokens) and extra key
 * bytes (may be NULL when extra_len is 0).  *cached_tokens receives the
 * number of prompt tokens whose K/V the cache already holds (a multiple of
 * block_size): the prefill only has to compute the rest. */
int pa_bm_add_request(pa_block_manager* bm, int64_t req, const int32_t* tokens,
                      int32_t num_tokens, const uint8_t* extra, int32_t extra_len,
                      int32_t* cached_tokens);

/* A new request sharing every block of parent (parallel sampling). */
int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* Append one token: *slot receives block * block_size + offset; when a
 * shared block had to be copied first, *cow_src / *cow_dst receive the pair
 * (else both -1). */
int pa_bm_append_token(pa_block_manager* bm, int64_t req, int32_t token, int64_t* slot,
                       int64_t* cow_src, int64_t* cow_dst);

/* Release a request's blocks. */
int pa_bm_free_request(pa_block_manager* bm, int64_t req);

/* One decode step over num_reqs requests: append tokens[i] to reqs[i] (in
 * order), then write, for the kernels of pa.h:
 *   block_tables   int32 [num_reqs][max_blocks_per_seq], -1 past each table
 *   context_lens   int32 [num_reqs] (including the appended token)
 *   slot_mapping   int64 [num_reqs]
 *   block_mapping  int64 [num_reqs][2] (copy-on-write pairs), *num_pairs of them
 * The blocks the step needs (new blocks and copies, counted exactly by a dry
 * run) are checked first: too few free blocks fail with PA_BM_ERR_NO_BLOCKS,
 * a table growing past max_blocks_per_seq or an unknown request with
 * PA_ERR_INVALID_ARG / PA_BM_ERR_REQUEST, each before anything changes.  A
 * request may appear more than once (its tokens are appended in order). */
int pa_bm_decode_step(pa_block_manager* bm, const int64_t* reqs, const int32_t* tokens,
                      int32_t num_reqs, int32_t max_blocks_per_seq, int32_t* block_tables,
                      int32_t* context_lens, int64_t* slot_mapping, int64_t* block_mapping,
                      int32_t* num_pairs);

/* Queries.  pa_bm_block_table writes up to capacity entries and returns the
 * table's length (or a negative code). */
int32_t pa_bm_block_table(const pa_block_manager* bm, int64_t req, int32_t* out,
                          int32_t capacity);
int32_t pa_bm_num_tokens(const pa_block_manager* bm, int64_t req);
int64_t pa_bm_num_free_blocks(const pa_block_manager* bm);
int64_t pa_bm_num_cached_blocks(const pa_block_manager* bm);
int32_t pa_bm_refcount(const pa_block_manager* bm, int64_t block);
/* The free queue front to back (up to capacity ids); returns its length. */
int64_t pa_bm_free_queue(const pa_block_manager* bm, int32_t* out, int64_t capacity);
/* Block holding a 32-byte key, or -1. */
int64_t pa_bm_lookup(const pa_block_manager* bm, const uint8_t* key);

/* The block key of the pages' rule, and SHA-256 itself (FIPS 180-4). */
int pa_bm_block_key(const uint8_t* parent, const int32_t* tokens, int32_t num_tokens,
                    const uint8_t* extra, int32_t extra_len, int32_t hash_kind, uint8_t* key);
int pa_bm_sha256(const uint8_t* data, size_t len, uint8_t* digest);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_PA_BLOCK_MANAGER_H */
