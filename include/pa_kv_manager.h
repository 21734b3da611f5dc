/*
 * pa_kv_manager.h -- host-side manager of the KV block pool (part of libpa.so).
 *
 * It decides which physical block of the pool each token of each request
 * lives in, and builds the per-step inputs of pa_step (query_start_loc,
 * seq_lens, context_lens, block_tables, slot_mapping) from those decisions.
 * It touches no device memory: the pool tensor itself belongs to the caller
 * (pa.h), and this manager only hands out block ids.
 *
 * What it follows:
 *  - Free block queue: all blocks start free, in id order. Allocation takes
 *    blocks from the front of the queue; a block whose last reference goes
 *    away is appended at the back ("Inside vLLM: Anatomy of a High-Throughput
 *    LLM Inference System", section "Scheduler", allocate_slots: a doubly
 *    linked free_block_queue, the first n blocks are taken; section "Engine
 *    loop": a finished request returns its blocks to the queue).
 *  - allocate_slots: a request that is to compute n more tokens needs
 *    ceil((computed + n) / block_size) blocks in all (17 new tokens from
 *    nothing need ceil(17/16) = 2); if the queue holds fewer than the missing
 *    ones, the call exits early and changes nothing (same section).
 *  - Prefix caching ("Inside vLLM", section "Prefix caching"; "Serving
 *    models at scale with vLLM", section "Prefix caching"): every full block
 *    of a request gets a hash of the previous block's hash and its own
 *    tokens (an optional cache salt enters the first block's hash), so a
 *    block's hash depends on every token before it. A new request looks its
 *    prompt's full blocks up in order and reuses the longest run of hits:
 *    their reference counts go up (to 2 if the first owner is still alive),
 *    and a hit on a freed block takes it back out of the free queue. Freed
 *    blocks keep their contents and hashes until allocation recycles them,
 *    least recently freed first; recycling drops the block's hash.
 *  - Shared blocks ("LLM Serving Frameworks #1: Deep Dive into vLLM",
 *    section "KVCacheManager": two requests' first logical blocks map to the
 *    same physical block #42).
 *
 * Readings where the pages are silent:
 *  - A prompt's hits stop one block short of covering the whole prompt: at
 *    most floor((n_prompt - 1) / block_size) blocks, so that the prompt's
 *    last token is always computed (a prefill ends by sampling from the last
 *    position's output).
 *  - A request's blocks are freed last block first, so that of one request
 *    the blocks deepest into its prefix chain are recycled first and the
 *    more shareable leading blocks stay cached longest.
 *  - Hash collisions never produce a false hit: a lookup also compares the
 *    stored parent hash and tokens of the block it finds.
 *  - Hits are taken (and pinned) when the request is added.
 *
 * Conventions: a manager is not thread-safe (one caller thread at a time).
 * All arrays are host memory owned by the caller; the manager copies what it
 * keeps. Errors return a pa_status with the text in pa_last_error(); a call
 * that fails changes nothing.
 */
#ifndef PA_KV_MANAGER_H_
#define PA_KV_MANAGER_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_kv_manager pa_kv_manager;

/* A pool of num_blocks blocks of block_size token slots (pa_step needs 16;
 * other sizes serve the bookkeeping alone). enable_prefix_caching != 0 turns
 * on hashing and reuse. *out receives the manager (free with
 * pa_kv_manager_destroy). PA_ERR_NULL if out is NULL; PA_ERR_SHAPE if
 * num_blocks < 1 or block_size < 1. */
pa_status pa_kv_manager_create(int32_t num_blocks, int32_t block_size, int32_t enable_prefix_caching,
                               pa_kv_manager** out);
void pa_kv_manager_destroy(pa_kv_manager* m);

/* Blocks in the free queue (including freed blocks that still hold a cached
 * prefix); -1 if m is NULL. */
int32_t pa_kv_manager_num_free_blocks(const pa_kv_manager* m);

/* Admit request req_id with its n_prompt >= 1 prompt token ids (copied) and
 * cache salt (0 = none). With prefix caching, reuses the longest run of
 * cached leading blocks (see the readings above) and writes the number of
 * prompt tokens whose K/V they already hold to *num_cached_tokens (a multiple
 * of block_size, 0 without caching). PA_ERR_REQUEST if req_id is in use. */
pa_status pa_kv_manager_add_request(pa_kv_manager* m, int64_t req_id, const int32_t* prompt, int64_t n_prompt,
                                    uint64_t salt, int64_t* num_cached_tokens);

/* Append n >= 0 token ids (e.g. sampled tokens) to the request's tokens. */
pa_status pa_kv_manager_append_tokens(pa_kv_manager* m, int64_t req_id, const int32_t* tokens, int64_t n);

/* allocate_slots: make the request's next num_new_tokens positions (after
 * the ones already computed) have slots, taking ceil((computed + n) /
 * block_size) - held blocks from the front of the free queue.
 * PA_ERR_REQUEST if the request does not hold that many tokens not yet
 * computed; PA_ERR_NO_BLOCKS if the free queue is too short. */
pa_status pa_kv_manager_allocate_slots(pa_kv_manager* m, int64_t req_id, int64_t num_new_tokens);

/* After the forward pass: the request's next num_new_tokens positions are
 * computed (their K/V are in the pool). With prefix caching, each block that
 * is now full gets its chained hash and enters the cache (unless a block with
 * the same contents is cached already). PA_ERR_REQUEST if those positions
 * have no slots or no tokens. */
pa_status pa_kv_manager_commit(pa_kv_manager* m, int64_t req_id, int64_t num_new_tokens);

/* Drop the request: its blocks lose one reference each, last block first;
 * blocks left with none go to the back of the free queue. */
pa_status pa_kv_manager_free(pa_kv_manager* m, int64_t req_id);

/* Inputs of one pa_step over num_reqs requests in the given order, request i
 * computing its next num_new[i] >= 1 tokens (their slots allocated). Host
 * arrays, written in full: query_start_loc[num_reqs + 1], seq_lens[num_reqs],
 * context_lens[num_reqs] (int32), block_tables[num_reqs][max_blocks] (int32,
 * row i holds the request's blocks in order, then 0), slot_mapping[T]
 * (int64, T = sum of num_new; token position p of a request goes to slot
 * block_tables[i][p / block_size] * block_size + p % block_size).
 * PA_ERR_REQUEST for an unknown or repeated request or missing slots;
 * PA_ERR_SHAPE if a request holds more than max_blocks blocks. */
pa_status pa_kv_manager_build_step(const pa_kv_manager* m, int64_t num_reqs, const int64_t* req_ids,
                                   const int64_t* num_new, int64_t max_blocks, int32_t* query_start_loc,
                                   int32_t* seq_lens, int32_t* context_lens, int32_t* block_tables,
                                   int64_t* slot_mapping);

/* The request's block ids in order (up to cap written to out) and their
 * count in *n_blocks; its computed token count in *num_computed (either
 * output may be NULL). */
pa_status pa_kv_manager_request_blocks(const pa_kv_manager* m, int64_t req_id, int32_t* out, int64_t cap,
                                       int64_t* n_blocks, int64_t* num_computed);

/* References held on a block (0 if free); -1 for an id outside the pool. */
int32_t pa_kv_manager_ref_count(const pa_kv_manager* m, int32_t block);

/* Whether the block currently holds a cached prefix (has a hash): 1 or 0;
 * -1 for an id outside the pool. */
int32_t pa_kv_manager_is_cached(const pa_kv_manager* m, int32_t block);

#ifdef __cplusplus
}
#endif

#endif /* PA_KV_MANAGER_H_ */
