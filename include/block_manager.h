/*
 * block_manager.h -- host-side block manager of the paged KV cache, part of
 * libpagedattn.so. It produces the metadata the attention calls of
 * paged_attn.h consume: block_tables, slot_mapping, context_lens, cu_seqlens
 * and positions.
 *
 * Defined by "Nano-vLLM System Architecture Analysis":
 *   - section 2, "Paged KV Cache": the cache is cut into fixed-size blocks;
 *     the manager keeps a free list of blocks, a table from content hash to
 *     block id for prefix caching, and reference counts for blocks shared
 *     between sequences;
 *   - section 2, "Scheduler": when the cache runs out, sequences are
 *     preempted (their blocks are released and they wait to be scheduled
 *     again); long prompts are prefilled in chunks over several steps;
 *   - section 3, "Lifecycle of a Request": prepare_inputs builds the
 *     positions, block tables and slot mappings of each step;
 *   - "Differences from Normal nanoGPT Inference", item 2: blocks are
 *     allocated on demand, and identical prompt prefixes share blocks,
 *     detected with xxhash.
 *
 * Rules of this implementation (the pages describe the parts, not the rules):
 *   - Free list: first in, first out. Blocks are taken from the head and
 *     released to the tail, so a released block keeps its cached content as
 *     long as possible. It starts as 0, 1, ..., num_blocks - 1.
 *   - Content hash of full block b of a sequence: XXH64 of the block's
 *     block_size token ids as little-endian int32, seeded with the hash of
 *     block b - 1 (0 for block 0), so equal hashes mean equal prefixes.
 *     Partial blocks are never hashed or shared.
 *   - A full block's hash enters the table in the prepare call that emits the
 *     slot of its last row (its K/V are complete once that step's store has
 *     run); the first block registered under a hash keeps the entry. A block
 *     taken from the free list for new content loses its entry.
 *   - Prefix hits at allocation: full blocks are looked up in order until the
 *     first miss; a hit needs the same hash and the same token ids (a hash
 *     collision is a miss). A hit on a block in use raises its reference
 *     count; a hit on a released block takes it back from the free list. If
 *     every token of the prompt would hit, the last block is not reused, so
 *     each prompt leaves at least one token to compute.
 *   - Shared blocks are full and never written again, so copy-on-write never
 *     has to copy: a sequence writes only into its last, private block.
 *   - Release (finish or preemption) drops the sequence's blocks last block
 *     first; a block whose count reaches 0 goes to the tail of the free list.
 *
 * Conventions: all pointers are host pointers; sequence ids are caller-chosen
 * int64 values; every call validates its arguments and either succeeds in full
 * or changes nothing. Returns PA_ERR_INVALID_ARG for bad arguments or state
 * (unknown or duplicate sequence id, a table too narrow), PA_ERR_NO_BLOCKS
 * when the free list cannot supply the blocks (the caller preempts a
 * sequence and retries). A manager is not thread-safe: one thread at a time.
 */
#ifndef PA_BLOCK_MANAGER_H_
#define PA_BLOCK_MANAGER_H_

#include <stddef.h>
#include <stdint.h>

#include "paged_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* XXH64 of `len` bytes with `seed` (the published xxHash 64-bit algorithm).
 * data may be NULL when len == 0. */
uint64_t pa_xxh64(const void* data, size_t len, uint64_t seed);

/* Creates a manager of num_blocks blocks of block_size tokens (both > 0,
 * num_blocks * block_size < 2^31). *out receives the handle. */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** out);

/* Releases the manager and everything it holds. NULL is a no-op. */
void pa_bm_destroy(pa_block_manager* bm);

/* Number of blocks on the free list; -1 for a NULL manager. */
int32_t pa_bm_num_free_blocks(const pa_block_manager* bm);

/* Reference count of a block (0 = free); -1 for a bad manager or block id. */
int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block_id);

/* Admits a sequence with its prompt (num_tokens >= 1 token ids): finds the
 * prefix hits and takes blocks for the rest of the prompt. On success
 * *num_cached_tokens (may be NULL) receives the number of leading tokens
 * whose K/V are already in the pool (a multiple of block_size). */
pa_status pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, const int32_t* token_ids, int32_t num_tokens,
                         int32_t* num_cached_tokens);

/* Would pa_bm_allocate of this prompt succeed now? *ok = 1 or 0. */
pa_status pa_bm_can_allocate(const pa_block_manager* bm, const int32_t* token_ids, int32_t num_tokens,
                             int32_t* ok);

/* Appends one (sampled) token to a sequence whose every token has been
 * emitted by a prepare call. Takes a new block when the token starts one. */
pa_status pa_bm_append_token(pa_block_manager* bm, int64_t seq_id, int32_t token_id);

/* pa_bm_append_token for num_seqs distinct sequences at once (one token
 * each, as after a decode step), all or nothing: PA_ERR_NO_BLOCKS when the
 * tokens that open a block outnumber the free blocks, and then no sequence
 * changes (the caller preempts and retries). */
pa_status pa_bm_append_tokens(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* token_ids,
                              int32_t num_seqs);

/* Releases a sequence (finished or preempted) and forgets it. */
pa_status pa_bm_free(pa_block_manager* bm, int64_t seq_id);

/* Sequence state: tokens held, tokens emitted by prepare calls so far, and
 * blocks held. Any output pointer may be NULL. */
pa_status pa_bm_seq_info(const pa_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                         int32_t* num_computed, int32_t* num_blocks);

/* Copies a sequence's block ids (in order) to out[0 .. num_blocks-1];
 * capacity must be at least its block count. */
pa_status pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out, int32_t capacity);

/*
 * Metadata of a prefill (or chunked-prefill, or verify) step over num_seqs
 * sequences. Sequence i contributes n_i = its tokens not yet emitted, capped
 * at max_new_tokens[i] when max_new_tokens is not NULL (each n_i must be
 * >= 1). Outputs, in the layout pa_paged_attn_prefill and pa_kv_store read:
 *   positions, slot_mapping : [total_q] (total_q = sum n_i <= max_total_q)
 *   block_tables : [num_seqs, max_blocks_per_seq], -1 past each table
 *   context_lens : [num_seqs], tokens emitted so far + n_i
 *   cu_seqlens   : [num_seqs + 1]
 *   *total_q     : sum n_i
 * The n_i tokens count as emitted afterwards, and full blocks whose last row
 * was emitted enter the hash table.
 */
pa_status pa_bm_prepare_prefill(pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                                const int32_t* max_new_tokens, int32_t max_blocks_per_seq, int32_t max_total_q,
                                int32_t* positions, int32_t* slot_mapping, int32_t* block_tables,
                                int32_t* context_lens, int32_t* cu_seqlens, int32_t* total_q);

/*
 * Metadata of a decode step: each sequence must have exactly one token not
 * yet emitted (the one appended after the previous step). Outputs:
 *   positions, slot_mapping, context_lens : [num_seqs]
 *   block_tables : [num_seqs, max_blocks_per_seq], -1 past each table
 * in the layout pa_kv_store and pa_paged_attn_decode read.
 */
pa_status pa_bm_prepare_decode(pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t* positions, int32_t* slot_mapping,
                               int32_t* block_tables, int32_t* context_lens);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H_ */
