/*
 * pa_blocks.h -- host-side block manager of the paged KV cache (part of libpa.so).
 *
 * Pages cited (title, then section):
 *   [Reading vLLM]  "啃透vLLM源码：从PagedAttention到连续批处理，大模型推理加速24倍的秘密"
 *   [vLLM basics]   "vLLM基础：架构、推理流程与关键组件"
 *
 * What it keeps, as the pages describe it:
 *  * The pool is cut into num_blocks fixed-size blocks of block_size token slots; a
 *    sequence holds only the blocks its tokens need, anywhere in the pool, and its
 *    block table maps logical block i to a physical block ([Reading vLLM] §2.2,
 *    PhysicalTokenBlock / LogicalTokenBlock; [vLLM basics] §2.3, block table).
 *  * New blocks come from a free list; a finished sequence returns every block it
 *    holds ([vLLM basics] §2.2 steps 4 and 7, §2.3).
 *  * Physical blocks carry a reference count, so several sequences can hold the same
 *    block (e.g. a common prompt); a holder that must write into a block others
 *    still hold gets its own copy first ([Reading vLLM] §2.2 ref_count; [vLLM basics]
 *    §2.3 copy-on-write).  Here the first ref_count - 1 writers copy and the last
 *    remaining holder writes in place.
 *  * Slot of logical token p of a sequence: table[p / block_size] * block_size +
 *    p % block_size -- the slot_mapping that pa_cache_append takes (pa.h).
 *
 * Pure host code: no call here touches a GPU.  A handle must not be used from two
 * threads at once.  Functions returning pa_status report failures through
 * pa_last_error() (pa.h) and leave the manager unchanged when they fail.  Sequence
 * ids are caller-chosen 64-bit integers.
 */
#ifndef PA_BLOCKS_H_
#define PA_BLOCKS_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* New manager over blocks 0 .. num_blocks-1, all free.  seed == 0: a new block is
 * the most recently freed one (initially the lowest id); seed != 0: a new block is
 * drawn uniformly from the free list by a SplitMix64 generator seeded with `seed`.
 * Returns NULL (last error set) when num_blocks or block_size is not positive or
 * num_blocks * block_size exceeds the int32 slot range.  The caller owns the handle
 * and releases it with pa_bm_destroy. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, uint64_t seed);
void pa_bm_destroy(pa_block_manager* bm);

/* The pool the manager was created over: its blocks, and token slots per block
 * (-1 for a NULL manager). */
int32_t pa_bm_num_blocks(const pa_block_manager* bm);
int32_t pa_bm_block_size(const pa_block_manager* bm);

/* Free blocks; 1 if ceil(num_tokens / block_size) blocks are free, else 0. */
int32_t pa_bm_num_free(const pa_block_manager* bm);
int32_t pa_bm_can_allocate(const pa_block_manager* bm, int32_t num_tokens);

/* Reference counts of all blocks into ref_counts[num_blocks]. */
pa_status pa_bm_ref_counts(const pa_block_manager* bm, int32_t* ref_counts);

/* Admit sequence seq_id holding num_tokens (>= 0) prompt tokens: allocate
 * ceil(num_tokens / block_size) blocks.  slots (may be NULL) receives the slot of each
 * prompt token, [num_tokens].  PA_ERR_OUT_OF_BLOCKS if they do not fit,
 * PA_ERR_INVALID_ARG if seq_id exists. */
pa_status pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, int32_t num_tokens,
                             int32_t* slots);

/* Admit n sequences at once (seq_ids[n], num_tokens[n]), in order; slots (may be
 * NULL) receives every prompt token's slot, the sequences' runs concatenated in
 * order.  All or nothing: PA_ERR_OUT_OF_BLOCKS (nothing changed) if the blocks of
 * all of them do not fit; PA_ERR_INVALID_ARG for an existing or repeated id. */
pa_status pa_bm_add_sequences(pa_block_manager* bm, const int64_t* seq_ids,
                              const int32_t* num_tokens, int32_t n, int32_t* slots);

/* child_id holds every block of parent_id (reference counts + 1) and its length. */
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id);

/* The sequence finished: each of its blocks loses one reference; a block no one
 * holds returns to the free list. */
pa_status pa_bm_free(pa_block_manager* bm, int64_t seq_id);

/* Reserve the slot of the next token of each listed sequence, in list order (a
 * sequence listed twice gets two consecutive tokens).  When the token starts a new
 * logical block, a new physical block is allocated; when it lands in a block that
 * others still hold, a private copy is allocated first and (source, destination) is
 * appended to copy_pairs, which the caller must carry out (pa_block_copy) before
 * writing the token.  Outputs: slots[n]; positions[n] (may be NULL): the token's
 * position, i.e. the sequence's length before it; copy_pairs[n][2]; *num_copies.
 * All or nothing: PA_ERR_OUT_OF_BLOCKS (nothing changed) if the blocks needed by the
 * whole list are not free. */
pa_status pa_bm_append_slots(pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                             int32_t* slots, int32_t* positions, int32_t* copy_pairs,
                             int32_t* num_copies);

/* Block tables [n, max_blocks] of the listed sequences, entries past each sequence's
 * blocks set to `pad`; PA_ERR_INVALID_ARG if one holds more than max_blocks. */
pa_status pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                             int32_t max_blocks, int32_t pad, int32_t* tables);

/* Context lengths (tokens) of the listed sequences, [n]. */
pa_status pa_bm_context_lens(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                             int32_t* context_lens);

/* Number of leading whole blocks (logical index < min length / block_size) that all
 * listed sequences hold as the same physical blocks -- the shared prefix that
 * pa_decode_shared_prefix can read once for all of them (prefix_lens = this *
 * block_size).  -1 (last error set) for an unknown id or n < 1. */
int32_t pa_bm_shared_prefix_blocks(const pa_block_manager* bm, const int64_t* seq_ids,
                                   int32_t n);

/* Blocks held by seq_id (-1 if unknown), and their physical ids into blocks[cap]
 * (the first min(cap, count) of them). */
int32_t pa_bm_num_seq_blocks(const pa_block_manager* bm, int64_t seq_id);
pa_status pa_bm_seq_blocks(const pa_block_manager* bm, int64_t seq_id, int32_t* blocks,
                           int32_t cap);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* PA_BLOCKS_H_ */
