/*
 * pa_step.h -- decode-step executor of the paged KV cache (part of libpa.so).
 *
 * Pages cited (title, then section):
 *   [vLLM basics]   "vLLM基础：架构、推理流程与关键组件"
 *   [Reading vLLM]  "啃透vLLM源码：从PagedAttention到连续批处理，大模型推理加速24倍的秘密"
 *
 * One host call runs a whole decode step of a running batch, in the order of the
 * request life cycle of [vLLM basics] §2.2:
 *   1. the block manager (pa_blocks.h) reserves the next slot of every running
 *      sequence: a fresh block when its last block is full, a private copy of the
 *      last block when other sequences still hold it ([vLLM basics] §2.3,
 *      copy-on-write);
 *   2. block tables and context lengths (counting the new token) are built; when
 *      groups are given, a group's prefix is the run of leading whole blocks that
 *      all of its members hold;
 *   3. waiting requests are admitted in order while their blocks fit, stopping at
 *      the first that does not ([Reading vLLM] §3, the scheduler step; [vLLM basics]
 *      §2.4, continuous batching), then the sequences that finished give their blocks
 *      back: a block given back in a step goes to new requests from the next step on,
 *      so no prompt row of a step lands in a block that step's decode reads;
 *   4. every small array the device needs is written into a pinned host buffer of
 *      the executor (device-mapped, one of two used in turn);
 *   5. without copy-on-write due and without groups, the step is one launch on
 *      `stream`: the decode (8-wave workgroups, batch order) reads the arrays from
 *      the pinned buffer itself, attends each sequence's new row from new_key /
 *      new_value and stores it, and writes the admitted prompts' rows, in trailing
 *      workgroups (pa_decode_append_ex with prompt rows).  Otherwise one small kernel
 *      on `stream` copies the arrays into a device buffer (so the kernels that follow
 *      wait on no DMA engine), then: pa_block_copy when copy-on-write pairs are due,
 *      pa_cache_append of the step's new K/V rows (in the staging launch when no copy
 *      is due), and the decode: without groups pa_decode_ex with the prompts' rows in
 *      trailing workgroups, 8-wave workgroups and, unless some block of the batch is
 *      held by several sequences, the longest contexts dispatched first; with groups
 *      pa_decode_shared_prefix followed by pa_cache_append of the prompts' rows.
 *
 * Ownership.  Unlike the entry points of pa.h, an executor allocates: two pinned
 * host staging buffers, a pinned host word into which each step's first launch (the
 * one-launch decode, or the staging kernel) writes its step number as it starts (the
 * host reuses a staging buffer once the step after the one that read it has started:
 * no event is recorded per step), one device
 * staging buffer (sized at creation) and a device workspace for the decode (grown
 * when a step needs more; before freeing the old one the executor synchronizes the
 * device).  The block
 * manager, the pools and every per-step array stay the caller's; the manager and
 * the pools must outlive the executor.  pa_step_destroy synchronizes the executor's
 * device, then frees what it allocated.  An executor must not be used from two threads at once,
 * and all of its steps must run on one stream (or on streams the caller orders):
 * the staging buffers are reused from step to step.
 *
 * Errors follow pa.h (status codes, pa_last_error()).
 */
#ifndef PA_STEP_H_
#define PA_STEP_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"
#include "pa_blocks.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_step_engine pa_step_engine;

typedef struct pa_step_config {
  int32_t num_heads;           /* H of the pools, > 0 */
  int32_t head_dim;            /* D, a head_dim pa_decode supports */
  pa_dtype dtype;              /* element type of the pools and of every row array */
  int32_t max_seqs;            /* running sequences per step, > 0 */
  int32_t max_blocks_per_seq;  /* block-table width, > 0 */
  int32_t max_admit_tokens;    /* prompt tokens requested per step, >= 0 */
  int32_t max_groups;          /* shared-prefix groups per step, >= 0 (0: never); > 0
                                  only with PA_F16 pools (the shared-prefix decode),
                                  else pa_step_create fails with PA_ERR_UNSUPPORTED */
} pa_step_config;

/* New executor over the manager `bm` and the device pools key_cache / value_cache
 * ([num_blocks, num_heads, block_size, head_dim], with the manager's num_blocks and
 * block_size).  It binds to the HIP device current at the call.  Returns NULL (last
 * error set) for a configuration pa_decode does not support or a failed allocation. */
pa_step_engine* pa_step_create(pa_block_manager* bm, const pa_step_config* config,
                               void* key_cache, void* value_cache);
void pa_step_destroy(pa_step_engine* engine);

typedef struct pa_step_args {
  /* Running sequences, one new token each; batch row i is sequence seq_ids[i].
   * Host array of distinct known ids, 1 <= num_seqs <= max_seqs. */
  const int64_t* seq_ids;
  int32_t num_seqs;
  const void* query;      /* device [num_seqs, H, D] */
  const void* new_key;    /* device [num_seqs, H, D]: the new token's K and V rows */
  const void* new_value;
  void* out;              /* device [num_seqs, H, D] */
  float scale;            /* softmax scale */
  /* Shared-prefix groups (NULL and 0: the decode is pa_decode).  Host array: rows
   * group_starts[g] .. group_starts[g + 1] - 1 form group g; group_starts[0] = 0,
   * group_starts[num_groups] = num_seqs, non-decreasing; num_groups <= max_groups.
   * The executor was created with max_groups > 0, so the pools are fp16, which
   * pa_decode_shared_prefix supports at every head dim and block size. */
  const int32_t* group_starts;
  int32_t num_groups;
  /* Sequences that finish with this step (host, distinct known ids; they may be
   * running in it): their blocks are given back after the step's slots are
   * reserved. */
  const int64_t* finished_ids;
  int32_t num_finished;
  /* Waiting requests (host): ids that are distinct and not known to the manager at
   * the call, and their prompt lengths (>= 0, each < max_blocks_per_seq * block_size
   * so that the next decode token still fits the table row, sum <=
   * max_admit_tokens).  They are admitted in order while their blocks fit. */
  const int64_t* admit_ids;
  const int32_t* admit_lens;
  int32_t num_admit;
  /* device [sum of admit_lens, H, D]: the requests' prompt rows, request after
   * request; the rows of the admitted ones are written (may be NULL when the sum is
   * 0) */
  const void* prompt_key;
  const void* prompt_value;
} pa_step_args;

typedef struct pa_step_result {
  int32_t num_copies;       /* copy-on-write pairs carried out before the append */
  int32_t num_admitted;     /* leading requests admitted (the rest stay waiting) */
  int32_t admitted_tokens;  /* their prompt rows written */
  int32_t max_context_len;  /* longest context of the step, the new token counted */
  int32_t max_prefix_len;   /* groups given: longest shared prefix (tokens); else 0 */
  int32_t max_suffix_len;   /* groups given: longest context after the prefix; else 0 */
  int32_t max_group_size;   /* groups given: members of the largest group; else 0 */
} pa_step_result;

/* One decode step (steps 1-5 above); `result` (may be NULL) receives its counts.
 * PA_ERR_INVALID_ARG / PA_ERR_NULL for bad arguments and PA_ERR_OUT_OF_BLOCKS when
 * the running sequences' slots do not fit: in these cases nothing has changed and
 * nothing is enqueued.  PA_ERR_HIP when a copy or a launch fails: the manager then
 * holds the step's changes and the device side is undefined.  A context must stay
 * within max_blocks_per_seq * block_size tokens (checked). */
pa_status pa_step_run(pa_step_engine* engine, const pa_step_args* args, void* stream,
                      pa_step_result* result);

typedef struct pa_step_view {
  int32_t num_seqs;
  int32_t num_groups;
  pa_step_result result;
  const int32_t* slots;          /* host [num_seqs]: slot of each row's new token */
  const int32_t* positions;      /* host [num_seqs]: its position (context - 1) */
  const int32_t* copy_pairs;     /* host [num_copies, 2]: (source, destination) */
  const int32_t* block_tables;   /* host [num_seqs, max_blocks_per_seq], 0-padded */
  const int32_t* context_lens;   /* host [num_seqs] */
  const int32_t* group_starts;   /* host [num_groups + 1], or NULL */
  const int32_t* prefix_lens;    /* host [num_seqs] (tokens), or NULL */
  const int32_t* admit_slots;    /* host [admitted_tokens]: the prompts' slots */
  const int32_t* dev_block_tables;  /* the arrays above as the step's kernels read them:
                                       the device copy, or the pinned buffer itself */
  const int32_t* dev_context_lens;
  const int32_t* dev_group_starts;
  const int32_t* dev_prefix_lens;
  void* workspace;               /* device workspace of the step's decode */
  size_t workspace_bytes;
  pa_decode_hints hints;         /* launch hints of the step's pa_decode (seq_order is
                                    device memory of the executor); unused with groups */
} pa_step_view;

/* Host and device arrays of the last pa_step_run of this executor, valid until its
 * next pa_step_run: to check a step, or to enqueue its decode again with the same
 * arrays.  PA_ERR_INVALID_ARG before the first step. */
pa_status pa_step_last(const pa_step_engine* engine, pa_step_view* view);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* PA_STEP_H_ */
