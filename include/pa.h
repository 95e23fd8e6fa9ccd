/*
 * pa.h -- C ABI of the paged KV-cache decode path for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title, then section):
 *   [Reading vLLM]  "啃透vLLM源码：从PagedAttention到连续批处理，大模型推理加速24倍的秘密"
 *                   (Reading the vLLM source: from PagedAttention to continuous batching)
 *   [vLLM basics]   "vLLM基础：架构、推理流程与关键组件"
 *                   (vLLM basics: architecture, inference flow and key components)
 *   [vLLM analysis] "VLLM源码解析：高效大规模语言模型推理的技术实现"
 *                   (vLLM source analysis: technical implementation of efficient inference)
 *
 * The method: each sequence's KV cache is cut into fixed-size blocks (16 tokens by
 * default) that may sit anywhere in a physical pool; a per-sequence block table maps
 * logical block i to its physical block ([Reading vLLM] §2.2; [vLLM basics] §2.3).
 * Attention for the newest token reads the query, the key and value caches and the
 * physical block indices ([vLLM analysis], design principles).  Blocks are shared
 * by reference count and copied before a sharer writes ([Reading vLLM] §2.2;
 * [vLLM basics] §2.3, copy-on-write).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  * Every array pointer is a DEVICE pointer owned by the caller.  The library keeps
 *    no pointer after a call returns and allocates no device memory.
 *  * All arrays are dense, row-major (C order) and 16-byte aligned.
 *  * `stream` is a hipStream_t (NULL = the legacy default stream).  Each call only
 *    enqueues work on it and returns without waiting; ordering between calls comes
 *    from stream order.
 *  * Element type: PA_F32 (float) or PA_F16 (IEEE binary16).  The query, both pools,
 *    the appended key/value rows and the output share one element type.
 *  * Layouts:
 *      query, out            [num_seqs, num_heads, head_dim]
 *      key, value (append)   [num_tokens, num_heads, head_dim]
 *      key_cache, value_cache[num_blocks, num_heads, block_size, head_dim]
 *      block_tables          int32 [num_seqs, max_blocks_per_seq]; row s entry i is
 *                            the physical block of logical block i of sequence s.
 *                            Entries at i >= ceil(context_lens[s] / block_size) are
 *                            never read for addressing and may hold any value.
 *      context_lens          int32 [num_seqs], tokens of each sequence, >= 0.
 *      slot_mapping          int32 [num_tokens]; slot = block * block_size + offset.
 *                            A negative slot means "skip this row".
 *      block_pairs           int32 [num_pairs, 2] = (source block, destination block).
 *  * Supported shapes: head_dim in {64, 80, 96, 128, 256}; block_size in {8, 16,
 *    32, 64, 128, 256} (pa_decode_shared_prefix: fp16, every head_dim above,
 *    block_size 8 to 256); other values return PA_ERR_UNSUPPORTED.  K/V heads
 *    equal query heads.
 *  * Errors: argument checks run on the host before anything is enqueued and return
 *    a status; nothing aborts and no C++ exception crosses the ABI.  A failed launch
 *    returns PA_ERR_HIP.  The text of the last error of the calling thread is
 *    available from pa_last_error().
 *  * Device-side contents are caller preconditions and are not checked: block ids in
 *    [0, num_blocks) for every live logical block, context_lens[s] <=
 *    min(max_context_len, max_blocks_per_seq * block_size), distinct non-negative
 *    slots below num_blocks * block_size, and copy pairs whose destinations are
 *    distinct and never a source.  Violations are undefined behaviour.
 *  * Debug build (libpa_debug.so, compiled with PA_DEBUG_CHECKS=1; pa_debug_checks()
 *    returns 1): every entry point first waits for the work already on its stream,
 *    copies the device arrays it is about to hand to a kernel (tables, context
 *    lengths, slots, copy pairs, dispatch order, groups) to the host and checks every
 *    precondition stated for them in this header.  A violation returns
 *    PA_ERR_INVALID_ARG, naming the offending entry in pa_last_error(), before the
 *    call has enqueued anything.
 *    The debug build synchronises inside every call, so it cannot be captured into a
 *    graph and runs slower; results are bit for bit those of the default build.
 *  * Concurrent calls from several host threads are safe; calls that write the same
 *    memory must be ordered by the caller (same stream or events).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 2

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,          /* a required pointer is NULL */
  PA_ERR_INVALID_ARG = 2,   /* a size or value is out of range or inconsistent */
  PA_ERR_UNSUPPORTED = 3,   /* dtype, head_dim or block_size not built */
  PA_ERR_WORKSPACE = 4,     /* workspace missing or smaller than required */
  PA_ERR_HIP = 5,           /* the HIP runtime reported an error */
  PA_ERR_OUT_OF_BLOCKS = 6  /* the block manager has too few free blocks (pa_blocks.h) */
} pa_status;

/* Version of this ABI (PA_ABI_VERSION of the library that was built). */
int32_t pa_abi_version(void);

/* 1 in the debug build (device data checked on the host before every launch, as
 * described above), 0 in the default build. */
int32_t pa_debug_checks(void);

/* Human-readable name of a status code (static storage, never NULL). */
const char* pa_status_string(pa_status status);

/* Message describing the last failing call made by this host thread, or "" if none
 * failed.  Static thread-local storage: valid until the thread's next call. */
const char* pa_last_error(void);

/*
 * Split-context planning.
 *
 * Decode attention of a sequence is computed over partitions of `partition_size`
 * consecutive tokens; each partition yields a partial softmax state that a second
 * pass merges by the log-sum-exp rule (Milakov & Gimelshein 2018, "Online
 * normalizer calculation for softmax").  This splitting is this library's own way
 * of spreading long contexts over the GPU; the pages state only the result, which
 * equals attention over the whole sequence.
 *
 * pa_decode_partition_size returns the partition length (tokens) that pa_decode
 * uses for these arguments: `partition_size` itself when it is > 0 (it must then be
 * a positive multiple of block_size), otherwise the library's choice.  The value
 * is always a multiple of block_size.  Returns -1 for invalid arguments.
 */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads,
                                 int32_t block_size, int32_t max_context_len,
                                 int32_t partition_size);

/* Number of partitions per (sequence, head) reserved in the workspace:
 * ceil(max_context_len / P) with P = pa_decode_partition_size(...), at least 1.
 * Returns -1 for invalid arguments. */
int32_t pa_decode_num_partitions(int32_t num_seqs, int32_t num_heads,
                                 int32_t block_size, int32_t max_context_len,
                                 int32_t partition_size);

/* Wave64s per workgroup the partition pass of pa_decode launches for these
 * arguments: 16 when each partition holds at least 32 units (the tokens a wave
 * folds at once: a block, or 8 loads of 16 bytes per lane when the block is
 * larger) and the launch has at least 1024 (sequence, head, partition)
 * workgroups, else 8.  The result is the same either way up to floating-point
 * rounding.  Returns -1 (last error set) for invalid arguments. */
int32_t pa_decode_waves(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                        int32_t block_size, int32_t max_context_len, int32_t partition_size,
                        pa_dtype dtype);

/*
 * Bytes of workspace pa_decode needs; 0 when every sequence fits one partition
 * (the workspace pointer may then be NULL).  Layout, with NP =
 * pa_decode_num_partitions(...), all float32:
 *     m [num_seqs, num_heads, NP]   at byte 0
 *     l [num_seqs, num_heads, NP]   at byte ws_align(S*H*NP*4)
 *     o [num_seqs, num_heads, NP, head_dim]   at byte 2*ws_align(S*H*NP*4)
 * where ws_align rounds up to 256.  For partition p of (s, h) over its tokens t:
 *     m = max_t z_t,  l = sum_t 2^(z_t - m),  o = sum_t 2^(z_t - m) * v_t,
 *     z_t = scale * log2(e) * <q, k_t>
 * (base-2 logits).  Returns 0 and sets the last error for invalid arguments.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode -- single-query paged attention ([vLLM analysis], design principles:
 * attention over query, key_cache, value_cache and the physical block indices).
 *
 * For every sequence s and head h, with L = context_lens[s]:
 *     k_t = key_cache[block_tables[s][t / bs], h, t % bs, :]  (likewise v_t), t < L
 *     out[s, h, :] = sum_t softmax_t(scale * <query[s, h, :], k_t>) * v_t
 * and out[s, h, :] = 0 when L = 0.  Arithmetic is float32 (products, softmax,
 * accumulation); the result is rounded once to the element type.
 *
 * max_context_len must be >= every context_lens[s] and <= max_blocks_per_seq *
 * block_size; it sizes the grid.  partition_size: 0 = library choice, else a positive
 * multiple of block_size.  workspace: device memory of at least
 * pa_decode_workspace_bytes(...) bytes (may be NULL if that is 0); its contents on
 * entry do not matter and on return are the partition states described above.
 * Enqueues pa_decode_partitions and, when more than one partition is reserved,
 * pa_decode_reduce.
 */
pa_status pa_decode(void* out, const void* query, const void* key_cache,
                    const void* value_cache, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                    int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                    pa_dtype dtype, int32_t partition_size, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * pa_decode_append -- one decode step in one call: each sequence's newest K/V row is
 * written into its slot and attended to, as the request life cycle orders it ([vLLM
 * basics] §2.2: the new token's K/V is stored, then attention runs over the context
 * that counts it).  For every s with L = context_lens[s] >= 1, with t = L - 1,
 * b = block_tables[s][t / bs] and o = t % bs, and every head h:
 *     key_cache[b, h, o, :] = new_key[s, h, :];  value_cache[b, h, o, :] = new_value[s, h, :]
 * then out as pa_decode over the L tokens.  The pools afterwards, and out, are bit for
 * bit those of pa_cache_append (slot_mapping[s] = b * bs + o) followed by pa_decode
 * with the same arguments; sequences with L = 0 write nothing.  new_key and new_value:
 * device [num_seqs, num_heads, head_dim] of the pools' type, 16-byte aligned.  The
 * attention takes the new row from new_key / new_value; one extra workgroup per
 * sequence stores it into the pools while the attention runs, so the slot must be
 * read by no other sequence of the call (copy-on-write carried out before, as
 * pa_cache_append requires distinct slots).  The store workgroups take
 * ceil(num_seqs / (partitions x num_heads)) grid z-slices after the sequences', and
 * num_seqs plus those must not exceed 65535 (PA_ERR_INVALID_ARG otherwise).  Other
 * arguments, workspace and errors as pa_decode; the same workspace size.  Saves the
 * separate append launch, which is most of a step's time at small batch.
 */
pa_status pa_decode_append(void* out, const void* query, void* key_cache, void* value_cache,
                           const void* new_key, const void* new_value,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_context_len, float scale, pa_dtype dtype,
                           int32_t partition_size, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Launch hints for pa_decode_ex and pa_decode_append_ex: what a caller that knows its
 * batch (a scheduler holds every context length on the host) can tell the library.
 * Pools are written bit for bit as without hints, and outputs stay within the stated
 * tolerance of the exact attention.
 *   seq_order  device int32 [num_seqs], 4-byte aligned, or NULL: a permutation of
 *              0 .. num_seqs-1 (caller precondition, unchecked device data); the
 *              workgroups of sequence seq_order[i] are dispatched i-th.  Longest
 *              context first lets the short sequences fill the end of the launch.
 *              The order changes no bit of the result: every floating-point
 *              operation's order depends only on logical token positions.
 *   waves      wave64s per workgroup of the partition pass: 0 for the library's
 *              choice (pa_decode_waves), else 8 or 16 (PA_ERR_INVALID_ARG otherwise).
 *              The wave count sets how a partition's tokens are dealt to waves and
 *              merged, so it changes the rounding of the output (bit for bit that of
 *              any call launched with the same count).  8 suits batches whose
 *              sequences re-read shared blocks through pa_decode (the caches serve
 *              the re-reads better with more, smaller workgroups in flight).
 */
typedef struct pa_decode_hints {
  const int32_t* seq_order;
  int32_t waves;
} pa_decode_hints;

/* pa_decode with launch hints (NULL hints = pa_decode). */
pa_status pa_decode_ex(void* out, const void* query, const void* key_cache,
                       const void* value_cache, const int32_t* block_tables,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                       int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                       pa_dtype dtype, int32_t partition_size, void* workspace,
                       size_t workspace_bytes, const pa_decode_hints* hints, void* stream);

/* pa_decode_append with launch hints (NULL hints = pa_decode_append). */
pa_status pa_decode_append_ex(void* out, const void* query, void* key_cache, void* value_cache,
                              const void* new_key, const void* new_value,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                              pa_dtype dtype, int32_t partition_size, void* workspace,
                              size_t workspace_bytes, const pa_decode_hints* hints,
                              void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device memory: code
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, result and errors as pa_decode, without the workspace: when some
 * sequence spans more than one partition, the partition states go to a scratch array
 * that the library holds in device memory (a file-scope device variable of
 * PA_NOALLOC_SCRATCH_BYTES bytes on every GPU the library runs on, kept until the
 * process ends; the call allocates nothing).  Arguments whose
 * pa_decode_workspace_bytes(...) exceeds that size return PA_ERR_WORKSPACE before
 * anything is enqueued.  The first call that needs the array on a device looks up its
 * address there (make it before capturing a graph).  Every call on one GPU shares that
 * GPU's array, which keeps the last call's partition states: calls that overlap on one
 * GPU (different streams, or host threads not ordered by the caller) race and give
 * undefined results; calls in one stream are ordered.  Nothing in the array needs to
 * start at zero.
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)

pa_status pa_decode_noalloc(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                            pa_dtype dtype, int32_t partition_size, void* stream);

/*
 * pa_decode_partitions -- first pass of pa_decode alone (same arguments).
 * Sequences with L <= P get their final output written to `out`; for the others,
 * every partition p < ceil(L / P) writes its (m, l, o) state to the workspace and
 * `out` is left for pa_decode_reduce.  Exposed so the two passes can be timed and
 * checked separately.
 */
pa_status pa_decode_partitions(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_context_len, float scale, pa_dtype dtype,
                               int32_t partition_size, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * pa_decode_reduce -- second pass: for every (s, h) with ceil(L / P) > 1, merge the
 * partition states in the workspace:
 *     M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p
 * rounded once to the element type.  Other sequences' outputs are not touched.
 * block_size, max_context_len and partition_size must be those given to
 * pa_decode_partitions.
 */
pa_status pa_decode_reduce(void* out, const void* workspace, size_t workspace_bytes,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_context_len, pa_dtype dtype,
                           int32_t partition_size, void* stream);

/*
 * pa_cache_append -- write each step's new K/V rows into the slots their positions
 * map to (blocks fill slot by slot: [Reading vLLM] §2.2, LogicalTokenBlock).
 * For i < num_tokens with slot = slot_mapping[i] >= 0, b = slot / block_size,
 * o = slot % block_size, and every head h:
 *     key_cache[b, h, o, :] = key[i, h, :];  value_cache[b, h, o, :] = value[i, h, :]
 * Bits are copied unchanged.  Rows with a negative slot are skipped.  Slots must be
 * distinct (caller precondition).
 */
pa_status pa_cache_append(void* key_cache, void* value_cache, const void* key,
                          const void* value, const int32_t* slot_mapping,
                          int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                          void* stream);

/*
 * pa_block_copy -- the copy-on-write duplication: when sequences that share a block
 * diverge, the writer first gets its own copy ([vLLM basics] §2.3, copy-on-write;
 * [Reading vLLM] §2.2, ref_count).  For each pair (src, dst):
 *     key_cache[dst] = key_cache[src];  value_cache[dst] = value_cache[src]
 * (all heads, all slots, bits unchanged).  Destinations must be distinct and never
 * a source (caller precondition), so the pairs may run in any order.
 */
pa_status pa_block_copy(void* key_cache, void* value_cache, const int32_t* block_pairs,
                        int32_t num_pairs, int32_t num_heads, int32_t head_dim,
                        int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                        void* stream);

/*
 * pa_swap_blocks -- move whole blocks between two pools that may live in different
 * memories: under memory pressure a scheduler moves the blocks of preempted
 * sequences out of the GPU pool into host memory and brings them back when the
 * sequences resume ([Reading vLLM] §3, blocks_to_swap_out / blocks_to_swap_in).
 * For each pair (src, dst) of block_pairs:
 *     dst_key[dst] = src_key[src];  dst_value[dst] = src_value[src]
 * (all heads and slots, bits unchanged).  Both pools have the layout
 * [num_blocks, num_heads, block_size, head_dim] (src_num_blocks and dst_num_blocks
 * blocks).  Each pool pointer, and block_pairs (int32 [num_pairs, 2]), must be
 * device memory or pinned host memory (hipHostMalloc; torch pin_memory=True): the
 * library asks the runtime for every pointer and refuses anything else (pageable
 * memory) with PA_ERR_INVALID_ARG before enqueuing.  The copy runs on the GPU and
 * reads or writes host memory across the host link.  Destinations must be distinct
 * and, when both sides are one pool, never a source; ids must lie in their pools
 * (caller preconditions).
 */
pa_status pa_swap_blocks(void* dst_key, void* dst_value, const void* src_key,
                         const void* src_value, const int32_t* block_pairs, int32_t num_pairs,
                         int32_t num_heads, int32_t head_dim, int32_t block_size,
                         int32_t src_num_blocks, int32_t dst_num_blocks, pa_dtype dtype,
                         void* stream);

/*
 * Shared-prefix decode.
 *
 * Sequences may share their leading blocks by reference count, e.g. the prompt of
 * several samples drawn from it ([Reading vLLM] §2.2, PhysicalTokenBlock.ref_count;
 * [vLLM basics] §2.3: sharing, and copy-on-write once a sharer writes).  Sharing
 * changes where the numbers live, not the attention, so pa_decode_shared_prefix
 * computes exactly what pa_decode computes (same definition, tolerances and output
 * layout).  It differs in how it reads the cache: each shared block is read once per
 * group for all of the group's queries, as small dense products on the matrix cores
 * (fp16 operands, fp32 accumulation; the softmax weights enter as two fp16 terms so
 * that no precision is lost to their rounding), and the tokens after the prefix are
 * read per sequence as in pa_decode.  The partial softmax states are then merged.
 *
 * Groups are ranges of sequences:
 *   group_starts   int32 [num_groups + 1], device: group g is sequences
 *                  [group_starts[g], group_starts[g + 1]); non-decreasing, within
 *                  [0, num_seqs]; ranges do not overlap.
 *   prefix_lens    int32 [num_seqs], device: the number of leading tokens that
 *                  sequence s shares with the rest of its group; a multiple of
 *                  block_size, <= context_lens[s] and <= max_prefix_len; the same
 *                  for every sequence of a group; 0 for a sequence in no group.
 *                  For every sequence of group g, the first prefix_lens[s] /
 *                  block_size entries of its block table equal those of sequence
 *                  group_starts[g].
 *   max_group_size host: the number of members of the largest group, or 0 for
 *                  the library's choice (the average group size).  Any value >= 0
 *                  gives the same result; it sizes the launch: each tile of 16
 *                  members of a group gets its own workgroups, and a group larger
 *                  than max_group_size walks its further tiles in turn.
 *   max_prefix_len host: >= every prefix_lens[s], a multiple of block_size.
 *   max_suffix_len host: >= every context_lens[s] - prefix_lens[s].
 * Both are <= max_blocks_per_seq * block_size, and every context_lens[s] is too.
 * Groups of any size are accepted; a group's prefix is read once per 16 members, by
 * workgroups that run side by side.
 * Built for PA_F16, head_dim in {64, 80, 96, 128, 256} and block_size in {8, 16, 32, 64, 128,
 * 256}; other values return PA_ERR_UNSUPPORTED.  The prefix pass reads whole tiles of 16
 * tokens: with block_size 8, the prefix of a sequence whose prefix_lens[s] is an odd
 * number of blocks is read by the pass after the prefix from its last 8 tokens on (the
 * rounded length below is P0 = prefix_lens[s] rounded down to a multiple of 16; P0 =
 * prefix_lens[s] for block_size >= 16).  partition_size applies to the tokens after P0
 * (as in pa_decode, sized by max_suffix_len, plus 8 with block_size 8);
 * prefix_partition_size is the number of prefix tokens one workgroup reads (0 = library
 * choice, else a positive multiple of max(16, block_size)).  The contents above are
 * caller preconditions (unchecked device data, as for pa_decode).
 *
 * Workspace (always needed when num_seqs > 0), float32, with NPp = prefix
 * partitions, NPs = partitions after the prefix and NS = NPp + NPs:
 *     m [num_seqs, num_heads, NS]   at byte 0
 *     l [num_seqs, num_heads, NS]   at byte ws_align(S*H*NS*4)
 *     o [num_seqs, num_heads, NS, head_dim]   at byte 2*ws_align(S*H*NS*4)
 * Slot p < NPp holds the state of prefix tokens [p*Pp, min((p+1)*Pp, P0)) and slot
 * NPp + p that of tokens [P0 + p*P, P0 + (p+1)*P), with the same
 * (m, l, o) definition as pa_decode's workspace.  Slots past a sequence's tokens are
 * not written, nor are the slots after the prefix of a sequence whose remaining
 * tokens fit one partition: that partition's workgroup merges the prefix states and
 * writes the output itself (the merge pass runs only when NPs > 1).  pa_decode_shared_prefix_workspace_bytes returns the size (0 and the
 * last error set for invalid arguments).
 */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                               int32_t head_dim, int32_t block_size,
                                               int32_t num_groups, int32_t max_group_size,
                                               int32_t max_prefix_len, int32_t max_suffix_len,
                                               int32_t partition_size,
                                               int32_t prefix_partition_size);

pa_status pa_decode_shared_prefix(void* out, const void* query, const void* key_cache,
                                  const void* value_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* group_starts,
                                  const int32_t* prefix_lens, int32_t num_seqs,
                                  int32_t num_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, int32_t max_blocks_per_seq,
                                  int32_t num_groups, int32_t max_group_size,
                                  int32_t max_prefix_len, int32_t max_suffix_len, float scale,
                                  pa_dtype dtype, int32_t partition_size,
                                  int32_t prefix_partition_size, void* workspace,
                                  size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* PA_H_ */
