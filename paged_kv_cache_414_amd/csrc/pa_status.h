// Internal: the thread-local last-error text behind pa_last_error() and the shape
// check of pa_decode, shared by every source file of the library.  Not part of the
// C ABI (hidden symbols).
#ifndef PA_STATUS_H_
#define PA_STATUS_H_

#include "pa.h"

struct pa_block_manager;  // include/pa_blocks.h

namespace pa {

// Record a printf-style message as this thread's last error and return `st`.
__attribute__((visibility("hidden"), format(printf, 2, 3))) pa_status set_error(pa_status st,
                                                                               const char* fmt, ...);
// Clear this thread's last error and return PA_OK.
__attribute__((visibility("hidden"))) pa_status clear_error();
// PA_OK if pa_decode is built for this element type, head_dim and block_size; else
// PA_ERR_UNSUPPORTED with the last error set.
__attribute__((visibility("hidden"))) pa_status check_dtype_shape(pa_dtype dtype, int32_t head_dim,
                                                                  int32_t block_size);

// True when some block held by one of the listed sequences has a reference count
// above 1 (held by another sequence too); unknown ids are skipped.
__attribute__((visibility("hidden"))) bool batch_shares_blocks(const ::pa_block_manager* bm,
                                                               const int64_t* seq_ids, int32_t n);

// pa_decode_ex whose launch also appends `extra_tokens` rows (extra_key / extra_value
// [extra_tokens, H, D], device) at extra_slots (int32, device-visible, negative:
// skipped) in trailing workgroups, K and V, bits unchanged.  The caller guarantees
// that no such slot lies in a block the decode reads (the executor's admitted
// prompts: their blocks were free before the step).  With new_key / new_value the
// launch is pa_decode_append_ex's as well (each sequence's newest row attended from
// them and stored at position context_lens[s] - 1; no other sequence may read that
// slot).  With started_flag, thread 0 of the launch's first workgroup writes `step`
// into it as the launch starts.  The pools are written through key_cache /
// value_cache; block_tables, context_lens and the hints' seq_order may be
// device-visible pinned host memory.
__attribute__((visibility("hidden"))) pa_status decode_with_rows(
    void* out, const void* query, void* key_cache, void* value_cache, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
    void* workspace, size_t workspace_bytes, const pa_decode_hints* hints, const void* extra_key,
    const void* extra_value, const int32_t* extra_slots, int32_t extra_tokens, const void* new_key,
    const void* new_value, int32_t* started_flag, int32_t step, void* stream);

}  // namespace pa

#endif  // PA_STATUS_H_
