// Internal: checks of the device data that every entry point takes as a caller
// precondition (include/pa.h: block ids, context lengths, slots, copy pairs, groups
// of shared prefixes).  In a build with PA_DEBUG_CHECKS=1 each entry point waits for
// the work already on its stream (which may write those arrays), copies the arrays it
// is about to hand to a kernel into host memory and checks them there, before
// anything is launched: a violation returns PA_ERR_INVALID_ARG with the offending
// entry named in pa_last_error(), and no kernel ever addresses memory through it.
// Such a build synchronises inside every call and so cannot be captured into a graph.
// In the default build (PA_DEBUG_CHECKS=0) every check is an inline PA_OK.
#ifndef PA_DEBUG_H_
#define PA_DEBUG_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "pa.h"

#ifndef PA_DEBUG_CHECKS
#define PA_DEBUG_CHECKS 0
#endif

namespace pa {
namespace debug {

// Context lengths and block tables of a decode launch, as copied to the host.
struct DecodeView {
  std::vector<int32_t> ctx;  // [S]
  std::vector<int32_t> bt;   // [S, MB]
  int32_t S = 0, MB = 0, BS = 0;
};

#if PA_DEBUG_CHECKS

#define PA_DEBUG_HIDDEN __attribute__((visibility("hidden")))

// context_lens[s] in [0, max_context_len] and, for every live logical block
// (i < ceil(context_lens[s] / block_size)), block_tables[s][i] in [0, num_blocks).
PA_DEBUG_HIDDEN pa_status decode_data(DecodeView* v, const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_blocks, int32_t max_blocks_per_seq,
                                      int32_t block_size, int32_t max_context_len, hipStream_t stream);
// context_lens[s] in [0, max_context_len] (the merge pass reads nothing else).
PA_DEBUG_HIDDEN pa_status lengths(const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                                  hipStream_t stream);
// seq_order (or NULL) is a permutation of 0 .. num_seqs - 1.
PA_DEBUG_HIDDEN pa_status seq_order(const int32_t* order, int32_t num_seqs, hipStream_t stream);
// pa_decode_append: the slots of the new rows (position context_lens[s] - 1) are
// distinct and read by no other sequence of the call.
PA_DEBUG_HIDDEN pa_status new_rows(const DecodeView& v);
// Rows appended by the decode launch's trailing workgroups: slots below
// num_blocks * block_size, the non-negative ones distinct, none in a block the
// decode reads.
PA_DEBUG_HIDDEN pa_status extra_rows(const DecodeView& v, const int32_t* slots, int32_t n, int32_t num_blocks,
                                     hipStream_t stream);
// Slot mapping of an append (device or host memory): every slot below
// num_blocks * block_size, the non-negative ones distinct.
PA_DEBUG_HIDDEN pa_status slots(const int32_t* slot_mapping, int32_t n, int32_t num_blocks, int32_t block_size,
                                hipStream_t stream);
// Copy pairs: sources in [0, src_blocks), destinations in [0, dst_blocks) and
// distinct; within one pool (same_pool) no destination is also a source.
PA_DEBUG_HIDDEN pa_status pairs(const int32_t* block_pairs, int32_t n, int32_t src_blocks, int32_t dst_blocks,
                                bool same_pool, hipStream_t stream);
// Groups of the shared-prefix decode: group_starts non-decreasing within
// [0, num_seqs]; prefix_lens multiples of block_size, <= context_lens and
// max_prefix_len, equal within a group, 0 outside every group; context_lens[s] -
// prefix_lens[s] <= max_suffix_len; each member's first prefix_lens / block_size
// table entries equal its group's first sequence's.
PA_DEBUG_HIDDEN pa_status groups(const DecodeView& v, const int32_t* group_starts, const int32_t* prefix_lens,
                                 int32_t num_groups, int32_t max_prefix_len, int32_t max_suffix_len,
                                 hipStream_t stream);

#undef PA_DEBUG_HIDDEN

#else  // checks compiled out

inline pa_status decode_data(DecodeView*, const int32_t*, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                             int32_t, hipStream_t) {
  return PA_OK;
}
inline pa_status lengths(const int32_t*, int32_t, int32_t, hipStream_t) { return PA_OK; }
inline pa_status seq_order(const int32_t*, int32_t, hipStream_t) { return PA_OK; }
inline pa_status new_rows(const DecodeView&) { return PA_OK; }
inline pa_status extra_rows(const DecodeView&, const int32_t*, int32_t, int32_t, hipStream_t) { return PA_OK; }
inline pa_status slots(const int32_t*, int32_t, int32_t, int32_t, hipStream_t) { return PA_OK; }
inline pa_status pairs(const int32_t*, int32_t, int32_t, int32_t, bool, hipStream_t) { return PA_OK; }
inline pa_status groups(const DecodeView&, const int32_t*, const int32_t*, int32_t, int32_t, int32_t,
                        hipStream_t) {
  return PA_OK;
}

#endif

}  // namespace debug
}  // namespace pa

#endif  // PA_DEBUG_H_
