// Internal interface between the C ABI (pa_api.cpp) and the HIP kernels
// (pa_kernels.hip: decode; pa_copy.hip: append and block copy).  Arguments here
// are already validated.
#ifndef PA_LAUNCH_H_
#define PA_LAUNCH_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Wave64s per workgroup of the decode partition pass: narrow for short partitions or
// launches of few workgroups, wide otherwise (DecodeParams::wide, chosen on the host).
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 8
#endif
#ifndef PA_DECODE_WAVES_WIDE
#define PA_DECODE_WAVES_WIDE 16
#endif
constexpr int kDecodeWavesNarrow = PA_DECODE_WAVES;
constexpr int kDecodeWavesWide = PA_DECODE_WAVES_WIDE;
#ifndef PA_SHARED_FUSED
#define PA_SHARED_FUSED 0  // 1: the shared-prefix decode runs both passes in one launch
#endif

// 16-byte chunks of K (and as many of V) a thread of the decode launch's trailing
// append workgroups moves with every load issued before the first store
constexpr int kExtraChunksPerThread = 2;

struct DecodeParams {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* token_begin;  // [S] first token of each sequence to attend, or nullptr (= 0)
  float* ws_m;  // [S, H, slots_per_pair]
  float* ws_l;  // [S, H, slots_per_pair]
  float* ws_o;  // [S, H, slots_per_pair, D]
  int32_t num_seqs;
  int32_t num_heads;
  int32_t max_blocks_per_seq;
  int32_t partition_tokens;  // P, a multiple of the block size
  int32_t num_partitions;    // partitions launched per (seq, head) = grid.x
  int32_t slots_per_pair;    // partial-state slots reserved per (seq, head)
  int32_t slot_offset;       // slot of partition 0 of this pass (= prefix slots)
  int32_t prefix_partition_tokens;  // with token_begin: the prefix states' partition length
  int32_t wide;              // 1: kDecodeWavesWide wave64s per workgroup, 0: kDecodeWavesNarrow
  float scale;
  // pa_decode_append: the row of each sequence's position context_lens[s] - 1 is
  // taken from new_key / new_value [S, H, D] and also written into the pools at that
  // position (the pools are then written through key_cache / value_cache); nullptr
  // for a plain decode.  Only with token_begin == nullptr.
  const void* new_key = nullptr;
  const void* new_value = nullptr;
  // [S] or nullptr: the workgroups of grid slice z decode sequence seq_order[z] (a
  // permutation of the batch), so the caller chooses the dispatch order
  const int32_t* seq_order = nullptr;
  // Rows appended by trailing workgroups of the same launch (a decode step's admitted
  // prompts): row i of extra_key / extra_value [extra_tokens, H, D] goes to slot
  // extra_slots[i] (negative: skipped), extra_per_group rows per workgroup.  The
  // caller guarantees that no such slot lies in a block this launch reads.
  const void* extra_key = nullptr;
  const void* extra_value = nullptr;
  const int32_t* extra_slots = nullptr;
  int32_t extra_tokens = 0;
  int32_t extra_per_group = 0;
  // 1: every partition writes its state to the workspace (none finishes a sequence),
  // for a merge pass with ReduceParams::merge_all; the prefix states may not exist yet
  int32_t states_only = 0;
  // heads one workgroup folds together (decode_heads_per_unit): grid y = num_heads / it
  int32_t heads_per_unit = 1;
  // The decode-step executor's word (device view of pinned host memory) into which
  // thread 0 of the launch's first workgroup writes `step` as the launch starts, or
  // nullptr
  int32_t* started_flag = nullptr;
  int32_t step = 0;
};

// Prefix pass of the shared-prefix decode: one workgroup per (prefix partition,
// head, group, tile of 16 of the group's queries); groups are ranges of sequences
// that share leading blocks.
struct PrefixParams {
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* group_starts;  // [G + 1]
  const int32_t* prefix_lens;   // [S]
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int32_t num_heads;
  int32_t max_blocks_per_seq;
  int32_t partition_tokens;  // a multiple of 16 and of the block size
  int32_t num_partitions;    // grid.x
  int32_t num_groups;        // grid.z = num_groups * query_tiles
  int32_t query_tiles;       // workgroups per (partition, head, group): 16 members each
  int32_t slots_per_pair;
  float scale;
};

struct ReduceParams {
  void* out;
  const float* ws_m;
  const float* ws_l;
  const float* ws_o;
  const int32_t* context_lens;
  const int32_t* prefix_lens;  // [S] tokens covered by the prefix pass, or nullptr
  int32_t num_seqs;
  int32_t num_heads;
  int32_t partition_tokens;         // of the states after the prefix
  int32_t prefix_partition_tokens;  // of the prefix states
  int32_t prefix_slots;             // slots [0, prefix_slots) hold prefix states
  int32_t slots_per_pair;
  // 1: merge and write every (sequence, head), also those with at most one state
  // after the prefix (zero output for an empty context); 0: only those with more
  int32_t merge_all = 0;
};

struct AppendParams {
  void* key_cache;
  void* value_cache;
  const void* key;
  const void* value;
  const int32_t* slot_mapping;
  int32_t num_tokens;
  int32_t num_heads;
  int32_t block_size;
  int32_t row_bytes;  // head_dim * element size, a multiple of 16
};

struct CopyParams {
  const void* src_key;  // source pool (block ids: first of each pair)
  const void* src_value;
  void* dst_key;        // destination pool (second of each pair); may be the source pool
  void* dst_value;
  const int32_t* block_pairs;
  int32_t num_pairs;
  int64_t block_bytes;  // heads * block_size * head_dim * element size
};

// Heads a decode workgroup folds per unit for this shape: 2 where a (block, head) chunk
// is 4 KiB and num_heads is even (the chunks of two adjacent heads are one 8 KiB run),
// else 1.  The result does not depend on it.
int32_t decode_heads_per_unit(bool f16, int head_dim, int block_size, int num_heads);
// z-slices of store workgroups the partition pass adds for pa_decode_append (0 otherwise)
int32_t store_slices(const DecodeParams& prm);
// z-slices of workgroups appending the extra rows (0 without them), after the store slices
int32_t extra_slices(const DecodeParams& prm);
hipError_t launch_decode_partitions(const DecodeParams& prm, bool f16, int head_dim,
                                    int block_size, hipStream_t stream);
hipError_t launch_decode_reduce(const ReduceParams& prm, bool f16, int head_dim,
                                hipStream_t stream);
hipError_t launch_decode_prefix(const PrefixParams& prm, int head_dim, int block_size,
                                hipStream_t stream);
// The prefix pass (pp) and the pass after the prefix (dp, states_only, 8 waves) in one
// launch; the caller then merges with launch_decode_reduce (merge_all).
hipError_t launch_decode_shared_fused(const PrefixParams& pp, const DecodeParams& dp, int head_dim, int block_size,
                                      hipStream_t stream);
hipError_t launch_cache_append(const AppendParams& prm, hipStream_t stream);
hipError_t launch_block_copy(const CopyParams& prm, hipStream_t stream);
// bytes / 16 words from `src` (device-visible pinned host memory) to `dst` (device);
// bytes a multiple of 16, both 16-byte aligned.  When `flag` (device view of a pinned
// host word) is given, the kernel writes `step` into it as it starts.
hipError_t launch_stage_copy(const void* src, void* dst, int64_t bytes, int32_t* flag, int32_t step,
                             hipStream_t stream);
// The staging copy and the slot-mapped append of `append` in one launch: the
// append's slot_mapping is read from the pinned host buffer itself (device view),
// not from the staged copy being written by the same launch.  `flag` as above.
hipError_t launch_stage_copy_append(const void* src, void* dst, int64_t bytes, const AppendParams& append,
                                    int32_t* flag, int32_t step, hipStream_t stream);

}  // namespace pa

#endif  // PA_LAUNCH_H_
