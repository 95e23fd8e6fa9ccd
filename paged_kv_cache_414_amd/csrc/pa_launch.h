// Internal interface between the C ABI (pa_api.cpp) and the HIP kernels
// (pa_kernels.hip).  Arguments here are already validated.
#ifndef PA_LAUNCH_H_
#define PA_LAUNCH_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct DecodeParams {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_m;  // [S, H, NP]
  float* ws_l;  // [S, H, NP]
  float* ws_o;  // [S, H, NP, D]
  int32_t num_seqs;
  int32_t num_heads;
  int32_t max_blocks_per_seq;
  int32_t partition_tokens;  // P, a multiple of the block size
  int32_t num_partitions;    // NP reserved per (seq, head) = grid.x
  float scale;
};

struct ReduceParams {
  void* out;
  const float* ws_m;
  const float* ws_l;
  const float* ws_o;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t partition_tokens;
  int32_t num_partitions;
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
  void* key_cache;
  void* value_cache;
  const int32_t* block_pairs;
  int32_t num_pairs;
  int64_t block_bytes;  // heads * block_size * head_dim * element size
};

hipError_t launch_decode_partitions(const DecodeParams& prm, bool f16, int head_dim,
                                    int block_size, hipStream_t stream);
hipError_t launch_decode_reduce(const ReduceParams& prm, bool f16, int head_dim,
                                hipStream_t stream);
hipError_t launch_cache_append(const AppendParams& prm, hipStream_t stream);
hipError_t launch_block_copy(const CopyParams& prm, hipStream_t stream);

}  // namespace pa

#endif  // PA_LAUNCH_H_
