// Staging copy of the decode-step executor (pa_step.cpp): pinned host memory ->
// device memory, one 16-byte word per thread.  Each step's small arrays (slots,
// block tables, context lengths, ...) move with this kernel rather than with an
// asynchronous copy by the DMA engines: the kernels that read the arrays then follow
// it in the same queue, with no hand-over between engines on every step.  When no
// copy-on-write is due, the step's slot-mapped append of its new K/V rows rides in
// the same launch (one launch and one inter-kernel gap less per step).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_launch.h"

namespace pa {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Thread 0 of workgroup 0 first writes `step` into the host word `flag` (when given):
// a step's staging kernel starts only after the previous step's kernels have finished,
// so the host learns from it that the previous staging kernel has read its pinned
// buffer, with no event in the queue.
__device__ __forceinline__ void mark_started(int32_t* flag, int32_t step) {
  if (flag && blockIdx.x == 0 && threadIdx.x == 0) *reinterpret_cast<volatile int32_t*>(flag) = step;
}

__global__ __launch_bounds__(256) void stage_copy_kernel(const u32x4* src, u32x4* dst, int64_t words,
                                                         int32_t* flag, int32_t step) {
  mark_started(flag, step);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    dst[i] = src[i];
}

// Workgroups [0, stage_groups) copy the staging words; the rest write one 16-byte
// chunk of a K row and of a V row per thread into the pools, exactly as
// cache_append_kernel does (row i of key/value, head h, to the slot's block and
// offset), reading each row's slot from the pinned buffer over the host link.
__global__ __launch_bounds__(256) void stage_copy_append_kernel(const u32x4* src, u32x4* dst, int64_t words,
                                                                int32_t stage_groups, AppendParams prm,
                                                                int32_t* flag, int32_t step) {
  mark_started(flag, step);
  if (static_cast<int32_t>(blockIdx.x) < stage_groups) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words;
         i += static_cast<int64_t>(stage_groups) * blockDim.x)
      dst[i] = src[i];
    return;
  }
  const int64_t idx = static_cast<int64_t>(blockIdx.x - stage_groups) * blockDim.x + threadIdx.x;
  const int chunks = prm.row_bytes / 16;
  const int64_t total = static_cast<int64_t>(prm.num_tokens) * prm.num_heads * chunks;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % chunks);
  const int64_t th = idx / chunks;  // token * heads + head
  const int h = static_cast<int>(th % prm.num_heads);
  const int i = static_cast<int>(th / prm.num_heads);
  const int slot = prm.slot_mapping[i];
  if (slot < 0) return;
  const int b = slot / prm.block_size;
  const int o = slot % prm.block_size;
  const size_t to = ((static_cast<size_t>(b) * prm.num_heads + h) * prm.block_size + o) *
                        static_cast<size_t>(prm.row_bytes) + static_cast<size_t>(c) * 16;
  const size_t from = static_cast<size_t>(th) * prm.row_bytes + static_cast<size_t>(c) * 16;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(prm.key) + from);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(prm.value) + from);
  *reinterpret_cast<u32x4*>(static_cast<char*>(prm.key_cache) + to) = kv;
  *reinterpret_cast<u32x4*>(static_cast<char*>(prm.value_cache) + to) = vv;
}

}  // namespace

hipError_t launch_stage_copy(const void* src, void* dst, int64_t bytes, int32_t* flag, int32_t step,
                             hipStream_t stream) {
  const int64_t words = bytes / 16;
  int64_t groups = (words + 255) / 256;
  if (groups > 64) groups = 64;  // grid-stride beyond 64 x 256 words (256 KiB)
  if (groups < 1) groups = 1;    // the flag is written even with nothing to copy
  hipLaunchKernelGGL(stage_copy_kernel, dim3(static_cast<unsigned>(groups)), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), words, flag, step);
  return hipGetLastError();
}

hipError_t launch_stage_copy_append(const void* src, void* dst, int64_t bytes, const AppendParams& append,
                                    int32_t* flag, int32_t step, hipStream_t stream) {
  const int64_t words = bytes / 16;
  int64_t stage_groups = (words + 255) / 256;
  if (stage_groups > 64) stage_groups = 64;
  const int64_t threads = static_cast<int64_t>(append.num_tokens) * append.num_heads * (append.row_bytes / 16);
  int64_t groups = stage_groups + (threads + 255) / 256;
  if (groups < 1) groups = 1;  // the flag is written even with nothing to copy
  hipLaunchKernelGGL(stage_copy_append_kernel, dim3(static_cast<unsigned>(groups)), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), words,
                     static_cast<int32_t>(stage_groups), append, flag, step);
  return hipGetLastError();
}

}  // namespace pa
