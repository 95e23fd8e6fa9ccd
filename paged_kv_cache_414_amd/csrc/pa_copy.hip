// Data movement of the paged KV cache on gfx950 (CDNA4, wave64): the slot-mapped
// append of new K/V rows and the block copy.
//
// Pages cited (title, then section):
//   [Reading vLLM]  "啃透vLLM源码：从PagedAttention到连续批处理，大模型推理加速24倍的秘密"
//   [vLLM basics]   "vLLM基础：架构、推理流程与关键组件"
//
// Pools are laid out [num_blocks, num_heads, block_size, head_dim].  A slot is
// block * block_size + offset: a block fills slot by slot as its sequence grows
// ([Reading vLLM] §2.2, logical blocks appending tokens).  A block copy duplicates
// every head of a block, K and V: the private copy a sharer of a ref-counted block
// gets before it writes ([vLLM basics] §2.3, copy-on-write), and, between the GPU
// pool and a pinned host pool of the same layout, the swap of a preempted
// sequence's blocks ([Reading vLLM] §3).  Both kernels move bits unchanged.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_launch.h"

namespace pa {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

[[maybe_unused]] __device__ __forceinline__ u32x4 load16(const char* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

[[maybe_unused]] __device__ __forceinline__ void store16(char* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Whole blocks are touched once per copy: streaming (non-temporal) loads and stores.
__device__ __forceinline__ u32x4 load16_stream(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void store16_stream(char* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// 16-byte chunks of K and as many of V that one copy thread moves per step, every
// load issued before the first store (the pools may alias as far as the compiler
// knows, so a store would otherwise hold back the next load).  Measured on MI355X
// (2048 pairs of 128 KiB K + 128 KiB V blocks, GB/s read + written): plain loads
// and stores 4,940 at 256 threads; streaming 5,080 at 256 threads and 5,110 at 512;
// hipMemcpy of 512 MiB device to device 5,310.
constexpr int kCopyChunksPerThread = 4;
constexpr int kCopyThreads = 512;
constexpr int kAppendThreads = 256;

// The append streams too: its rows are read once and the pool rows it writes are next
// read by a decode, which streams them from HBM.  Measured on MI355X (4,096 prompt rows
// into 256 whole blocks, 134 MB read + written): 26.1 us streaming against 27.2-27.4 us
// with plain loads and stores; moving 2 or 4 tokens per thread with every load issued
// first was slower (29.5-31.2 us).  (Block copy, same machine: 8 or 2 chunks per thread
// instead of 4, or 256 threads per workgroup, measured no faster.)
#ifndef PA_APPEND_STREAM
#define PA_APPEND_STREAM 1
#endif

__device__ __forceinline__ u32x4 append_load(const char* p) {
#if PA_APPEND_STREAM
  return load16_stream(p);
#else
  return load16(p);
#endif
}

__device__ __forceinline__ void append_store(char* p, const u32x4& v) {
#if PA_APPEND_STREAM
  store16_stream(p, v);
#else
  store16(p, v);
#endif
}

// ---------------------------------------------------------------------------------
// cache append: grid (chunk groups of a token's rows, tokens); one thread per 16
// bytes of a (token, head) row, K and V.  All threads of a workgroup serve one token,
// so its slot is one uniform load.
// ---------------------------------------------------------------------------------

__global__ __launch_bounds__(kAppendThreads) void cache_append_kernel(AppendParams prm) {
  const int chunks = prm.row_bytes / 16;  // per (token, head) row
  const int64_t c_row = static_cast<int64_t>(blockIdx.x) * kAppendThreads + threadIdx.x;
  if (c_row >= static_cast<int64_t>(prm.num_heads) * chunks) return;
  const int h = static_cast<int>(c_row) / chunks;
  const int c = static_cast<int>(c_row) - h * chunks;
  for (int64_t i = blockIdx.y; i < prm.num_tokens; i += gridDim.y) {
    const int slot = prm.slot_mapping[i];
    if (slot < 0) continue;
    const int b = slot / prm.block_size;
    const int o = slot - b * prm.block_size;
    const size_t dst = ((static_cast<size_t>(b) * prm.num_heads + h) * prm.block_size + o) *
                           static_cast<size_t>(prm.row_bytes) + static_cast<size_t>(c) * 16;
    const size_t src = (static_cast<size_t>(i) * prm.num_heads + h) * prm.row_bytes +
                       static_cast<size_t>(c) * 16;
    const u32x4 kv = append_load(static_cast<const char*>(prm.key) + src);
    const u32x4 vv = append_load(static_cast<const char*>(prm.value) + src);
    append_store(static_cast<char*>(prm.key_cache) + dst, kv);
    append_store(static_cast<char*>(prm.value_cache) + dst, vv);
  }
}

// ---------------------------------------------------------------------------------
// block copy between pools (the same pool for copy-on-write, the GPU pool and a
// pinned host pool for swapping): grid (pairs, chunk groups of a block)
// ---------------------------------------------------------------------------------

__global__ __launch_bounds__(kCopyThreads) void block_copy_kernel(CopyParams prm) {
  const int pair = blockIdx.x;
  const int src = prm.block_pairs[2 * pair];
  const int dst = prm.block_pairs[2 * pair + 1];
  const int64_t chunks = prm.block_bytes / 16;
  const char* ks = static_cast<const char*>(prm.src_key) + static_cast<size_t>(src) * prm.block_bytes;
  const char* vs = static_cast<const char*>(prm.src_value) + static_cast<size_t>(src) * prm.block_bytes;
  char* kd = static_cast<char*>(prm.dst_key) + static_cast<size_t>(dst) * prm.block_bytes;
  char* vd = static_cast<char*>(prm.dst_value) + static_cast<size_t>(dst) * prm.block_bytes;
  constexpr int64_t kSpan = static_cast<int64_t>(kCopyThreads) * kCopyChunksPerThread;
  for (int64_t base = static_cast<int64_t>(blockIdx.y) * kSpan + threadIdx.x; base < chunks;
       base += static_cast<int64_t>(gridDim.y) * kSpan) {
    u32x4 k[kCopyChunksPerThread];
    u32x4 v[kCopyChunksPerThread];
#pragma unroll
    for (int j = 0; j < kCopyChunksPerThread; ++j) {
      const int64_t c = base + static_cast<int64_t>(j) * kCopyThreads;
      if (c < chunks) {
        k[j] = load16_stream(ks + c * 16);
        v[j] = load16_stream(vs + c * 16);
      }
    }
#pragma unroll
    for (int j = 0; j < kCopyChunksPerThread; ++j) {
      const int64_t c = base + static_cast<int64_t>(j) * kCopyThreads;
      if (c < chunks) {
        store16_stream(kd + c * 16, k[j]);
        store16_stream(vd + c * 16, v[j]);
      }
    }
  }
}

}  // namespace

// The caller has checked num_heads * (row_bytes / 16) <= INT32_MAX.
hipError_t launch_cache_append(const AppendParams& prm, hipStream_t stream) {
  const int64_t row_chunks = static_cast<int64_t>(prm.num_heads) * (prm.row_bytes / 16);
  const int64_t gx = (row_chunks + kAppendThreads - 1) / kAppendThreads;
  const int32_t gy = prm.num_tokens < 65535 ? prm.num_tokens : 65535;  // tokens past it loop
  hipLaunchKernelGGL(cache_append_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                     dim3(kAppendThreads), 0, stream, prm);
  return hipGetLastError();
}

hipError_t launch_block_copy(const CopyParams& prm, hipStream_t stream) {
  const int64_t chunks = prm.block_bytes / 16;
  const int64_t span = static_cast<int64_t>(kCopyThreads) * kCopyChunksPerThread;
  int64_t gy = (chunks + span - 1) / span;  // one step per thread when it fits
  if (gy < 1) gy = 1;
  if (gy > 1024) gy = 1024;
  hipLaunchKernelGGL(block_copy_kernel, dim3(prm.num_pairs, static_cast<unsigned>(gy)), dim3(kCopyThreads), 0,
                     stream, prm);
  return hipGetLastError();
}

}  // namespace pa
