// pa_decode_noalloc: pa_decode with its split-context workspace in a file-scope
// device array of this library, for callers that cannot allocate device memory.
// The contract is documented in include/pa.h.
//
// The array is a static __device__ variable: every GPU the library runs on holds its
// own copy, at its own address, from the moment the code object is loaded until the
// process ends.  Host code never passes the array's name to a kernel (on the host the
// name is only a stand-in for the symbol); it asks the runtime for the device address
// once per device and passes that.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "pa.h"
#include "pa_status.h"

namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_lookup;

// Address of this library's scratch array on the current device: looked up with the
// device current on its first use there, then reused.
pa_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess)
    return pa::set_error(PA_ERR_HIP, "pa_decode_noalloc: hipGetDevice: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return pa::set_error(PA_ERR_UNSUPPORTED, "pa_decode_noalloc: device %d beyond the %d the library tracks", dev,
                         kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (err != hipSuccess || !p)
        return pa::set_error(PA_ERR_HIP, "pa_decode_noalloc: address of the scratch array on device %d: %s", dev,
                             hipGetErrorString(err));
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_noalloc(void* out, const void* query, const void* key_cache, const void* value_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
                            int32_t partition_size, void* stream) {
  // the size first, on the host: a request beyond the array is refused before anything
  // is looked up or enqueued (invalid arguments give 0 here and are reported by
  // pa_decode's own checks below)
  const size_t need = pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, block_size, max_context_len,
                                                partition_size);
  if (need > kScratchBytes)
    return pa::set_error(PA_ERR_WORKSPACE,
                         "pa_decode_noalloc: these arguments need %zu bytes of workspace, the library's "
                         "scratch array holds %zu (PA_NOALLOC_SCRATCH_BYTES)",
                         need, kScratchBytes);
  // every sequence in one partition: no workspace at all (pa_decode checks the rest)
  void* ws = nullptr;
  if (need > 0) {
    pa_status st = scratch_on_current_device(&ws);
    if (st != PA_OK) return st;
  }
  return pa_decode(out, query, key_cache, value_cache, block_tables, context_lens, num_seqs, num_heads, head_dim,
                   block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype, partition_size, ws,
                   ws ? kScratchBytes : 0, stream);
}

}  // extern "C"
