// Decode-step executor: one host call per decode step (block manager, staging of
// the step's small arrays in pinned memory, one host-to-device copy, the kernels of
// pa.h).  The contract is documented in include/pa_step.h.

#include "pa_step.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdint>
#include <thread>
#include <new>
#include <vector>

#include "pa_debug.h"
#include "pa_launch.h"
#include "pa_status.h"

namespace {

constexpr int64_t kAlign = 4;  // int32 elements: every staged array starts 16-byte aligned

int64_t aligned(int64_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// True once the staging kernel of step `step` (or a later one) has started: the
// kernel writes its step number into the pinned word as it starts (step numbers
// compared modulo 2^32).
bool step_started(const int32_t* word, uint32_t step) {
  const uint32_t seen = static_cast<uint32_t>(__atomic_load_n(word, __ATOMIC_ACQUIRE));
  return static_cast<int32_t>(seen - step) >= 0;
}

// One-launch steps (see step 4 of pa_step_run), and whether they keep the longest-first
// dispatch order.  Measured on one MI355X, interleaved builds, wall clock of
// the warm mixes (seq.steps/s): continuous batching 794-803K through the staging
// kernel, 801-805K in one launch with the longest-first order (each workgroup first
// reads its slot of the order from the pinned buffer, one more dependent trip over
// the host link), 817-823K in one launch in batch order; the shared-prefix mix through
// pa_decode 615-616K staged, 627-636K in one launch.
#ifndef PA_STEP_DIRECT
#define PA_STEP_DIRECT 1  // 0: every step's arrays go through the staging kernel
#endif
#ifndef PA_STEP_DIRECT_ORDER
#define PA_STEP_DIRECT_ORDER 0  // 1: one-launch steps keep the longest-first order
#endif

// How long the host polls the word before it falls back to synchronizing the stream.
constexpr auto kPollFor = std::chrono::milliseconds(5);

pa_status hip_fail(hipError_t err, const char* what) {
  return pa::set_error(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

template <typename T>
bool all_distinct(const T* ids, int32_t n, std::vector<T>& scratch) {
  scratch.assign(ids, ids + n);
  std::sort(scratch.begin(), scratch.end());
  return std::adjacent_find(scratch.begin(), scratch.end()) == scratch.end();
}

}  // namespace

struct pa_step_engine {
  pa_block_manager* bm = nullptr;
  pa_step_config cfg{};
  int32_t block_size = 0;
  int32_t num_blocks = 0;
  void* key_cache = nullptr;
  void* value_cache = nullptr;
  int device = 0;

  // Staging layout, int32 offsets; the same in the pinned and the device buffer.
  int64_t off_pairs = 0, off_slots = 0, off_tables = 0, off_ctx = 0, off_starts = 0,
          off_prefix = 0, off_order = 0, off_admit = 0, capacity = 0;
  int32_t* host[2] = {nullptr, nullptr};       // pinned, written by the host
  const void* host_dev[2] = {nullptr, nullptr};  // the same buffers as the device sees them
  // Pinned host word into which each step's staging kernel writes its step number as it
  // starts; step numbers count the staging launches (wrapping at 2^32).
  int32_t* started = nullptr;
  int32_t* started_dev = nullptr;
  uint32_t next_step = 0;
  bool used[2] = {false, false};       // buffer i has staged a step ...
  uint32_t used_by[2] = {0, 0};        // ... this one
  bool any_step = false;
  int turn = 0;
  int32_t* dev = nullptr;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;

  std::vector<int32_t> positions;
  std::vector<int64_t> id_scratch;
  std::vector<int32_t> order;

  // the last step, for pa_step_last
  bool has_last = false;
  int last_turn = 0;
  int32_t last_n = 0;
  int32_t last_groups = 0;
  pa_step_result last{};
  pa_decode_hints last_hints{};
  bool last_direct = false;  // the last step's decode read the pinned buffer itself

  ~pa_step_engine() {
    // the device may still run the last step, reading the staging buffers and the
    // workspace: wait for it before freeing them
    if (any_step) {
      int current = device;
      (void)hipGetDevice(&current);
      if (current != device) (void)hipSetDevice(device);
      (void)hipDeviceSynchronize();
      if (current != device) (void)hipSetDevice(current);
    }
    for (int i = 0; i < 2; ++i)
      if (host[i]) (void)hipHostFree(host[i]);
    if (started) (void)hipHostFree(started);
    if (dev) (void)hipFree(dev);
    if (workspace) (void)hipFree(workspace);
  }

  const int32_t* dev_at(int64_t off) const { return dev + off; }
  int32_t* dev_at(int64_t off) { return dev + off; }
};

extern "C" {

pa_step_engine* pa_step_create(pa_block_manager* bm, const pa_step_config* config, void* key_cache,
                               void* value_cache) {
  if (!bm || !config || !key_cache || !value_cache) {
    pa::set_error(PA_ERR_NULL, "manager, config and both pools must not be NULL");
    return nullptr;
  }
  if (!aligned16(key_cache) || !aligned16(value_cache)) {
    pa::set_error(PA_ERR_INVALID_ARG, "pools must be 16-byte aligned");
    return nullptr;
  }
  const pa_step_config& c = *config;
  const int32_t bs = pa_bm_block_size(bm);
  if (pa::check_dtype_shape(c.dtype, c.head_dim, bs) != PA_OK) return nullptr;
  if (c.num_heads <= 0 || c.max_seqs <= 0 || c.max_blocks_per_seq <= 0 || c.max_admit_tokens < 0 ||
      c.max_groups < 0) {
    pa::set_error(PA_ERR_INVALID_ARG,
                  "num_heads %d, max_seqs %d, max_blocks_per_seq %d must be positive; max_admit_tokens %d "
                  "and max_groups %d non-negative",
                  c.num_heads, c.max_seqs, c.max_blocks_per_seq, c.max_admit_tokens, c.max_groups);
    return nullptr;
  }
  if (c.max_groups > 0 && c.dtype != PA_F16) {
    // the shared-prefix decode is built for fp16; refused here, not halfway through a step
    pa::set_error(PA_ERR_UNSUPPORTED, "max_groups %d needs PA_F16 pools (the shared-prefix decode)", c.max_groups);
    return nullptr;
  }
  if (static_cast<int64_t>(c.max_blocks_per_seq) * bs > INT32_MAX) {
    pa::set_error(PA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size exceeds the int32 range");
    return nullptr;
  }
  pa_step_engine* e = new (std::nothrow) pa_step_engine;
  if (!e) {
    pa::set_error(PA_ERR_INVALID_ARG, "out of host memory");
    return nullptr;
  }
  e->bm = bm;
  e->cfg = c;
  e->block_size = bs;
  e->num_blocks = pa_bm_num_blocks(bm);
  e->key_cache = key_cache;
  e->value_cache = value_cache;

  const int64_t s = c.max_seqs;
  int64_t at = 0;
  e->off_pairs = at;  at += aligned(2 * s);
  e->off_slots = at;  at += aligned(s);
  e->off_tables = at; at += aligned(s * c.max_blocks_per_seq);
  e->off_ctx = at;    at += aligned(s);
  e->off_starts = at; at += c.max_groups > 0 ? aligned(c.max_groups + 1) : 0;
  e->off_prefix = at; at += c.max_groups > 0 ? aligned(s) : 0;
  e->off_order = at;  at += aligned(s);
  e->off_admit = at;  at += aligned(c.max_admit_tokens);
  e->capacity = at;
  e->positions.resize(s);
  e->order.resize(s);

  hipError_t err = hipGetDevice(&e->device);
  const size_t bytes = static_cast<size_t>(e->capacity) * sizeof(int32_t);
  for (int i = 0; i < 2 && err == hipSuccess; ++i) {
    // coherent: the staging kernel reads what the host wrote just before the launch
    err = hipHostMalloc(reinterpret_cast<void**>(&e->host[i]), bytes,
                        hipHostMallocMapped | hipHostMallocCoherent);
    void* mapped = nullptr;
    if (err == hipSuccess) err = hipHostGetDevicePointer(&mapped, e->host[i], 0);
    e->host_dev[i] = mapped;
  }
  if (err == hipSuccess)
    err = hipHostMalloc(reinterpret_cast<void**>(&e->started), 64, hipHostMallocMapped | hipHostMallocCoherent);
  if (err == hipSuccess) {
    *e->started = -1;
    void* mapped = nullptr;
    err = hipHostGetDevicePointer(&mapped, e->started, 0);
    e->started_dev = static_cast<int32_t*>(mapped);
  }
  if (err == hipSuccess) err = hipMalloc(reinterpret_cast<void**>(&e->dev), bytes);
  if (err != hipSuccess) {
    hip_fail(err, "pa_step_create: allocation");
    delete e;
    return nullptr;
  }
  pa::clear_error();
  return e;
}

void pa_step_destroy(pa_step_engine* engine) { delete engine; }

pa_status pa_step_run(pa_step_engine* e, const pa_step_args* a, void* stream, pa_step_result* result) {
  if (!e || !a) return pa::set_error(PA_ERR_NULL, "engine and args must not be NULL");
  const pa_step_config& c = e->cfg;
  const int32_t n = a->num_seqs;
  const int32_t bs = e->block_size;
  const int32_t mb = c.max_blocks_per_seq;

  // ---- argument checks: nothing changes before all of them pass ----
  if (n < 1 || n > c.max_seqs)
    return pa::set_error(PA_ERR_INVALID_ARG, "num_seqs %d outside [1, %d]", n, c.max_seqs);
  if (!a->seq_ids || !a->query || !a->new_key || !a->new_value || !a->out)
    return pa::set_error(PA_ERR_NULL, "seq_ids, query, new_key, new_value and out must not be NULL");
  if (!aligned16(a->query) || !aligned16(a->new_key) || !aligned16(a->new_value) || !aligned16(a->out) ||
      !aligned16(a->prompt_key) || !aligned16(a->prompt_value))
    return pa::set_error(PA_ERR_INVALID_ARG, "query, rows, out and prompt rows must be 16-byte aligned");
  if (a->num_groups < 0 || a->num_groups > c.max_groups)
    return pa::set_error(PA_ERR_INVALID_ARG, "num_groups %d outside [0, %d]", a->num_groups, c.max_groups);
  const int32_t g_count = a->num_groups;
  if (g_count > 0) {
    if (!a->group_starts) return pa::set_error(PA_ERR_NULL, "group_starts must not be NULL");
    if (a->group_starts[0] != 0 || a->group_starts[g_count] != n)
      return pa::set_error(PA_ERR_INVALID_ARG, "group_starts must run from 0 to num_seqs %d", n);
    for (int32_t g = 0; g < g_count; ++g) {
      if (a->group_starts[g + 1] < a->group_starts[g])
        return pa::set_error(PA_ERR_INVALID_ARG, "group_starts must be non-decreasing");
    }
  }
  if (a->num_finished < 0 || a->num_admit < 0)
    return pa::set_error(PA_ERR_INVALID_ARG, "num_finished %d and num_admit %d must be >= 0", a->num_finished,
                         a->num_admit);
  if (a->num_finished > 0 && !a->finished_ids) return pa::set_error(PA_ERR_NULL, "finished_ids is NULL");
  if (a->num_admit > 0 && (!a->admit_ids || !a->admit_lens))
    return pa::set_error(PA_ERR_NULL, "admit_ids and admit_lens must not be NULL");
  if (!all_distinct(a->seq_ids, n, e->id_scratch))
    return pa::set_error(PA_ERR_INVALID_ARG, "a running sequence is listed twice");
  if (!all_distinct(a->finished_ids, a->num_finished, e->id_scratch))
    return pa::set_error(PA_ERR_INVALID_ARG, "a finished sequence is listed twice");
  if (!all_distinct(a->admit_ids, a->num_admit, e->id_scratch))
    return pa::set_error(PA_ERR_INVALID_ARG, "a request id is listed twice");
  int64_t requested = 0;
  for (int32_t i = 0; i < a->num_admit; ++i) {
    if (a->admit_lens[i] < 0) return pa::set_error(PA_ERR_INVALID_ARG, "admit_lens[%d] is negative", i);
    // an admitted prompt must leave room in its table row for the next decode token,
    // or every later step that lists it would be refused
    if (static_cast<int64_t>(a->admit_lens[i]) >= static_cast<int64_t>(mb) * bs)
      return pa::set_error(PA_ERR_INVALID_ARG,
                           "admit_lens[%d] = %d leaves no room for a decode token in %d blocks of %d tokens", i,
                           a->admit_lens[i], mb, bs);
    if (pa_bm_num_seq_blocks(e->bm, a->admit_ids[i]) >= 0)
      return pa::set_error(PA_ERR_INVALID_ARG, "request id %lld is a known sequence", (long long)a->admit_ids[i]);
    requested += a->admit_lens[i];
  }
  if (requested > c.max_admit_tokens)
    return pa::set_error(PA_ERR_INVALID_ARG, "%lld prompt tokens requested, the executor stages %d",
                         (long long)requested, c.max_admit_tokens);
  if (requested > 0 && (!a->prompt_key || !a->prompt_value))
    return pa::set_error(PA_ERR_NULL, "prompt_key and prompt_value must not be NULL");
  for (int32_t i = 0; i < a->num_finished; ++i) {
    if (pa_bm_num_seq_blocks(e->bm, a->finished_ids[i]) < 0)
      return pa::set_error(PA_ERR_INVALID_ARG, "finished sequence %lld is unknown", (long long)a->finished_ids[i]);
  }
  int current_device = 0;
  hipError_t err = hipGetDevice(&current_device);
  if (err != hipSuccess) return hip_fail(err, "pa_step_run: hipGetDevice");
  if (current_device != e->device)
    return pa::set_error(PA_ERR_INVALID_ARG, "the executor lives on device %d, device %d is current", e->device,
                         current_device);

  // ---- this step's pinned buffer: the staging kernel that last read it (two steps
  // ago) must be done, which the start of the next staging kernel shows.  No event
  // sits in the queue for this: measured on MI355X, each event record left the queue
  // idle 1.5-2.2 us even without its system-scope fence, and 3.2 us with it. ----
  const int t = e->turn;
  if (e->used[t]) {
    const uint32_t need = e->used_by[t] + 1;
    const auto until = std::chrono::steady_clock::now() + kPollFor;
    while (!step_started(e->started, need) && std::chrono::steady_clock::now() < until)
      std::this_thread::yield();
    if (!step_started(e->started, need)) {
      // the stream is slow or the caller switched streams: wait for the device itself
      err = hipDeviceSynchronize();
      if (err != hipSuccess) return hip_fail(err, "pa_step_run: waiting for the staging copy");
    }
  }
  int32_t* h = e->host[t];
  int32_t* ctx = h + e->off_ctx;

  // Context lengths before the step bound the table width; also rejects unknown ids.
  pa_status st = pa_bm_context_lens(e->bm, a->seq_ids, n, ctx);
  if (st != PA_OK) return st;
  for (int32_t i = 0; i < n; ++i) {
    if (static_cast<int64_t>(ctx[i]) + 1 > static_cast<int64_t>(mb) * bs)
      return pa::set_error(PA_ERR_INVALID_ARG, "sequence %lld would exceed %d blocks", (long long)a->seq_ids[i],
                           mb);
  }

  // ---- 1. slots of the new tokens (all or nothing) ----
  int32_t copies = 0;
  st = pa_bm_append_slots(e->bm, a->seq_ids, n, h + e->off_slots, e->positions.data(), h + e->off_pairs, &copies);
  if (st != PA_OK) return st;

  // ---- 2. tables, lengths, shared prefixes ----
  pa_bm_block_tables(e->bm, a->seq_ids, n, mb, 0, h + e->off_tables);
  int32_t max_ctx = 0;
  for (int32_t i = 0; i < n; ++i) {
    ctx[i] = e->positions[i] + 1;
    max_ctx = std::max(max_ctx, ctx[i]);
  }
  int32_t max_prefix = 0, max_suffix = 0, max_group = 0;
  if (g_count > 0) {
    int32_t* starts = h + e->off_starts;
    int32_t* prefix = h + e->off_prefix;
    for (int32_t g = 0; g <= g_count; ++g) starts[g] = a->group_starts[g];
    for (int32_t g = 0; g < g_count; ++g) {
      const int32_t r0 = starts[g], r1 = starts[g + 1];
      max_group = std::max(max_group, r1 - r0);
      if (r1 == r0) continue;
      const int32_t shared = pa_bm_shared_prefix_blocks(e->bm, a->seq_ids + r0, r1 - r0);
      for (int32_t r = r0; r < r1; ++r) {
        prefix[r] = shared * bs;
        max_prefix = std::max(max_prefix, prefix[r]);
        max_suffix = std::max(max_suffix, ctx[r] - prefix[r]);
      }
    }
  }

  // ---- 3. admit while the blocks fit, then retire ----
  // Admission takes only blocks that were free before this step's retirements: no
  // admitted prompt row lands in a block this step's decode reads, so those rows are
  // written by the decode's own launch.  Blocks given back here serve the next step.
  int32_t admitted = 0;
  int64_t admitted_tokens = 0;
  {
    int64_t free_blocks = pa_bm_num_free(e->bm);
    while (admitted < a->num_admit) {
      const int64_t need = (static_cast<int64_t>(a->admit_lens[admitted]) + bs - 1) / bs;
      if (need > free_blocks) break;
      free_blocks -= need;
      admitted_tokens += a->admit_lens[admitted];
      ++admitted;
    }
    // the ids were checked unknown and distinct and the blocks counted: this succeeds
    if (admitted > 0) {
      st = pa_bm_add_sequences(e->bm, a->admit_ids, a->admit_lens, admitted, h + e->off_admit);
      if (st != PA_OK) return st;
    }
  }
  for (int32_t i = 0; i < a->num_finished; ++i) pa_bm_free(e->bm, a->finished_ids[i]);

  // ---- launch hints of the decode ----
  // Measured on MI355X (fp16, 32 heads x 128): a batch whose sequences re-read shared
  // blocks through pa_decode decodes faster with 8-wave workgroups in batch order (8 x
  // 8 samples sharing 1024 tokens: 108.3 us against 122.1 with 16 waves; longest first
  // 161 us, it splits the groups); other batches with 8 waves and the longest contexts
  // dispatched first (64 x U[1, 562]: 43.1 us against 44.7 with the library's choice;
  // the Llama-shaped batch the same within 0.2 %).  That order costs one-launch steps
  // more than it gains, so they keep batch order (PA_STEP_DIRECT_ORDER).
  pa_decode_hints hints{};
  hints.waves = pa::kDecodeWavesNarrow;
  const bool longest_first = g_count == 0 && !pa::batch_shares_blocks(e->bm, a->seq_ids, n);
  if (longest_first) {
    int32_t* order = h + e->off_order;
    for (int32_t i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order, order + n, [ctx](int32_t x, int32_t y) { return ctx[x] > ctx[y]; });
  }

  // ---- 4. the staged arrays reach the device.  Without copy-on-write and groups the
  // step is one launch: the decode reads them from the pinned buffer itself, attends
  // the step's new rows from new_key / new_value and stores them and the admitted
  // prompts' rows in trailing workgroups.  Otherwise a kernel on the step's stream
  // copies them (with no copy-on-write due, the append of the step's rows rides in
  // that launch). ----
  const int32_t H = c.num_heads, D = c.head_dim, NB = e->num_blocks;
  const int64_t used = aligned(admitted_tokens > 0 ? e->off_admit + admitted_tokens : e->off_admit);
  const int64_t used_bytes = used * static_cast<int64_t>(sizeof(int32_t));
  const bool direct = PA_STEP_DIRECT && copies == 0 && g_count == 0;
  const int32_t* staged = direct ? static_cast<const int32_t*>(e->host_dev[t]) : e->dev;  // as the device reads
  if (longest_first && (PA_STEP_DIRECT_ORDER || !direct)) hints.seq_order = staged + e->off_order;
  const int32_t this_step = static_cast<int32_t>(e->next_step);
  // once the launch that starts the step (and writes its number into the pinned word)
  // is enqueued, buffer t is in use until that word shows the next step
  auto mark_used = [e, t]() {
    e->used[t] = true;
    e->used_by[t] = e->next_step++;
    e->any_step = true;
    e->turn ^= 1;
  };
  err = hipSuccess;
  if (direct) {
    // the decode launch below marks the step started
  } else if (copies == 0) {
    pa::AppendParams ap;
    ap.key_cache = e->key_cache;
    ap.value_cache = e->value_cache;
    ap.key = a->new_key;
    ap.value = a->new_value;
    ap.slot_mapping = static_cast<const int32_t*>(e->host_dev[t]) + e->off_slots;
    ap.num_tokens = n;
    ap.num_heads = H;
    ap.block_size = bs;
    ap.row_bytes = D * (c.dtype == PA_F16 ? 2 : 4);
    st = pa::debug::slots(h + e->off_slots, n, NB, bs, static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
    err = pa::launch_stage_copy_append(e->host_dev[t], e->dev, used_bytes, ap, e->started_dev,
                                       static_cast<int32_t>(e->next_step), static_cast<hipStream_t>(stream));
  } else {
    err = pa::launch_stage_copy(e->host_dev[t], e->dev, used_bytes, e->started_dev,
                                static_cast<int32_t>(e->next_step), static_cast<hipStream_t>(stream));
  }
  if (err != hipSuccess) return hip_fail(err, "pa_step_run: staging copy");
  if (!direct) mark_used();

  // ---- 5. kernels, in stream order ----
  const size_t need_ws =
      g_count > 0 ? pa_decode_shared_prefix_workspace_bytes(n, H, D, bs, g_count, max_group, max_prefix, max_suffix,
                                                            0, 0)
                  : pa_decode_workspace_bytes(n, H, D, bs, max_ctx, 0);
  if (need_ws > e->workspace_bytes) {
    // only earlier steps used the old workspace: wait for them (rare: the workspace
    // only grows)
    if (e->workspace) err = hipDeviceSynchronize();
    if (err == hipSuccess && e->workspace) err = hipFree(e->workspace);
    e->workspace = nullptr;
    e->workspace_bytes = 0;
    const size_t grown = need_ws + need_ws / 4;
    if (err == hipSuccess) err = hipMalloc(&e->workspace, grown);
    if (err != hipSuccess) return hip_fail(err, "pa_step_run: decode workspace");
    e->workspace_bytes = grown;
  }
  if (copies > 0) {  // the copies first: the new rows go into the fresh private blocks
    st = pa_block_copy(e->key_cache, e->value_cache, e->dev_at(e->off_pairs), copies, H, D, bs, NB, c.dtype,
                       stream);
    if (st != PA_OK) return st;
    st = pa_cache_append(e->key_cache, e->value_cache, a->new_key, a->new_value, e->dev_at(e->off_slots), n, H,
                         D, bs, NB, c.dtype, stream);
    if (st != PA_OK) return st;
  }
  if (g_count > 0) {
    st = pa_decode_shared_prefix(a->out, a->query, e->key_cache, e->value_cache, e->dev_at(e->off_tables),
                                 e->dev_at(e->off_ctx), e->dev_at(e->off_starts), e->dev_at(e->off_prefix), n, H,
                                 D, bs, NB, mb, g_count, max_group, max_prefix, max_suffix, a->scale, c.dtype,
                                 0, 0, e->workspace, e->workspace_bytes, stream);
    if (st != PA_OK) return st;
    if (admitted_tokens > 0) {
      st = pa_cache_append(e->key_cache, e->value_cache, a->prompt_key, a->prompt_value, e->dev_at(e->off_admit),
                           static_cast<int32_t>(admitted_tokens), H, D, bs, NB, c.dtype, stream);
      if (st != PA_OK) return st;
    }
  } else {
    // the admitted prompts' rows are written by trailing workgroups of the decode launch
    st = pa::decode_with_rows(a->out, a->query, e->key_cache, e->value_cache, staged + e->off_tables,
                              staged + e->off_ctx, n, H, D, bs, NB, mb, max_ctx, a->scale, c.dtype, e->workspace,
                              e->workspace_bytes, &hints, a->prompt_key, a->prompt_value, staged + e->off_admit,
                              static_cast<int32_t>(admitted_tokens), direct ? a->new_key : nullptr,
                              direct ? a->new_value : nullptr, direct ? e->started_dev : nullptr, this_step,
                              stream);
    if (st != PA_OK) return st;
    if (direct) mark_used();
  }
  e->last_direct = direct;

  pa_step_result r{};
  r.num_copies = copies;
  r.num_admitted = admitted;
  r.admitted_tokens = static_cast<int32_t>(admitted_tokens);
  r.max_context_len = max_ctx;
  r.max_prefix_len = max_prefix;
  r.max_suffix_len = max_suffix;
  r.max_group_size = max_group;
  e->last = r;
  e->has_last = true;
  e->last_turn = t;
  e->last_n = n;
  e->last_groups = g_count;
  e->last_hints = hints;
  if (result) *result = r;
  return pa::clear_error();
}

pa_status pa_step_last(const pa_step_engine* e, pa_step_view* v) {
  if (!e || !v) return pa::set_error(PA_ERR_NULL, "engine and view must not be NULL");
  if (!e->has_last) return pa::set_error(PA_ERR_INVALID_ARG, "no step has run on this executor");
  const int32_t* h = e->host[e->last_turn];
  const bool grouped = e->last_groups > 0;
  v->num_seqs = e->last_n;
  v->num_groups = e->last_groups;
  v->result = e->last;
  v->slots = h + e->off_slots;
  v->positions = e->positions.data();
  v->copy_pairs = h + e->off_pairs;
  v->block_tables = h + e->off_tables;
  v->context_lens = h + e->off_ctx;
  v->group_starts = grouped ? h + e->off_starts : nullptr;
  v->prefix_lens = grouped ? h + e->off_prefix : nullptr;
  v->admit_slots = h + e->off_admit;
  const int32_t* dev = e->last_direct ? static_cast<const int32_t*>(e->host_dev[e->last_turn]) : e->dev;
  v->dev_block_tables = dev + e->off_tables;
  v->dev_context_lens = dev + e->off_ctx;
  v->dev_group_starts = grouped ? dev + e->off_starts : nullptr;
  v->dev_prefix_lens = grouped ? dev + e->off_prefix : nullptr;
  v->workspace = e->workspace;
  v->workspace_bytes = e->workspace_bytes;
  v->hints = e->last_hints;
  return pa::clear_error();
}

}  // extern "C"
