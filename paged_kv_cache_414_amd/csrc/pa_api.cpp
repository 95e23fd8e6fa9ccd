// C ABI of the paged KV-cache decode path: argument checks, planning of the
// split-context pass, dispatch to the HIP kernels and error reporting.
// The contract of every entry point is documented in include/pa.h.

#include "pa.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "pa_debug.h"
#include "pa_launch.h"
#include "pa_status.h"

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

namespace pa {

pa_status set_error(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

pa_status clear_error() {
  g_last_error[0] = '\0';
  return PA_OK;
}

pa_status check_dtype_shape(pa_dtype dtype, int32_t head_dim, int32_t block_size) {
  if (dtype != PA_F32 && dtype != PA_F16)
    return set_error(PA_ERR_UNSUPPORTED, "dtype %d is not PA_F32 or PA_F16", (int)dtype);
  if (head_dim != 64 && head_dim != 80 && head_dim != 96 && head_dim != 128 && head_dim != 256)
    return set_error(PA_ERR_UNSUPPORTED, "head_dim %d is not built (64, 80, 96, 128, 256)", head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128 &&
      block_size != 256)
    return set_error(PA_ERR_UNSUPPORTED, "block_size %d is not built (8, 16, 32, 64, 128, 256)", block_size);
  return PA_OK;
}

}  // namespace pa

namespace {

using fail_fn = pa_status (*)(pa_status, const char*, ...);
constexpr fail_fn fail = pa::set_error;
pa_status ok() { return pa::clear_error(); }

pa_status from_hip(hipError_t err, const char* what) {
  if (err == hipSuccess) return ok();
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

// Builds with PA_DEBUG_CHECKS: the device data a decode launch will read (tables,
// context lengths, dispatch order), checked on the host; PA_OK otherwise.
pa_status debug_decode(pa::debug::DecodeView* view, const pa::DecodeParams& p, int32_t num_blocks,
                       int32_t block_size, int32_t max_context_len, hipStream_t stream) {
  const pa_status st = pa::debug::decode_data(view, p.block_tables, p.context_lens, p.num_seqs, num_blocks,
                                              p.max_blocks_per_seq, block_size, max_context_len, stream);
  if (st != PA_OK) return st;
  return pa::debug::seq_order(p.seq_order, p.num_seqs, stream);
}

// Library choice of the partition length: start from the whole longest context
// (one partition per sequence, no merge pass) and halve while the launch would hold
// fewer than kAutoMinUnits (sequence, head, partition) workgroups -- two per compute
// unit of a 256-CU MI355X -- as long as the half stays at or above
// kAutoMinPartitionTokens.  Measured on MI355X (fp16, 32 heads x 128): few long
// workgroups stream fastest as long as there are at least about two per CU; e.g. 64
// sequences of contexts up to 562 tokens: one partition 47.7 us, two 54.5 us; 8
// sequences of 16K-32K tokens: 512 workgroups 6.55 TB/s, 4096 workgroups 6.25 TB/s,
// 256 workgroups 6.52 TB/s, but 4 sequences at 128 workgroups only 5.55 TB/s.
constexpr int64_t kAutoMinUnits = 512;
#if PA_SHARED_FUSED
// Workgroups one 1-D launch of the shared-prefix passes may hold (its grid in work-items
// must fit 32 bits at 512 work-items per workgroup).
constexpr int64_t kMaxFusedWorkgroups = (int64_t{1} << 32) / 512 - 1;
#endif
constexpr int32_t kAutoMinPartitionTokens = 256;
constexpr int32_t kMaxGridYZ = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(pa_dtype dt) { return dt == PA_F16 ? 2 : 4; }

size_t ws_align(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

using pa::check_dtype_shape;

int32_t round_up(int64_t x, int32_t m) { return static_cast<int32_t>(((x + m - 1) / m) * m); }

// The address a kernel can use for `p`, or nullptr when `p` is neither device
// memory nor pinned host memory mapped into the GPU (pageable host memory, unknown
// addresses): such pointers are refused on the host, never handed to a kernel.
const void* device_visible(const void* p) {
  if (!p) return nullptr;
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeHost) return nullptr;
  return attr.devicePointer;
}

// Resolved partition length, or -1 with the last error set.
int32_t resolve_partition(int32_t num_seqs, int32_t num_heads, int32_t block_size,
                          int32_t max_context_len, int32_t partition_size) {
  if (block_size <= 0) {
    fail(PA_ERR_INVALID_ARG, "block_size %d must be positive", block_size);
    return -1;
  }
  if (max_context_len < 0) {
    fail(PA_ERR_INVALID_ARG, "max_context_len %d is negative", max_context_len);
    return -1;
  }
  if (partition_size < 0 || (partition_size > 0 && partition_size % block_size != 0)) {
    fail(PA_ERR_INVALID_ARG, "partition_size %d must be 0 or a positive multiple of block_size %d",
         partition_size, block_size);
    return -1;
  }
  if (partition_size > 0) return partition_size;
  const int64_t pairs = static_cast<int64_t>(num_seqs > 0 ? num_seqs : 1) * (num_heads > 0 ? num_heads : 1);
  const int32_t floor_p = round_up(kAutoMinPartitionTokens, block_size);
  int32_t P = round_up(max_context_len > 0 ? max_context_len : 1, block_size);
  while (P > floor_p) {
    const int64_t units = pairs * ((static_cast<int64_t>(max_context_len) + P - 1) / P);
    if (units >= kAutoMinUnits) break;
    const int32_t half = round_up(P / 2, block_size);
    if (half < floor_p) break;  // no short tail partitions below the floor
    P = half;
  }
  return P;
}

// Library choice of the decode workgroup: 16 wave64s rather than 8 when every wave
// still folds about two units of the partition (32 units or more: tokens one wave
// folds at once, the kernel's unit of work, computed below as the kernel does) and
// the launch holds at least 1024 workgroups.  Shorter work per workgroup evens out
// the end of a launch of many workgroups; with few workgroups, or short partitions,
// the wide groups leave waves idle.  Measured on MI355X (fp16, 32 heads x 128, GB/s,
// 8 / 16 waves): 96 x U[300, 2048] 6,401 / 6,563; 64 x U[1, 562] 6,024 / 6,139;
// 32 x U[1, 1024] 5,795 / 6,280; 64 x U[400, 700] 6,345 / 6,592; but 16 x
// U[4096, 8192] (512 workgroups) 6,424 / 6,185, 64 x U[100, 300] (19 units) 6,022 /
// 5,437 and 256 x U[1, 256] 6,375 / 4,875.
constexpr int32_t kWideMinUnits = 32;
constexpr int64_t kWideMinWorkgroups = 1024;


int32_t unit_tokens(pa_dtype dtype, int32_t head_dim, int32_t block_size) {
  const int32_t vec = dtype == PA_F16 ? 8 : 4;  // elements per 16-byte load
  int32_t lanes = 1;                            // lanes per token row: a power of two
  while (lanes < head_dim / vec) lanes *= 2;
  const int32_t rows_per_load = 64 / lanes;
  const int32_t most = rows_per_load * 8;       // at most 8 loads per unit
  return block_size < most ? block_size : most;
}

// `heads_per_unit` heads share a workgroup (pa::decode_heads_per_unit), so the launch
// holds num_seqs * num_heads / heads_per_unit * NP workgroups.
bool wide_workgroups(pa_dtype dtype, int32_t head_dim, int32_t block_size, int32_t P, int32_t num_seqs,
                     int32_t num_heads, int32_t NP) {
  const int32_t unit = unit_tokens(dtype, head_dim, block_size);
  const int64_t units = (static_cast<int64_t>(P) + unit - 1) / unit;
  const int32_t hu = pa::decode_heads_per_unit(dtype == PA_F16, head_dim, block_size, num_heads);
  const int64_t groups = static_cast<int64_t>(num_seqs) * (num_heads / hu) * NP;
  return units >= kWideMinUnits && groups >= kWideMinWorkgroups;
}

int32_t partitions_for(int32_t max_context_len, int32_t P) {
  const int64_t np = (static_cast<int64_t>(max_context_len) + P - 1) / P;
  return np < 1 ? 1 : static_cast<int32_t>(np);
}

size_t workspace_bytes_for(int32_t S, int32_t H, int32_t D, int32_t NP) {
  if (NP <= 1) return 0;
  const size_t states = static_cast<size_t>(S) * H * NP;
  return 2 * ws_align(states * 4) + ws_align(states * D * 4);
}

struct DecodePlan {
  pa::DecodeParams prm;
  int32_t NP;
};

pa_status plan_decode(DecodePlan* plan, void* out, const void* query, const void* key_cache,
                      const void* value_cache, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                      pa_dtype dtype, int32_t partition_size, void* workspace,
                      size_t workspace_bytes) {
  pa_status st = check_dtype_shape(dtype, head_dim, block_size);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG,
                "sizes must be positive (num_seqs %d >= 0, num_heads %d, num_blocks %d, max_blocks_per_seq %d)",
                num_seqs, num_heads, num_blocks, max_blocks_per_seq);
  if (num_seqs > kMaxGridYZ || num_heads > kMaxGridYZ)
    return fail(PA_ERR_INVALID_ARG, "num_seqs %d and num_heads %d must be <= %d", num_seqs, num_heads,
                kMaxGridYZ);
  if (max_context_len < 0 ||
      static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PA_ERR_INVALID_ARG, "max_context_len %d must be in [0, max_blocks_per_seq * block_size = %lld]",
                max_context_len, static_cast<long long>(max_blocks_per_seq) * block_size);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  const int32_t P = resolve_partition(num_seqs, num_heads, block_size, max_context_len, partition_size);
  if (P < 0) return PA_ERR_INVALID_ARG;
  const int32_t NP = partitions_for(max_context_len, P);
  plan->NP = NP;
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return fail(PA_ERR_NULL, "a required pointer is NULL (out, query, key_cache, value_cache, block_tables, context_lens)");
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_ERR_INVALID_ARG, "out, query and the caches must be 16-byte aligned");
  const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, NP);
  if (need > 0) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
    if (workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  pa::DecodeParams& p = plan->prm;
  p.out = out;
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  const size_t states = static_cast<size_t>(num_seqs) * num_heads * NP;
  char* ws = static_cast<char*>(workspace);
  p.ws_m = need ? reinterpret_cast<float*>(ws) : nullptr;
  p.ws_l = need ? reinterpret_cast<float*>(ws + ws_align(states * 4)) : nullptr;
  p.ws_o = need ? reinterpret_cast<float*>(ws + 2 * ws_align(states * 4)) : nullptr;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.token_begin = nullptr;
  p.partition_tokens = P;
  p.num_partitions = NP;
  p.slots_per_pair = NP;
  p.slot_offset = 0;
  p.prefix_partition_tokens = P;
  p.heads_per_unit = pa::decode_heads_per_unit(dtype == PA_F16, head_dim, block_size, num_heads);
  p.wide = wide_workgroups(dtype, head_dim, block_size, P, num_seqs, num_heads, NP) ? 1 : 0;
  p.scale = scale;
  return PA_OK;
}

// Caller hints on top of the library's plan: a dispatch order and a workgroup size.
pa_status apply_hints(DecodePlan* plan, const pa_decode_hints* hints) {
  if (!hints) return PA_OK;
  if (hints->waves != 0 && hints->waves != pa::kDecodeWavesNarrow && hints->waves != pa::kDecodeWavesWide)
    return fail(PA_ERR_INVALID_ARG, "hints->waves %d is not 0, %d or %d", hints->waves, pa::kDecodeWavesNarrow,
                pa::kDecodeWavesWide);
  if (hints->seq_order && (reinterpret_cast<uintptr_t>(hints->seq_order) & 3u) != 0)
    return fail(PA_ERR_INVALID_ARG, "hints->seq_order must be 4-byte aligned");
  if (hints->waves != 0) plan->prm.wide = hints->waves == pa::kDecodeWavesWide ? 1 : 0;
  plan->prm.seq_order = hints->seq_order;
  return PA_OK;
}

// Library choice of the prefix partition length (tokens of the shared prefix that
// one workgroup reads for a tile of 16 of a group's queries): the whole longest
// prefix, halved while fewer than kPrefixMinUnits (group, query tile, head,
// partition) workgroups -- one per compute unit -- would be launched, as long as the
// half stays at or above kPrefixMinTokens.  Measured on MI355X (8 groups x 32 heads,
// 1024 shared tokens): one partition per (group, head) beats 2, 4 and 8 (76.6,
// 79.3, 81, 93 us).
constexpr int64_t kPrefixMinUnits = 256;
constexpr int32_t kPrefixMinTokens = 64;
constexpr int32_t kPrefixTile = 16;  // tokens per matrix-core tile of the prefix pass,
                                     // and queries per query tile

// Query tiles (16 members each) launched per group: enough for the largest group,
// as given, or for the average group when max_group_size is 0; within the grid's
// z limit.  Groups with more tiles than this loop over the rest in the workgroup.
int32_t prefix_query_tiles(int32_t num_seqs, int32_t num_groups, int32_t max_group_size) {
  if (num_groups <= 0) return 1;
  const int64_t members = max_group_size > 0 ? max_group_size : (static_cast<int64_t>(num_seqs) + num_groups - 1) / num_groups;
  int64_t tiles = (members + kPrefixTile - 1) / kPrefixTile;
  if (tiles < 1) tiles = 1;
  const int64_t cap = kMaxGridYZ / num_groups;
  return static_cast<int32_t>(tiles < cap ? tiles : (cap > 0 ? cap : 1));
}

int32_t resolve_prefix_partition(int32_t num_groups, int32_t query_tiles, int32_t num_heads,
                                 int32_t block_size, int32_t max_prefix_len,
                                 int32_t prefix_partition_size) {
  const int32_t unit = block_size > kPrefixTile ? block_size : kPrefixTile;
  if (prefix_partition_size < 0 || (prefix_partition_size > 0 && prefix_partition_size % unit != 0)) {
    fail(PA_ERR_INVALID_ARG, "prefix_partition_size %d must be 0 or a positive multiple of %d",
         prefix_partition_size, unit);
    return -1;
  }
  if (prefix_partition_size > 0) return prefix_partition_size;
  const int64_t pairs = static_cast<int64_t>(num_groups > 0 ? num_groups : 1) * query_tiles *
                       (num_heads > 0 ? num_heads : 1);
  const int32_t floor_p = round_up(kPrefixMinTokens, unit);
  int32_t P = round_up(max_prefix_len > 0 ? max_prefix_len : 1, unit);
  while (P > floor_p) {
    const int64_t units = pairs * ((static_cast<int64_t>(max_prefix_len) + P - 1) / P);
    if (units >= kPrefixMinUnits) break;
    const int32_t half = round_up(P / 2, unit);
    if (half < floor_p) break;
    P = half;
  }
  return P;
}

struct SharedPlan {
  int32_t Pp, NPp;  // prefix pass
  int32_t QT;       // query tiles per group in the prefix pass's grid
  int32_t P, NPs;   // pass over the tokens after the prefix
  int32_t slots;    // NPp + NPs states per (sequence, head)
  size_t ws_bytes;
};

pa_status plan_shared(SharedPlan* plan, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_groups, int32_t max_group_size,
                      int32_t max_prefix_len, int32_t max_suffix_len, int32_t partition_size,
                      int32_t prefix_partition_size) {
  if (head_dim != 64 && head_dim != 80 && head_dim != 96 && head_dim != 128 && head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d is not built (64, 80, 96, 128, 256)", head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128 &&
      block_size != 256)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d is not built for the shared-prefix decode (8 to 256)",
                block_size);
  if (num_seqs < 0 || num_heads <= 0 || num_groups < 0)
    return fail(PA_ERR_INVALID_ARG, "num_seqs %d >= 0, num_heads %d > 0, num_groups %d >= 0 required",
                num_seqs, num_heads, num_groups);
  if (num_seqs > kMaxGridYZ || num_heads > kMaxGridYZ || num_groups > kMaxGridYZ)
    return fail(PA_ERR_INVALID_ARG, "num_seqs, num_heads and num_groups must be <= %d", kMaxGridYZ);
  if (max_prefix_len < 0 || max_prefix_len % block_size != 0)
    return fail(PA_ERR_INVALID_ARG, "max_prefix_len %d must be a non-negative multiple of block_size %d",
                max_prefix_len, block_size);
  if (max_suffix_len < 0) return fail(PA_ERR_INVALID_ARG, "max_suffix_len %d is negative", max_suffix_len);
  if (max_group_size < 0) return fail(PA_ERR_INVALID_ARG, "max_group_size %d is negative", max_group_size);
  const int32_t QT = prefix_query_tiles(num_seqs, num_groups, max_group_size);
  const int32_t Pp = resolve_prefix_partition(num_groups, QT, num_heads, block_size, max_prefix_len,
                                              prefix_partition_size);
  if (Pp < 0) return PA_ERR_INVALID_ARG;
  // The prefix pass reads whole 16-token tiles: with blocks of 8 tokens a prefix may end
  // half a tile past the last whole tile, and those 8 tokens join the pass after it.
  const int32_t suffix_cap = max_suffix_len + (block_size < kPrefixTile ? kPrefixTile - block_size : 0);
  const int32_t P = resolve_partition(num_seqs, num_heads, block_size, suffix_cap, partition_size);
  if (P < 0) return PA_ERR_INVALID_ARG;
  plan->Pp = Pp;
  plan->QT = QT;
  plan->NPp = max_prefix_len > 0 ? partitions_for(max_prefix_len, Pp) : 0;
  plan->P = P;
  plan->NPs = partitions_for(suffix_cap, P);
  plan->slots = plan->NPp + plan->NPs;
  const size_t states = static_cast<size_t>(num_seqs) * num_heads * plan->slots;
  plan->ws_bytes = num_seqs > 0 ? 2 * ws_align(states * 4) + ws_align(states * head_dim * 4) : 0;
  return PA_OK;
}

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

int32_t pa_debug_checks(void) { return PA_DEBUG_CHECKS; }

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
  }
  return "PA_ERR_UNKNOWN";
}

const char* pa_last_error(void) { return g_last_error; }

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t block_size,
                                 int32_t max_context_len, int32_t partition_size) {
  return resolve_partition(num_seqs, num_heads, block_size, max_context_len, partition_size);
}

int32_t pa_decode_num_partitions(int32_t num_seqs, int32_t num_heads, int32_t block_size,
                                 int32_t max_context_len, int32_t partition_size) {
  const int32_t P = resolve_partition(num_seqs, num_heads, block_size, max_context_len, partition_size);
  if (P < 0) return -1;
  return partitions_for(max_context_len, P);
}

int32_t pa_decode_waves(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size,
                        int32_t max_context_len, int32_t partition_size, pa_dtype dtype) {
  if (check_dtype_shape(dtype, head_dim, block_size) != PA_OK) return -1;
  if (num_seqs < 0 || num_heads <= 0) {
    fail(PA_ERR_INVALID_ARG, "num_seqs %d >= 0 and num_heads %d > 0 required", num_seqs, num_heads);
    return -1;
  }
  const int32_t P = resolve_partition(num_seqs, num_heads, block_size, max_context_len, partition_size);
  if (P < 0) return -1;
  const int32_t NP = partitions_for(max_context_len, P);
  ok();
  return wide_workgroups(dtype, head_dim, block_size, P, num_seqs, num_heads, NP) ? pa::kDecodeWavesWide
                                                                                : pa::kDecodeWavesNarrow;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_context_len,
                                 int32_t partition_size) {
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0) {
    fail(PA_ERR_INVALID_ARG, "num_seqs %d, num_heads %d, head_dim %d out of range", num_seqs, num_heads,
         head_dim);
    return 0;
  }
  const int32_t P = resolve_partition(num_seqs, num_heads, block_size, max_context_len, partition_size);
  if (P < 0) return 0;
  return workspace_bytes_for(num_seqs, num_heads, head_dim, partitions_for(max_context_len, P));
}

static pa_status decode_partitions_hinted(void* out, const void* query, const void* key_cache,
                                          const void* value_cache, const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                          int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                          int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                          pa_dtype dtype, int32_t partition_size, void* workspace,
                                          size_t workspace_bytes, const pa_decode_hints* hints, void* stream) {
  DecodePlan plan;
  pa_status st = plan_decode(&plan, out, query, key_cache, value_cache, block_tables, context_lens,
                             num_seqs, num_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                             max_context_len, scale, dtype, partition_size, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  st = apply_hints(&plan, hints);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return ok();
  pa::debug::DecodeView view;
  st = debug_decode(&view, plan.prm, num_blocks, block_size, max_context_len, static_cast<hipStream_t>(stream));
  if (st != PA_OK) return st;
  return from_hip(pa::launch_decode_partitions(plan.prm, dtype == PA_F16, head_dim, block_size,
                                               static_cast<hipStream_t>(stream)),
                  "decode partition pass launch");
}

pa_status pa_decode_partitions(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                               pa_dtype dtype, int32_t partition_size, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return decode_partitions_hinted(out, query, key_cache, value_cache, block_tables, context_lens, num_seqs,
                                  num_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                  max_context_len, scale, dtype, partition_size, workspace, workspace_bytes,
                                  nullptr, stream);
}

pa_status pa_decode_reduce(void* out, const void* workspace, size_t workspace_bytes,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_context_len,
                           pa_dtype dtype, int32_t partition_size, void* stream) {
  pa_status st = check_dtype_shape(dtype, head_dim, block_size);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_heads <= 0 || num_seqs > kMaxGridYZ || num_heads > kMaxGridYZ)
    return fail(PA_ERR_INVALID_ARG, "num_seqs %d / num_heads %d out of range", num_seqs, num_heads);
  const int32_t P = resolve_partition(num_seqs, num_heads, block_size, max_context_len, partition_size);
  if (P < 0) return PA_ERR_INVALID_ARG;
  const int32_t NP = partitions_for(max_context_len, P);
  if (num_seqs == 0 || NP <= 1) return ok();  // nothing to merge
  if (!out || !workspace || !context_lens)
    return fail(PA_ERR_NULL, "out, workspace and context_lens must not be NULL");
  const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, NP);
  if (workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  if (!aligned16(out) || !aligned16(workspace))
    return fail(PA_ERR_INVALID_ARG, "out and workspace must be 16-byte aligned");
  st = pa::debug::lengths(context_lens, num_seqs, max_context_len, static_cast<hipStream_t>(stream));
  if (st != PA_OK) return st;
  const size_t states = static_cast<size_t>(num_seqs) * num_heads * NP;
  const char* ws = static_cast<const char*>(workspace);
  pa::ReduceParams prm;
  prm.out = out;
  prm.ws_m = reinterpret_cast<const float*>(ws);
  prm.ws_l = reinterpret_cast<const float*>(ws + ws_align(states * 4));
  prm.ws_o = reinterpret_cast<const float*>(ws + 2 * ws_align(states * 4));
  prm.context_lens = context_lens;
  prm.prefix_lens = nullptr;
  prm.num_seqs = num_seqs;
  prm.num_heads = num_heads;
  prm.partition_tokens = P;
  prm.prefix_partition_tokens = P;
  prm.prefix_slots = 0;
  prm.slots_per_pair = NP;
  return from_hip(pa::launch_decode_reduce(prm, dtype == PA_F16, head_dim, static_cast<hipStream_t>(stream)),
                  "decode reduce pass launch");
}

pa_status pa_decode_ex(void* out, const void* query, const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                       int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
                       int32_t partition_size, void* workspace, size_t workspace_bytes,
                       const pa_decode_hints* hints, void* stream) {
  pa_status st = decode_partitions_hinted(out, query, key_cache, value_cache, block_tables, context_lens,
                                          num_seqs, num_heads, head_dim, block_size, num_blocks,
                                          max_blocks_per_seq, max_context_len, scale, dtype, partition_size,
                                          workspace, workspace_bytes, hints, stream);
  if (st != PA_OK) return st;
  return pa_decode_reduce(out, workspace, workspace_bytes, context_lens, num_seqs, num_heads, head_dim,
                          block_size, max_context_len, dtype, partition_size, stream);
}

pa_status pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                    int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
                    int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  return pa_decode_ex(out, query, key_cache, value_cache, block_tables, context_lens, num_seqs, num_heads,
                      head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                      partition_size, workspace, workspace_bytes, nullptr, stream);
}

pa_status pa_decode_append_ex(void* out, const void* query, void* key_cache, void* value_cache,
                              const void* new_key, const void* new_value, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
                              int32_t partition_size, void* workspace, size_t workspace_bytes,
                              const pa_decode_hints* hints, void* stream) {
  DecodePlan plan;
  pa_status st = plan_decode(&plan, out, query, key_cache, value_cache, block_tables, context_lens,
                             num_seqs, num_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                             max_context_len, scale, dtype, partition_size, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  st = apply_hints(&plan, hints);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return ok();
  if (!new_key || !new_value) return fail(PA_ERR_NULL, "new_key and new_value must not be NULL");
  if (!aligned16(new_key) || !aligned16(new_value))
    return fail(PA_ERR_INVALID_ARG, "new_key and new_value must be 16-byte aligned");
  plan.prm.new_key = new_key;
  plan.prm.new_value = new_value;
  if (static_cast<int64_t>(num_seqs) + pa::store_slices(plan.prm) > kMaxGridYZ)  // store workgroups
    return fail(PA_ERR_INVALID_ARG, "num_seqs %d leaves no room for the store workgroups (grid z <= %d)",
                num_seqs, kMaxGridYZ);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  pa::debug::DecodeView view;
  st = debug_decode(&view, plan.prm, num_blocks, block_size, max_context_len, hs);
  if (st == PA_OK) st = pa::debug::new_rows(view);
  if (st != PA_OK) return st;
  st = from_hip(pa::launch_decode_partitions(plan.prm, dtype == PA_F16, head_dim, block_size, hs),
                "decode partition pass launch");
  if (st != PA_OK) return st;
  return pa_decode_reduce(out, workspace, workspace_bytes, context_lens, num_seqs, num_heads, head_dim,
                          block_size, max_context_len, dtype, partition_size, stream);
}

pa_status pa_decode_append(void* out, const void* query, void* key_cache, void* value_cache,
                           const void* new_key, const void* new_value, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
                           int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  return pa_decode_append_ex(out, query, key_cache, value_cache, new_key, new_value, block_tables, context_lens,
                             num_seqs, num_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                             max_context_len, scale, dtype, partition_size, workspace, workspace_bytes, nullptr,
                             stream);
}

}  // extern "C"

namespace pa {

pa_status decode_with_rows(void* out, const void* query, void* key_cache, void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
                           void* workspace, size_t workspace_bytes, const pa_decode_hints* hints,
                           const void* extra_key, const void* extra_value, const int32_t* extra_slots,
                           int32_t extra_tokens, const void* new_key, const void* new_value,
                           int32_t* started_flag, int32_t step, void* stream) {
  DecodePlan plan;
  pa_status st = plan_decode(&plan, out, query, key_cache, value_cache, block_tables, context_lens, num_seqs,
                             num_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                             scale, dtype, 0, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  st = apply_hints(&plan, hints);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return ok();
  if (!new_key != !new_value) return fail(PA_ERR_NULL, "new_key and new_value go together");
  if (new_key) {
    if (!aligned16(new_key) || !aligned16(new_value))
      return fail(PA_ERR_INVALID_ARG, "new_key and new_value must be 16-byte aligned");
    plan.prm.new_key = new_key;
    plan.prm.new_value = new_value;
  }
  plan.prm.started_flag = started_flag;
  plan.prm.step = step;
  if (extra_tokens < 0) return fail(PA_ERR_INVALID_ARG, "extra_tokens %d is negative", extra_tokens);
  if (extra_tokens > 0) {
    if (!extra_key || !extra_value || !extra_slots)
      return fail(PA_ERR_NULL, "extra rows and their slots must not be NULL");
    if (!aligned16(extra_key) || !aligned16(extra_value))
      return fail(PA_ERR_INVALID_ARG, "extra rows must be 16-byte aligned");
    if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
      return fail(PA_ERR_INVALID_ARG, "num_blocks * block_size exceeds the int32 slot range");
    // rows per workgroup: as many as its threads move in one round of loads and stores
    // (many small workgroups fill the end of the decode launch; a workgroup looping
    // over rounds would leave a tail of its own)
    const int64_t row_chunks = static_cast<int64_t>(num_heads) * (head_dim * static_cast<int64_t>(elem_bytes(dtype)) / 16);
    const int64_t threads = 64 * static_cast<int64_t>(plan.prm.wide ? pa::kDecodeWavesWide : pa::kDecodeWavesNarrow);
    int64_t per_group = threads * pa::kExtraChunksPerThread / row_chunks;
    if (per_group < 1) per_group = 1;
    if (per_group * row_chunks > INT32_MAX)
      return fail(PA_ERR_INVALID_ARG, "num_heads * head_dim too large for the extra rows");
    plan.prm.extra_key = extra_key;
    plan.prm.extra_value = extra_value;
    plan.prm.extra_slots = extra_slots;
    plan.prm.extra_tokens = extra_tokens;
    plan.prm.extra_per_group = static_cast<int32_t>(per_group);
  }
  if (static_cast<int64_t>(num_seqs) + pa::store_slices(plan.prm) + pa::extra_slices(plan.prm) > kMaxGridYZ)
    return fail(PA_ERR_INVALID_ARG, "%d extra rows and the new rows do not fit the grid after %d sequences",
                extra_tokens, num_seqs);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  pa::debug::DecodeView view;
  st = debug_decode(&view, plan.prm, num_blocks, block_size, max_context_len, hs);
  if (st == PA_OK && new_key) st = pa::debug::new_rows(view);
  if (st == PA_OK && extra_tokens > 0) st = pa::debug::extra_rows(view, extra_slots, extra_tokens, num_blocks, hs);
  if (st != PA_OK) return st;
  st = from_hip(pa::launch_decode_partitions(plan.prm, dtype == PA_F16, head_dim, block_size, hs),
                "decode partition pass launch");
  if (st != PA_OK) return st;
  return pa_decode_reduce(out, workspace, workspace_bytes, context_lens, num_seqs, num_heads, head_dim, block_size,
                          max_context_len, dtype, 0, stream);
}

}  // namespace pa

extern "C" {

pa_status pa_cache_append(void* key_cache, void* value_cache, const void* key, const void* value,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                          void* stream) {
  pa_status st = check_dtype_shape(dtype, head_dim, block_size);
  if (st != PA_OK) return st;
  if (num_tokens < 0 || num_heads <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_tokens %d >= 0, num_heads %d > 0, num_blocks %d > 0 required",
                num_tokens, num_heads, num_blocks);
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_blocks * block_size exceeds the int32 slot range");
  const int32_t row_bytes = head_dim * static_cast<int32_t>(elem_bytes(dtype));
  if (static_cast<int64_t>(num_heads) * (row_bytes / 16) > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_heads * head_dim too large for one launch");
  if (num_tokens == 0) return ok();
  if (!key_cache || !value_cache || !key || !value || !slot_mapping)
    return fail(PA_ERR_NULL, "a required pointer is NULL (key_cache, value_cache, key, value, slot_mapping)");
  if (!aligned16(key_cache) || !aligned16(value_cache) || !aligned16(key) || !aligned16(value))
    return fail(PA_ERR_INVALID_ARG, "caches and key/value rows must be 16-byte aligned");
  pa::AppendParams prm;
  prm.key_cache = key_cache;
  prm.value_cache = value_cache;
  prm.key = key;
  prm.value = value;
  prm.slot_mapping = slot_mapping;
  prm.num_tokens = num_tokens;
  prm.num_heads = num_heads;
  prm.block_size = block_size;
  prm.row_bytes = row_bytes;
  st = pa::debug::slots(slot_mapping, num_tokens, num_blocks, block_size, static_cast<hipStream_t>(stream));
  if (st != PA_OK) return st;
  return from_hip(pa::launch_cache_append(prm, static_cast<hipStream_t>(stream)), "cache append launch");
}

pa_status pa_block_copy(void* key_cache, void* value_cache, const int32_t* block_pairs, int32_t num_pairs,
                        int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                        pa_dtype dtype, void* stream) {
  pa_status st = check_dtype_shape(dtype, head_dim, block_size);
  if (st != PA_OK) return st;
  if (num_pairs < 0 || num_heads <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_pairs %d >= 0, num_heads %d > 0, num_blocks %d > 0 required",
                num_pairs, num_heads, num_blocks);
  if (num_pairs == 0) return ok();
  if (!key_cache || !value_cache || !block_pairs)
    return fail(PA_ERR_NULL, "a required pointer is NULL (key_cache, value_cache, block_pairs)");
  if (!aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_ERR_INVALID_ARG, "caches must be 16-byte aligned");
  pa::CopyParams prm;
  prm.src_key = key_cache;
  prm.src_value = value_cache;
  prm.dst_key = key_cache;
  prm.dst_value = value_cache;
  prm.block_pairs = block_pairs;
  prm.num_pairs = num_pairs;
  prm.block_bytes = static_cast<int64_t>(num_heads) * block_size * head_dim * static_cast<int64_t>(elem_bytes(dtype));
  st = pa::debug::pairs(block_pairs, num_pairs, num_blocks, num_blocks, true, static_cast<hipStream_t>(stream));
  if (st != PA_OK) return st;
  return from_hip(pa::launch_block_copy(prm, static_cast<hipStream_t>(stream)), "block copy launch");
}

pa_status pa_swap_blocks(void* dst_key, void* dst_value, const void* src_key, const void* src_value,
                         const int32_t* block_pairs, int32_t num_pairs, int32_t num_heads, int32_t head_dim,
                         int32_t block_size, int32_t src_num_blocks, int32_t dst_num_blocks, pa_dtype dtype,
                         void* stream) {
  pa_status st = check_dtype_shape(dtype, head_dim, block_size);
  if (st != PA_OK) return st;
  if (num_pairs < 0 || num_heads <= 0 || src_num_blocks <= 0 || dst_num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_pairs %d >= 0, num_heads %d > 0 and pool sizes %d, %d > 0 required",
                num_pairs, num_heads, src_num_blocks, dst_num_blocks);
  if (num_pairs == 0) return ok();
  if (!dst_key || !dst_value || !src_key || !src_value || !block_pairs)
    return fail(PA_ERR_NULL, "a required pointer is NULL (dst_key, dst_value, src_key, src_value, block_pairs)");
  if (!aligned16(dst_key) || !aligned16(dst_value) || !aligned16(src_key) || !aligned16(src_value))
    return fail(PA_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  const void* ptrs[5] = {dst_key, dst_value, src_key, src_value, block_pairs};
  const void* dev[5];
  static const char* const names[5] = {"dst_key", "dst_value", "src_key", "src_value", "block_pairs"};
  for (int i = 0; i < 5; ++i) {
    dev[i] = device_visible(ptrs[i]);
    if (!dev[i])
      return fail(PA_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", names[i]);
  }
  pa::CopyParams prm;
  prm.dst_key = const_cast<void*>(dev[0]);
  prm.dst_value = const_cast<void*>(dev[1]);
  prm.src_key = dev[2];
  prm.src_value = dev[3];
  prm.block_pairs = static_cast<const int32_t*>(dev[4]);
  prm.num_pairs = num_pairs;
  prm.block_bytes = static_cast<int64_t>(num_heads) * block_size * head_dim * static_cast<int64_t>(elem_bytes(dtype));
  st = pa::debug::pairs(block_pairs, num_pairs, src_num_blocks, dst_num_blocks, false,
                        static_cast<hipStream_t>(stream));
  if (st != PA_OK) return st;
  return from_hip(pa::launch_block_copy(prm, static_cast<hipStream_t>(stream)), "block swap launch");
}

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                               int32_t block_size, int32_t num_groups,
                                               int32_t max_group_size, int32_t max_prefix_len,
                                               int32_t max_suffix_len, int32_t partition_size,
                                               int32_t prefix_partition_size) {
  SharedPlan plan;
  if (plan_shared(&plan, num_seqs, num_heads, head_dim, block_size, num_groups, max_group_size,
                  max_prefix_len, max_suffix_len, partition_size, prefix_partition_size) != PA_OK)
    return 0;
  return plan.ws_bytes;
}

pa_status pa_decode_shared_prefix(void* out, const void* query, const void* key_cache,
                                  const void* value_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* group_starts,
                                  const int32_t* prefix_lens, int32_t num_seqs, int32_t num_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t num_groups,
                                  int32_t max_group_size, int32_t max_prefix_len,
                                  int32_t max_suffix_len, float scale, pa_dtype dtype,
                                  int32_t partition_size, int32_t prefix_partition_size,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "the shared-prefix decode is built for PA_F16 only (dtype %d)", (int)dtype);
  SharedPlan plan;
  pa_status st = plan_shared(&plan, num_seqs, num_heads, head_dim, block_size, num_groups, max_group_size,
                             max_prefix_len, max_suffix_len, partition_size, prefix_partition_size);
  if (st != PA_OK) return st;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_blocks %d and max_blocks_per_seq %d must be positive", num_blocks,
                max_blocks_per_seq);
  const int64_t row_tokens = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  if (max_prefix_len > row_tokens || max_suffix_len > row_tokens)
    return fail(PA_ERR_INVALID_ARG, "max_prefix_len %d and max_suffix_len %d must be <= max_blocks_per_seq * block_size = %lld",
                max_prefix_len, max_suffix_len, static_cast<long long>(row_tokens));
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  if (num_seqs == 0) return ok();
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens || !prefix_lens ||
      (num_groups > 0 && !group_starts))
    return fail(PA_ERR_NULL, "a required pointer is NULL (out, query, key_cache, value_cache, block_tables, "
                             "context_lens, prefix_lens, group_starts)");
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_ERR_INVALID_ARG, "out, query and the caches must be 16-byte aligned");
  if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", plan.ws_bytes);
  if (workspace_bytes < plan.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, plan.ws_bytes);
  if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  const size_t states = static_cast<size_t>(num_seqs) * num_heads * plan.slots;
  char* ws = static_cast<char*>(workspace);
  float* ws_m = reinterpret_cast<float*>(ws);
  float* ws_l = reinterpret_cast<float*>(ws + ws_align(states * 4));
  float* ws_o = reinterpret_cast<float*>(ws + 2 * ws_align(states * 4));
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  {
    pa::debug::DecodeView view;
    st = pa::debug::decode_data(&view, block_tables, context_lens, num_seqs, num_blocks, max_blocks_per_seq,
                                block_size, static_cast<int32_t>(row_tokens), hs);
    if (st == PA_OK)
      st = pa::debug::groups(view, group_starts, prefix_lens, num_groups, max_prefix_len, max_suffix_len, hs);
    if (st != PA_OK) return st;
  }

  const bool prefix_pass = num_groups > 0 && plan.NPp > 0;
  pa::PrefixParams pp;
  pp.query = query;
  pp.key_cache = key_cache;
  pp.value_cache = value_cache;
  pp.block_tables = block_tables;
  pp.group_starts = group_starts;
  pp.prefix_lens = prefix_lens;
  pp.ws_m = ws_m;
  pp.ws_l = ws_l;
  pp.ws_o = ws_o;
  pp.num_heads = num_heads;
  pp.max_blocks_per_seq = max_blocks_per_seq;
  pp.partition_tokens = plan.Pp;
  pp.num_partitions = plan.NPp;
  pp.num_groups = num_groups;
  pp.query_tiles = plan.QT;
  pp.slots_per_pair = plan.slots;
  pp.scale = scale;

  pa::DecodeParams dp;
  dp.out = out;
  dp.query = query;
  dp.key_cache = key_cache;
  dp.value_cache = value_cache;
  dp.block_tables = block_tables;
  dp.context_lens = context_lens;
  dp.token_begin = prefix_lens;
  dp.ws_m = ws_m;
  dp.ws_l = ws_l;
  dp.ws_o = ws_o;
  dp.num_seqs = num_seqs;
  dp.num_heads = num_heads;
  dp.max_blocks_per_seq = max_blocks_per_seq;
  dp.partition_tokens = plan.P;
  dp.num_partitions = plan.NPs;
  dp.slots_per_pair = plan.slots;
  dp.slot_offset = plan.NPp;
  dp.prefix_partition_tokens = plan.Pp;
  dp.heads_per_unit = pa::decode_heads_per_unit(true, head_dim, block_size, num_heads);
  dp.wide = wide_workgroups(PA_F16, head_dim, block_size, plan.P, num_seqs, num_heads, plan.NPs) ? 1 : 0;
  dp.scale = scale;

  pa::ReduceParams rp;
  rp.out = out;
  rp.ws_m = ws_m;
  rp.ws_l = ws_l;
  rp.ws_o = ws_o;
  rp.context_lens = context_lens;
  rp.prefix_lens = prefix_lens;
  rp.num_seqs = num_seqs;
  rp.num_heads = num_heads;
  rp.partition_tokens = plan.P;
  rp.prefix_partition_tokens = plan.Pp;
  rp.prefix_slots = plan.NPp;
  rp.slots_per_pair = plan.slots;

#if PA_SHARED_FUSED
  if (prefix_pass) {
    // both passes in one launch (8-wave workgroups), every state to the workspace,
    // then the merge of every (sequence, head)
    const int64_t groups = static_cast<int64_t>(plan.NPp) * num_heads * num_groups * plan.QT +
                           static_cast<int64_t>(plan.NPs) * num_heads * num_seqs;
    if (groups > kMaxFusedWorkgroups)
      return fail(PA_ERR_INVALID_ARG, "%lld workgroups exceed one launch (%lld)", static_cast<long long>(groups),
                  static_cast<long long>(kMaxFusedWorkgroups));
    dp.states_only = 1;
    dp.wide = 0;
    dp.heads_per_unit = 1;
    st = from_hip(pa::launch_decode_shared_fused(pp, dp, head_dim, block_size, hs), "shared-prefix passes launch");
    if (st != PA_OK) return st;
    rp.merge_all = 1;
    return from_hip(pa::launch_decode_reduce(rp, true, head_dim, hs), "shared-prefix merge launch");
  }
#endif
  if (prefix_pass) {
    st = from_hip(pa::launch_decode_prefix(pp, head_dim, block_size, hs), "shared-prefix pass launch");
    if (st != PA_OK) return st;
  }
  st = from_hip(pa::launch_decode_partitions(dp, true, head_dim, block_size, hs), "suffix pass launch");
  if (st != PA_OK) return st;
  // sequences whose tokens after the prefix fit one partition are finished above
  if (plan.NPs <= 1) return ok();
  return from_hip(pa::launch_decode_reduce(rp, true, head_dim, hs), "shared-prefix merge launch");
}

}  // extern "C\"
