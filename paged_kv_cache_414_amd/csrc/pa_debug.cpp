// Host-side checks of the device data behind every entry point, compiled in builds
// with PA_DEBUG_CHECKS=1 (the contract of each check is in pa_debug.h).  The data is
// copied to the host after the stream has drained, so that arrays written by earlier
// work on the same stream (the executor's staged tables, for instance) are seen as
// the kernels would see them.

#include "pa_debug.h"

#if PA_DEBUG_CHECKS

#include <cstddef>
#include <unordered_map>
#include <unordered_set>
#include <utility>

#include "pa_status.h"

namespace pa {
namespace debug {

namespace {

// Wait for the work on `stream`, then copy n int32 from `src` (device or host memory).
pa_status fetch(std::vector<int32_t>* v, const int32_t* src, size_t n, hipStream_t stream) {
  v->assign(n, 0);
  if (n == 0) return PA_OK;
  hipError_t err = hipStreamSynchronize(stream);
  if (err == hipSuccess) err = hipMemcpy(v->data(), src, n * sizeof(int32_t), hipMemcpyDefault);
  if (err != hipSuccess)
    return set_error(PA_ERR_HIP, "device data check: reading the arrays failed: %s", hipGetErrorString(err));
  return PA_OK;
}

int32_t live_blocks(const DecodeView& v, int32_t s) { return (v.ctx[s] + v.BS - 1) / v.BS; }

}  // namespace

pa_status decode_data(DecodeView* v, const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_blocks, int32_t max_blocks_per_seq, int32_t block_size, int32_t max_context_len,
                      hipStream_t stream) {
  v->S = num_seqs;
  v->MB = max_blocks_per_seq;
  v->BS = block_size;
  pa_status st = fetch(&v->ctx, context_lens, static_cast<size_t>(num_seqs), stream);
  if (st == PA_OK)
    st = fetch(&v->bt, block_tables, static_cast<size_t>(num_seqs) * max_blocks_per_seq, stream);
  if (st != PA_OK) return st;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t c = v->ctx[s];
    if (c < 0 || c > max_context_len)
      return set_error(PA_ERR_INVALID_ARG, "device data: context_lens[%d] = %d is outside [0, max_context_len %d]",
                       s, c, max_context_len);
    for (int32_t i = 0; i < live_blocks(*v, s); ++i) {
      const int32_t id = v->bt[static_cast<size_t>(s) * max_blocks_per_seq + i];
      if (id < 0 || id >= num_blocks)
        return set_error(PA_ERR_INVALID_ARG, "device data: block_tables[%d][%d] = %d is outside [0, num_blocks %d)",
                         s, i, id, num_blocks);
    }
  }
  return PA_OK;
}

pa_status lengths(const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len, hipStream_t stream) {
  std::vector<int32_t> ctx;
  const pa_status st = fetch(&ctx, context_lens, static_cast<size_t>(num_seqs), stream);
  if (st != PA_OK) return st;
  for (int32_t s = 0; s < num_seqs; ++s)
    if (ctx[s] < 0 || ctx[s] > max_context_len)
      return set_error(PA_ERR_INVALID_ARG, "device data: context_lens[%d] = %d is outside [0, max_context_len %d]",
                       s, ctx[s], max_context_len);
  return PA_OK;
}

pa_status seq_order(const int32_t* order, int32_t num_seqs, hipStream_t stream) {
  if (!order) return PA_OK;
  std::vector<int32_t> o;
  const pa_status st = fetch(&o, order, static_cast<size_t>(num_seqs), stream);
  if (st != PA_OK) return st;
  std::vector<char> seen(static_cast<size_t>(num_seqs), 0);
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (o[i] < 0 || o[i] >= num_seqs || seen[o[i]])
      return set_error(PA_ERR_INVALID_ARG, "device data: seq_order is not a permutation of 0..%d (entry %d = %d)",
                       num_seqs - 1, i, o[i]);
    seen[o[i]] = 1;
  }
  return PA_OK;
}

pa_status new_rows(const DecodeView& v) {
  // the slot of each sequence's new row (position context_lens[s] - 1), or -1
  std::vector<int64_t> slot(static_cast<size_t>(v.S), -1);
  std::unordered_map<int64_t, int32_t> writer;  // slot -> sequence
  for (int32_t s = 0; s < v.S; ++s) {
    if (v.ctx[s] < 1) continue;
    const int32_t t = v.ctx[s] - 1;
    slot[s] = static_cast<int64_t>(v.bt[static_cast<size_t>(s) * v.MB + t / v.BS]) * v.BS + t % v.BS;
    const auto ins = writer.emplace(slot[s], s);
    if (!ins.second)
      return set_error(PA_ERR_INVALID_ARG, "device data: the new rows of sequences %d and %d go to one slot %lld",
                       ins.first->second, s, static_cast<long long>(slot[s]));
  }
  // every pool slot the decode reads from: (block, offset < tokens read from it)
  for (int32_t s = 0; s < v.S; ++s)
    for (int32_t i = 0; i < live_blocks(v, s); ++i) {
      const int32_t tokens = v.ctx[s] - i * v.BS < v.BS ? v.ctx[s] - i * v.BS : v.BS;
      const int64_t first = static_cast<int64_t>(v.bt[static_cast<size_t>(s) * v.MB + i]) * v.BS;
      const bool own_last = i == (v.ctx[s] - 1) / v.BS;  // its new row comes from new_key / new_value
      for (int32_t o = 0; o < tokens; ++o) {
        const auto w = writer.find(first + o);
        if (w == writer.end() || (own_last && w->second == s && o == tokens - 1)) continue;
        return set_error(PA_ERR_INVALID_ARG,
                         "device data: the new row of sequence %d goes to slot %lld, which sequence %d reads "
                         "(copy-on-write not done)",
                         w->second, static_cast<long long>(first + o), s);
      }
    }
  return PA_OK;
}

pa_status extra_rows(const DecodeView& v, const int32_t* slot_list, int32_t n, int32_t num_blocks,
                     hipStream_t stream) {
  std::vector<int32_t> sl;
  const pa_status st = fetch(&sl, slot_list, static_cast<size_t>(n), stream);
  if (st != PA_OK) return st;
  std::unordered_set<int32_t> read;
  for (int32_t s = 0; s < v.S; ++s)
    for (int32_t i = 0; i < live_blocks(v, s); ++i) read.insert(v.bt[static_cast<size_t>(s) * v.MB + i]);
  std::unordered_set<int32_t> seen;
  const int64_t limit = static_cast<int64_t>(num_blocks) * v.BS;
  for (int32_t i = 0; i < n; ++i) {
    if (sl[i] < 0) continue;
    if (sl[i] >= limit)
      return set_error(PA_ERR_INVALID_ARG, "device data: extra row %d has slot %d, past num_blocks * block_size %lld",
                       i, sl[i], static_cast<long long>(limit));
    if (!seen.insert(sl[i]).second)
      return set_error(PA_ERR_INVALID_ARG, "device data: extra rows share slot %d (row %d)", sl[i], i);
    if (read.count(sl[i] / v.BS))
      return set_error(PA_ERR_INVALID_ARG, "device data: extra row %d goes to block %d, which the decode reads", i,
                       sl[i] / v.BS);
  }
  return PA_OK;
}

pa_status slots(const int32_t* slot_mapping, int32_t n, int32_t num_blocks, int32_t block_size,
                hipStream_t stream) {
  std::vector<int32_t> sl;
  const pa_status st = fetch(&sl, slot_mapping, static_cast<size_t>(n), stream);
  if (st != PA_OK) return st;
  std::unordered_set<int32_t> seen;
  const int64_t limit = static_cast<int64_t>(num_blocks) * block_size;
  for (int32_t i = 0; i < n; ++i) {
    if (sl[i] < 0) continue;
    if (sl[i] >= limit)
      return set_error(PA_ERR_INVALID_ARG, "device data: slot_mapping[%d] = %d is past num_blocks * block_size %lld",
                       i, sl[i], static_cast<long long>(limit));
    if (!seen.insert(sl[i]).second)
      return set_error(PA_ERR_INVALID_ARG, "device data: slot %d appears twice in slot_mapping (entry %d)", sl[i], i);
  }
  return PA_OK;
}

pa_status pairs(const int32_t* block_pairs, int32_t n, int32_t src_blocks, int32_t dst_blocks, bool same_pool,
                hipStream_t stream) {
  std::vector<int32_t> p;
  const pa_status st = fetch(&p, block_pairs, 2 * static_cast<size_t>(n), stream);
  if (st != PA_OK) return st;
  std::unordered_set<int32_t> srcs, dsts;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = p[2 * i], d = p[2 * i + 1];
    if (s < 0 || s >= src_blocks)
      return set_error(PA_ERR_INVALID_ARG, "device data: pair %d has source block %d outside [0, %d)", i, s,
                       src_blocks);
    if (d < 0 || d >= dst_blocks)
      return set_error(PA_ERR_INVALID_ARG, "device data: pair %d has destination block %d outside [0, %d)", i, d,
                       dst_blocks);
    if (!dsts.insert(d).second)
      return set_error(PA_ERR_INVALID_ARG, "device data: destination block %d appears twice (pair %d)", d, i);
    srcs.insert(s);
  }
  if (same_pool)
    for (int32_t i = 0; i < n; ++i)
      if (srcs.count(p[2 * i + 1]))
        return set_error(PA_ERR_INVALID_ARG, "device data: block %d is both a source and a destination (pair %d)",
                         p[2 * i + 1], i);
  return PA_OK;
}

pa_status groups(const DecodeView& v, const int32_t* group_starts, const int32_t* prefix_lens, int32_t num_groups,
                 int32_t max_prefix_len, int32_t max_suffix_len, hipStream_t stream) {
  std::vector<int32_t> gs, pl;
  pa_status st = fetch(&pl, prefix_lens, static_cast<size_t>(v.S), stream);
  if (st == PA_OK && num_groups > 0) st = fetch(&gs, group_starts, static_cast<size_t>(num_groups) + 1, stream);
  if (st != PA_OK) return st;
  std::vector<int32_t> leader(static_cast<size_t>(v.S), -1);  // first sequence of s's group
  for (int32_t g = 0; g < num_groups; ++g) {
    if (gs[g] < 0 || gs[g] > gs[g + 1] || gs[g + 1] > v.S)
      return set_error(PA_ERR_INVALID_ARG,
                       "device data: group_starts[%d..%d] = %d, %d is not a non-decreasing range within [0, %d]", g,
                       g + 1, gs[g], gs[g + 1], v.S);
    for (int32_t s = gs[g]; s < gs[g + 1]; ++s) leader[s] = gs[g];
  }
  for (int32_t s = 0; s < v.S; ++s) {
    const int32_t p = pl[s];
    if (p < 0 || p % v.BS != 0 || p > v.ctx[s] || p > max_prefix_len)
      return set_error(PA_ERR_INVALID_ARG,
                       "device data: prefix_lens[%d] = %d is not a multiple of block_size %d within [0, min("
                       "context_lens %d, max_prefix_len %d)]",
                       s, p, v.BS, v.ctx[s], max_prefix_len);
    if (v.ctx[s] - p > max_suffix_len)
      return set_error(PA_ERR_INVALID_ARG,
                       "device data: sequence %d has %d tokens after its prefix, more than max_suffix_len %d", s,
                       v.ctx[s] - p, max_suffix_len);
    const int32_t l = leader[s];
    if (l < 0) {
      if (p != 0)
        return set_error(PA_ERR_INVALID_ARG, "device data: sequence %d is in no group but prefix_lens[%d] = %d", s,
                         s, p);
      continue;
    }
    if (p != pl[l])
      return set_error(PA_ERR_INVALID_ARG, "device data: prefix_lens[%d] = %d differs from its group's %d", s, p,
                       pl[l]);
    for (int32_t i = 0; i < p / v.BS; ++i)
      if (v.bt[static_cast<size_t>(s) * v.MB + i] != v.bt[static_cast<size_t>(l) * v.MB + i])
        return set_error(PA_ERR_INVALID_ARG,
                         "device data: block_tables[%d][%d] = %d differs from block_tables[%d][%d] = %d within the "
                         "shared prefix",
                         s, i, v.bt[static_cast<size_t>(s) * v.MB + i], l, i, v.bt[static_cast<size_t>(l) * v.MB + i]);
  }
  return PA_OK;
}

}  // namespace debug
}  // namespace pa

#endif  // PA_DEBUG_CHECKS
