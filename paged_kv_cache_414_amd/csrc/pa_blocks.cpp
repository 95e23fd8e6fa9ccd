// Host-side block manager: free list, reference counts, block tables, slot mapping
// and the copy-on-write trigger.  The contract of every function is in
// include/pa_blocks.h; the page passages it follows are cited there.

#include "pa_blocks.h"

#include <climits>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa_status.h"

namespace {

struct Sequence {
  std::vector<int32_t> blocks;  // logical block i -> physical block
  int32_t length = 0;           // tokens
};

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): a 64-bit counter passed through a bijective mixer.
uint64_t splitmix64_next(uint64_t& state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Uniform integer in [0, n), n > 0: multiply-high with rejection of the biased low
// range (Lemire, "Fast random integer generation in an interval", TOMACS 2019).
uint32_t uniform_below(uint64_t& state, uint32_t n) {
  uint64_t m = (splitmix64_next(state) >> 32) * n;
  uint32_t low = static_cast<uint32_t>(m);
  if (low < n) {
    const uint32_t threshold = static_cast<uint32_t>(-n) % n;
    while (low < threshold) {
      m = (splitmix64_next(state) >> 32) * n;
      low = static_cast<uint32_t>(m);
    }
  }
  return static_cast<uint32_t>(m >> 32);
}

int32_t blocks_for(int64_t tokens, int32_t block_size) {
  return static_cast<int32_t>((tokens + block_size - 1) / block_size);
}

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  bool random_pick = false;
  uint64_t rng = 0;
  std::vector<int32_t> ref_count;
  std::vector<int32_t> free_list;  // the next block is taken from the back
  std::unordered_map<int64_t, Sequence> seqs;

  // Caller has checked that a block is free.
  int32_t take_block() {
    if (random_pick) {
      const uint32_t i = uniform_below(rng, static_cast<uint32_t>(free_list.size()));
      std::swap(free_list[i], free_list.back());
    }
    const int32_t b = free_list.back();
    free_list.pop_back();
    ref_count[b] = 1;
    return b;
  }

  void drop_ref(int32_t b) {
    if (--ref_count[b] == 0) free_list.push_back(b);
  }

  int32_t slot(const Sequence& s, int32_t pos) const {
    return s.blocks[pos / block_size] * block_size + pos % block_size;
  }
};

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, uint64_t seed) {
  if (num_blocks <= 0 || block_size <= 0) {
    pa::set_error(PA_ERR_INVALID_ARG, "num_blocks %d and block_size %d must be positive", num_blocks,
                  block_size);
    return nullptr;
  }
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) {
    pa::set_error(PA_ERR_INVALID_ARG, "num_blocks * block_size exceeds the int32 slot range");
    return nullptr;
  }
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (!bm) {
    pa::set_error(PA_ERR_INVALID_ARG, "out of host memory");
    return nullptr;
  }
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->random_pick = seed != 0;
  bm->rng = seed;
  bm->ref_count.assign(num_blocks, 0);
  bm->free_list.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) bm->free_list[i] = num_blocks - 1 - i;  // lowest id last
  pa::clear_error();
  return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_num_blocks(const pa_block_manager* bm) { return bm ? bm->num_blocks : -1; }

int32_t pa_bm_block_size(const pa_block_manager* bm) { return bm ? bm->block_size : -1; }

int32_t pa_bm_num_free(const pa_block_manager* bm) {
  return bm ? static_cast<int32_t>(bm->free_list.size()) : -1;
}

int32_t pa_bm_can_allocate(const pa_block_manager* bm, int32_t num_tokens) {
  if (!bm || num_tokens < 0) return 0;
  return blocks_for(num_tokens, bm->block_size) <= static_cast<int64_t>(bm->free_list.size()) ? 1 : 0;
}

pa_status pa_bm_ref_counts(const pa_block_manager* bm, int32_t* ref_counts) {
  if (!bm || !ref_counts) return pa::set_error(PA_ERR_NULL, "manager and ref_counts must not be NULL");
  for (int32_t b = 0; b < bm->num_blocks; ++b) ref_counts[b] = bm->ref_count[b];
  return pa::clear_error();
}

pa_status pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, int32_t num_tokens, int32_t* slots) {
  if (!bm) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  if (num_tokens < 0) return pa::set_error(PA_ERR_INVALID_ARG, "num_tokens %d is negative", num_tokens);
  if (bm->seqs.count(seq_id)) return pa::set_error(PA_ERR_INVALID_ARG, "sequence %lld exists", (long long)seq_id);
  const int32_t n_blk = blocks_for(num_tokens, bm->block_size);
  if (n_blk > static_cast<int64_t>(bm->free_list.size()))
    return pa::set_error(PA_ERR_OUT_OF_BLOCKS, "%d blocks needed, %zu free", n_blk, bm->free_list.size());
  Sequence& s = bm->seqs[seq_id];
  s.blocks.reserve(n_blk + 1);
  for (int32_t i = 0; i < n_blk; ++i) s.blocks.push_back(bm->take_block());
  s.length = num_tokens;
  if (slots) {
    for (int32_t p = 0; p < num_tokens; ++p) slots[p] = bm->slot(s, p);
  }
  return pa::clear_error();
}

pa_status pa_bm_add_sequences(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* num_tokens,
                              int32_t n, int32_t* slots) {
  if (!bm) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  if (n < 0) return pa::set_error(PA_ERR_INVALID_ARG, "n %d is negative", n);
  if (n > 0 && (!seq_ids || !num_tokens)) return pa::set_error(PA_ERR_NULL, "seq_ids and num_tokens must not be NULL");
  int64_t needed = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (num_tokens[i] < 0) return pa::set_error(PA_ERR_INVALID_ARG, "num_tokens[%d] = %d is negative", i, num_tokens[i]);
    if (bm->seqs.count(seq_ids[i])) return pa::set_error(PA_ERR_INVALID_ARG, "sequence %lld exists", (long long)seq_ids[i]);
    for (int32_t j = 0; j < i; ++j) {
      if (seq_ids[j] == seq_ids[i])
        return pa::set_error(PA_ERR_INVALID_ARG, "sequence %lld listed twice", (long long)seq_ids[i]);
    }
    needed += blocks_for(num_tokens[i], bm->block_size);
  }
  if (needed > static_cast<int64_t>(bm->free_list.size()))
    return pa::set_error(PA_ERR_OUT_OF_BLOCKS, "%lld blocks needed, %zu free", (long long)needed, bm->free_list.size());
  int64_t cursor = 0;
  for (int32_t i = 0; i < n; ++i) {
    pa_bm_add_sequence(bm, seq_ids[i], num_tokens[i], slots ? slots + cursor : nullptr);
    cursor += num_tokens[i];
  }
  return pa::clear_error();
}

pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end()) return pa::set_error(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)parent_id);
  if (bm->seqs.count(child_id)) return pa::set_error(PA_ERR_INVALID_ARG, "sequence %lld exists", (long long)child_id);
  Sequence child = it->second;  // copy before inserting (the map may rehash)
  for (int32_t b : child.blocks) ++bm->ref_count[b];
  bm->seqs.emplace(child_id, std::move(child));
  return pa::clear_error();
}

pa_status pa_bm_free(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pa::set_error(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq_id);
  for (int32_t b : it->second.blocks) bm->drop_ref(b);
  bm->seqs.erase(it);
  return pa::clear_error();
}

pa_status pa_bm_append_slots(pa_block_manager* bm, const int64_t* seq_ids, int32_t n, int32_t* slots,
                             int32_t* positions, int32_t* copy_pairs, int32_t* num_copies) {
  if (!bm) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  if (n < 0) return pa::set_error(PA_ERR_INVALID_ARG, "n %d is negative", n);
  if (n > 0 && (!seq_ids || !slots || !copy_pairs || !num_copies))
    return pa::set_error(PA_ERR_NULL, "seq_ids, slots, copy_pairs and num_copies must not be NULL");
  // First pass, nothing changed yet: look every sequence up and count the blocks
  // the list needs.  A token at a block boundary needs a new block.  Only the first
  // token of a sequence in this call can land in a block that others hold (after
  // that write its last block is private).  The w listed writers into a block with
  // r holders (w <= r) make min(w, r - 1) copies: each copy drops one holder and the
  // last remaining holder writes in place.
  std::vector<Sequence*> seq(n);
  std::unordered_map<Sequence*, int32_t> seen;   // tokens already counted in this call
  std::unordered_map<int32_t, int32_t> writers;  // shared last block -> listed writers
  int64_t needed = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return pa::set_error(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq_ids[i]);
    seq[i] = &it->second;
    const int32_t k = seen[seq[i]]++;
    const int32_t pos = seq[i]->length + k;
    if (pos % bm->block_size == 0) {
      ++needed;
    } else if (k == 0 && bm->ref_count[seq[i]->blocks.back()] > 1) {
      ++writers[seq[i]->blocks.back()];
    }
  }
  for (const auto& w : writers) {
    const int32_t r = bm->ref_count[w.first];
    needed += w.second < r - 1 ? w.second : r - 1;
  }
  if (needed > static_cast<int64_t>(bm->free_list.size()))
    return pa::set_error(PA_ERR_OUT_OF_BLOCKS, "%lld blocks needed, %zu free", (long long)needed,
                         bm->free_list.size());
  // Second pass: apply.
  int32_t copies = 0;
  for (int32_t i = 0; i < n; ++i) {
    Sequence& s = *seq[i];
    const int32_t pos = s.length;
    if (pos % bm->block_size == 0) {
      s.blocks.push_back(bm->take_block());
    } else {
      const int32_t last = s.blocks.back();
      if (bm->ref_count[last] > 1) {
        const int32_t fresh = bm->take_block();
        bm->drop_ref(last);
        s.blocks.back() = fresh;
        copy_pairs[2 * copies] = last;
        copy_pairs[2 * copies + 1] = fresh;
        ++copies;
      }
    }
    slots[i] = bm->slot(s, pos);
    if (positions) positions[i] = pos;
    s.length = pos + 1;
  }
  *num_copies = copies;
  return pa::clear_error();
}

pa_status pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                             int32_t pad, int32_t* tables) {
  if (!bm) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  if (n < 0 || max_blocks <= 0) return pa::set_error(PA_ERR_INVALID_ARG, "n %d >= 0 and max_blocks %d > 0 required", n, max_blocks);
  if (n > 0 && (!seq_ids || !tables)) return pa::set_error(PA_ERR_NULL, "seq_ids and tables must not be NULL");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return pa::set_error(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq_ids[i]);
    if (static_cast<int64_t>(it->second.blocks.size()) > max_blocks)
      return pa::set_error(PA_ERR_INVALID_ARG, "sequence %lld holds %zu > %d blocks", (long long)seq_ids[i],
                           it->second.blocks.size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>& blk = bm->seqs.find(seq_ids[i])->second.blocks;
    int32_t* row = tables + static_cast<int64_t>(i) * max_blocks;
    const int32_t nb = static_cast<int32_t>(blk.size());
    for (int32_t j = 0; j < nb; ++j) row[j] = blk[j];
    for (int32_t j = nb; j < max_blocks; ++j) row[j] = pad;
  }
  return pa::clear_error();
}

pa_status pa_bm_context_lens(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n, int32_t* context_lens) {
  if (!bm) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  if (n < 0) return pa::set_error(PA_ERR_INVALID_ARG, "n %d is negative", n);
  if (n > 0 && (!seq_ids || !context_lens)) return pa::set_error(PA_ERR_NULL, "seq_ids and context_lens must not be NULL");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return pa::set_error(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq_ids[i]);
    context_lens[i] = it->second.length;
  }
  return pa::clear_error();
}

int32_t pa_bm_shared_prefix_blocks(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n) {
  if (!bm || !seq_ids || n < 1) {
    pa::set_error(PA_ERR_INVALID_ARG, "manager, seq_ids and n >= 1 required");
    return -1;
  }
  std::vector<const Sequence*> seq(n);
  int32_t lead = INT32_MAX;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) {
      pa::set_error(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq_ids[i]);
      return -1;
    }
    seq[i] = &it->second;
    const int32_t whole = it->second.length / bm->block_size;
    if (whole < lead) lead = whole;
  }
  for (int32_t j = 0; j < lead; ++j) {
    const int32_t b = seq[0]->blocks[j];
    for (int32_t i = 1; i < n; ++i) {
      if (seq[i]->blocks[j] != b) {
        pa::clear_error();
        return j;
      }
    }
  }
  pa::clear_error();
  return lead;
}

int32_t pa_bm_num_seq_blocks(const pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? -1 : static_cast<int32_t>(it->second.blocks.size());
}

pa_status pa_bm_seq_blocks(const pa_block_manager* bm, int64_t seq_id, int32_t* blocks, int32_t cap) {
  if (!bm || (cap > 0 && !blocks)) return pa::set_error(PA_ERR_NULL, "manager and blocks must not be NULL");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pa::set_error(PA_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq_id);
  const std::vector<int32_t>& blk = it->second.blocks;
  for (int32_t j = 0; j < cap && j < static_cast<int32_t>(blk.size()); ++j) blocks[j] = blk[j];
  return pa::clear_error();
}

}  // extern "C"

namespace pa {

bool batch_shares_blocks(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n) {
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) continue;
    for (int32_t b : it->second.blocks)
      if (bm->ref_count[b] > 1) return true;
  }
  return false;
}

}  // namespace pa
