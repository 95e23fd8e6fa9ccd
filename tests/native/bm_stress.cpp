// Host-only stress driver for the block manager (csrc/pa_blocks.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_blocks_sanitized.py.
// Random admissions (single and batched), forks, appends with copy-on-write and
// frees, plus every error path; after each operation the reference counts must equal
// the number of tables holding each block and free + held blocks must cover the pool.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <vector>

#include "pa_blocks.h"
#include "pa_status.h"

// The library's last-error text lives in pa_api.cpp, which needs the HIP runtime;
// this host-only build provides its own.
namespace pa {
static char g_text[512];
pa_status set_error(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_text, sizeof(g_text), fmt, ap);
  va_end(ap);
  return st;
}
pa_status clear_error() {
  g_text[0] = '\0';
  return PA_OK;
}
}  // namespace pa

static uint64_t rng_state = 12345;
static uint32_t next_u32() {
  rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
  return static_cast<uint32_t>(rng_state >> 33);
}

#define REQUIRE(cond)                                                     \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
      return 1;                                                           \
    }                                                                     \
  } while (0)

int main() {
  const int32_t nb = 80, bs = 8;
  pa_block_manager* bm = pa_bm_create(nb, bs, 99);
  REQUIRE(bm);
  REQUIRE(pa_bm_create(0, 8, 1) == nullptr);
  std::map<int64_t, int32_t> len;
  int64_t next_id = 0;
  std::vector<int32_t> slots(4096), pairs(4096), pos(4096), rc(nb), tables(64 * 64), blk(64);
  int32_t ncopy = 0;
  for (int it = 0; it < 20000; ++it) {
    const uint32_t op = next_u32() % 6;
    if (op == 0 || len.empty()) {
      const int32_t n = static_cast<int32_t>(next_u32() % 40);
      const pa_status st = pa_bm_add_sequence(bm, next_id, n, slots.data());
      if (st == PA_OK) len[next_id] = n;
      else REQUIRE(st == PA_ERR_OUT_OF_BLOCKS);
      ++next_id;
    } else if (op == 1) {
      int64_t ids[3] = {next_id, next_id + 1, next_id + 2};
      int32_t ns[3] = {static_cast<int32_t>(next_u32() % 20), 0, static_cast<int32_t>(next_u32() % 20)};
      const pa_status st = pa_bm_add_sequences(bm, ids, ns, 3, slots.data());
      if (st == PA_OK) {
        for (int i = 0; i < 3; ++i) len[ids[i]] = ns[i];
      } else {
        REQUIRE(st == PA_ERR_OUT_OF_BLOCKS);
      }
      next_id += 3;
    } else if (op == 2) {
      auto p = len.begin();
      std::advance(p, next_u32() % len.size());
      REQUIRE(pa_bm_fork(bm, p->first, next_id) == PA_OK);
      len[next_id++] = p->second;
    } else if (op == 3) {
      std::vector<int64_t> ids;
      const int k = 1 + static_cast<int>(next_u32() % 6);
      for (int i = 0; i < k; ++i) {
        auto p = len.begin();
        std::advance(p, next_u32() % len.size());
        ids.push_back(p->first);
      }
      const pa_status st = pa_bm_append_slots(bm, ids.data(), k, slots.data(), pos.data(), pairs.data(), &ncopy);
      if (st == PA_OK) {
        for (int64_t id : ids) ++len[id];
      } else {
        REQUIRE(st == PA_ERR_OUT_OF_BLOCKS);
      }
    } else if (op == 4) {
      auto p = len.begin();
      std::advance(p, next_u32() % len.size());
      REQUIRE(pa_bm_free(bm, p->first) == PA_OK);
      len.erase(p);
    } else {
      // error paths must fail cleanly and change nothing
      REQUIRE(pa_bm_free(bm, -7) == PA_ERR_INVALID_ARG);
      REQUIRE(pa_bm_fork(bm, -7, -8) == PA_ERR_INVALID_ARG);
      REQUIRE(pa_bm_add_sequence(bm, 0, -1, nullptr) == PA_ERR_INVALID_ARG);
      int64_t bad = -9;
      REQUIRE(pa_bm_context_lens(bm, &bad, 1, pos.data()) == PA_ERR_INVALID_ARG);
      REQUIRE(pa_bm_shared_prefix_blocks(bm, &bad, 1) == -1);
      REQUIRE(pa_bm_append_slots(bm, &bad, 1, slots.data(), pos.data(), pairs.data(), &ncopy) == PA_ERR_INVALID_ARG);
    }
    // invariants
    REQUIRE(pa_bm_ref_counts(bm, rc.data()) == PA_OK);
    std::vector<int32_t> holders(nb, 0);
    for (const auto& kv : len) {
      const int32_t n = pa_bm_num_seq_blocks(bm, kv.first);
      REQUIRE(n == (kv.second + bs - 1) / bs);
      REQUIRE(pa_bm_seq_blocks(bm, kv.first, blk.data(), 64) == PA_OK);
      for (int32_t j = 0; j < n && j < 64; ++j) ++holders[blk[j]];
      int32_t c = -1;
      REQUIRE(pa_bm_context_lens(bm, &kv.first, 1, &c) == PA_OK && c == kv.second);
    }
    int32_t held = 0;
    for (int32_t b = 0; b < nb; ++b) {
      REQUIRE(rc[b] == holders[b]);
      held += holders[b] > 0;
    }
    REQUIRE(pa_bm_num_free(bm) + held == nb);
    if (!len.empty() && len.size() <= 64) {
      std::vector<int64_t> ids;
      for (const auto& kv : len) ids.push_back(kv.first);
      REQUIRE(pa_bm_block_tables(bm, ids.data(), static_cast<int32_t>(ids.size()), 64, -1, tables.data()) == PA_OK);
      REQUIRE(pa_bm_shared_prefix_blocks(bm, ids.data(), static_cast<int32_t>(ids.size())) >= 0);
    }
  }
  pa_bm_destroy(bm);
  std::printf("bm_stress ok: %lld sequences created\n", static_cast<long long>(next_id));
  return 0;
}
