// Host stress test of the C++ block manager, built by
// tests/test_block_manager_sanitized.py with AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; no GPU).
//
// Random streams of add / append / batched append / free over prompts drawn
// from a few shared prefixes, on small pools so that failures (no blocks) are
// frequent.  After every call it checks, through the C API only:
//   * every live sequence's table has ceil(length / bs) distinct entries in
//     [0, num_blocks), and its slots follow the table;
//   * blocks referenced by live tables plus free blocks account for the pool:
//     num_free == num_blocks - |blocks referenced by some table|;
//   * a failed call (PA_ERR_NO_BLOCKS) leaves num_free and every table as it was.
// Exit status 0 when all checks pass.
#include <stdint.h>
#include <stdio.h>

#include <map>
#include <random>
#include <set>
#include <vector>

#include "paged_kv.h"

#define CHECK(c)                                                       \
  do {                                                                 \
    if (!(c)) {                                                        \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                        \
    }                                                                  \
  } while (0)

static int snapshot(const pa_block_manager* bm, const std::map<int64_t, int32_t>& live, int32_t nb, int32_t bs,
                    std::map<int64_t, std::vector<int32_t>>* tables) {
  std::set<int32_t> used;
  tables->clear();
  for (const auto& kv : live) {
    std::vector<int32_t> t(4096);
    int32_t n = 0;
    CHECK(pa_bm_block_table(bm, kv.first, t.data(), (int32_t)t.size(), &n) == PA_OK);
    t.resize((size_t)n);
    CHECK(pa_bm_length(bm, kv.first) == kv.second);
    CHECK(n == (kv.second + bs - 1) / bs);
    CHECK(std::set<int32_t>(t.begin(), t.end()).size() == t.size());
    for (int32_t b : t) CHECK(b >= 0 && b < nb);
    used.insert(t.begin(), t.end());
    if (kv.second > 0) {
      std::vector<int64_t> s((size_t)kv.second);
      CHECK(pa_bm_slots(bm, kv.first, 0, kv.second, s.data()) == PA_OK);
      for (int32_t p = 0; p < kv.second; ++p) CHECK(s[(size_t)p] == (int64_t)t[(size_t)(p / bs)] * bs + p % bs);
    }
    (*tables)[kv.first] = t;
  }
  CHECK(pa_bm_num_free(bm) == nb - (int32_t)used.size());
  return 0;
}

int main() {
  std::mt19937_64 rng(12345);
  int calls = 0, failures = 0;
  for (int trial = 0; trial < 200; ++trial) {
    const int32_t bs = 1 + (int32_t)(rng() % 8);
    const int32_t nb = 4 + (int32_t)(rng() % 60);
    pa_block_manager* bm = pa_bm_create(nb, bs);
    CHECK(bm != nullptr);
    std::vector<std::vector<int64_t>> prefixes(3);
    for (auto& p : prefixes) {
      const int len = (int)(rng() % (size_t)(4 * bs + 1));
      for (int i = 0; i < len; ++i) p.push_back((int64_t)(rng() % 20));
    }
    std::map<int64_t, int32_t> live;   // id -> length
    std::map<int64_t, std::vector<int32_t>> before, after;
    for (int step = 0; step < 150; ++step) {
      if (snapshot(bm, live, nb, bs, &before)) return 1;
      const int32_t free0 = pa_bm_num_free(bm);
      const int op = (int)(rng() % 10);
      int st = PA_OK;
      if (op < 4 || live.empty()) {
        std::vector<int64_t> toks = prefixes[rng() % 3];
        const int extra = (int)(rng() % (size_t)(2 * bs + 1));
        for (int i = 0; i < extra; ++i) toks.push_back((int64_t)(rng() % 20));
        int64_t id = -1;
        int32_t cached = -1;
        st = pa_bm_add_sequence(bm, toks.data(), (int32_t)toks.size(), &id, &cached);
        if (st == PA_OK) {
          CHECK(cached >= 0 && cached % bs == 0 && cached <= (int32_t)toks.size());
          live[id] = (int32_t)toks.size();
        }
      } else if (op < 7) {
        auto it = live.begin();
        std::advance(it, (long)(rng() % live.size()));
        int64_t slot = -1;
        st = pa_bm_append(bm, it->first, (int64_t)(rng() % 20), &slot);
        if (st == PA_OK) {
          const int32_t p = it->second++;
          int64_t s = -1;
          CHECK(pa_bm_slots(bm, it->first, p, 1, &s) == PA_OK && s == slot);
        }
      } else if (op < 9) {
        std::vector<int64_t> ids, toks;
        for (const auto& kv : live)
          if (rng() % 2) ids.push_back(kv.first);
        for (size_t i = 0; i < ids.size(); ++i) toks.push_back((int64_t)(rng() % 20));
        std::vector<int64_t> slots(ids.size());
        st = pa_bm_append_batch(bm, ids.data(), toks.data(), (int32_t)ids.size(), slots.data());
        if (st == PA_OK)
          for (int64_t id : ids) ++live[id];
      } else {
        auto it = live.begin();
        std::advance(it, (long)(rng() % live.size()));
        CHECK(pa_bm_free_sequence(bm, it->first) == PA_OK);
        live.erase(it);
      }
      ++calls;
      CHECK(st == PA_OK || st == PA_ERR_NO_BLOCKS);
      if (snapshot(bm, live, nb, bs, &after)) return 1;
      if (st == PA_ERR_NO_BLOCKS) {
        ++failures;
        CHECK(pa_bm_num_free(bm) == free0 && after == before);
      }
    }
    // unknown ids and bad arguments are rejected
    int64_t slot = 0;
    CHECK(pa_bm_append(bm, 1 << 30, 1, &slot) == PA_ERR_NO_SEQUENCE);
    CHECK(pa_bm_free_sequence(bm, -5) == PA_ERR_NO_SEQUENCE);
    CHECK(pa_bm_add_sequence(bm, nullptr, 3, &slot, nullptr) == PA_ERR_NULL);
    pa_bm_destroy(bm);
  }
  printf("ok: %d calls, %d refused for lack of blocks\n", calls, failures);
  return 0;
}
