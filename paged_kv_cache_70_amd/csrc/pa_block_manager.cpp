// Host block manager with prefix sharing: hands out the physical blocks whose
// ids fill the block tables, slot mappings and context lengths the kernels
// consume.
//
// Sources: the third page's BlockManager (a C++ engine write-up): a pool of
// fixed-size blocks, each with its token ids and a hash of its tokens chained
// with its prefix's hash, a hash -> block map, a queue of free ids, and an
// allocate call that reports how many leading tokens are already cached;
// "PagedAttention kernel：paged KV cache 与 block table", 面试官追问: sequences
// that share a prompt prefix point their tables at the same physical blocks.
// Where the pages stop (reference counts, freeing, eviction), the reading is:
//   * full blocks are shared under the chained key h_i = FNV-1a-64 of the
//     8-byte little-endian words (h_{i-1}, t_0 .. t_{bs-1}), h_{-1} = all ones,
//     and only when the stored tokens are equal too; partial blocks are
//     private; a block is registered once it is full;
//   * a new sequence reuses cached blocks from its start up to the first
//     block that is not cached; everything after is new;
//   * reference counts; a block whose count drops to 0 goes to the back of
//     the free queue and keeps its key, so a later sequence can revive it;
//   * new blocks come from the front of the queue (initially 0 .. NB-1); a
//     cached block reused that way is evicted (its key dropped);
//   * an operation that cannot get its blocks fails and changes nothing.
// Not thread-safe: one manager per thread, or a lock around it.
//
// Every operation is O(1) per block: the free queue is a doubly linked list
// threaded through per-block next/prev arrays (pop front, push back, unlink a
// revived block), the key map is a hash map reserved for the pool.
#include <stdint.h>
#include <string.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/paged_kv.h"

namespace {

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;   // FNV-1a 64-bit offset basis
constexpr uint64_t kFnvPrime = 0x100000001B3ull;         // FNV 64-bit prime
constexpr uint64_t kNoParent = ~0ull;

inline uint64_t fnv_word(uint64_t h, uint64_t w) {
  for (int i = 0; i < 8; ++i) {
    h ^= (w >> (8 * i)) & 0xffu;
    h *= kFnvPrime;
  }
  return h;
}

uint64_t block_key(uint64_t parent, const int64_t* tokens, int32_t bs) {
  uint64_t h = fnv_word(kFnvOffset, parent);
  for (int32_t i = 0; i < bs; ++i) h = fnv_word(h, (uint64_t)tokens[i]);
  return h;
}

struct Sequence {
  std::vector<int64_t> tokens;
  std::vector<int32_t> blocks;
  std::vector<uint64_t> keys;   // keys of the full blocks, in order
  uint64_t stamp = 0;           // last batched append that listed it
};

}  // namespace

struct pa_block_manager {
  int32_t nb, bs;
  std::vector<int32_t> refs;
  std::vector<uint8_t> registered;
  std::vector<uint64_t> key;
  std::vector<int64_t> tokens;        // [nb * bs]: the tokens of registered blocks
  std::vector<int32_t> next, prev;    // free queue links (-1: none)
  std::vector<uint8_t> in_free;
  int32_t head = -1, tail = -1, nfree = 0;
  std::unordered_map<uint64_t, int32_t> by_key;
  std::unordered_map<int64_t, Sequence> seqs;
  int64_t next_seq = 0;
  uint64_t batch_stamp = 0;
  std::vector<Sequence*> batch;   // scratch of pa_bm_append_batch

  pa_block_manager(int32_t n, int32_t b)
      : nb(n), bs(b), refs(n, 0), registered(n, 0), key(n, 0), tokens((size_t)n * b, 0),
        next(n, -1), prev(n, -1), in_free(n, 0) {
    by_key.reserve((size_t)n);
    for (int32_t i = 0; i < n; ++i) push_back(i);
  }

  void push_back(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_free[b] = 1;
    ++nfree;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    in_free[b] = 0;
    --nfree;
  }
  // A new block from the front of the queue; a cached block there is evicted.
  int32_t take() {
    const int32_t b = head;
    unlink(b);
    if (registered[b]) {
      by_key.erase(key[b]);
      registered[b] = 0;
    }
    refs[b] = 1;
    return b;
  }
  void register_block(int32_t b, uint64_t k, const int64_t* toks) {
    if (by_key.find(k) != by_key.end()) return;
    by_key.emplace(k, b);
    registered[b] = 1;
    key[b] = k;
    memcpy(&tokens[(size_t)b * bs], toks, sizeof(int64_t) * (size_t)bs);
  }
  int32_t lookup(uint64_t k, const int64_t* toks) const {
    const auto it = by_key.find(k);
    if (it == by_key.end()) return -1;
    const int32_t b = it->second;
    return memcmp(&tokens[(size_t)b * bs], toks, sizeof(int64_t) * (size_t)bs) == 0 ? b : -1;
  }
};

// One sequence's append, after the checks (known id, a block available).
static int64_t append_one(pa_block_manager* bm, Sequence& s, int64_t token) {
  const int32_t bs = bm->bs;
  const int64_t pos = (int64_t)s.tokens.size();
  if (pos % bs == 0) s.blocks.push_back(bm->take());
  s.tokens.push_back(token);
  const int32_t b = s.blocks[(size_t)(pos / bs)];
  if (pos % bs == bs - 1) {   // the block just filled up
    const size_t i = (size_t)(pos / bs);
    const uint64_t k = block_key(i ? s.keys[i - 1] : kNoParent, &s.tokens[i * bs], bs);
    s.keys.push_back(k);
    bm->register_block(b, k, &s.tokens[i * bs]);
  }
  return (int64_t)b * bs + pos % bs;
}

// Runs an entry point's body; a C++ exception (a failed host allocation) must
// not cross the C ABI, so it becomes PA_ERR_NO_MEMORY.
template <typename F>
static int guarded(F&& body) {
  try {
    return body();
  } catch (...) {
    return PA_ERR_NO_MEMORY;
  }
}

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  try {
    return new pa_block_manager(num_blocks, block_size);
  } catch (...) {
    return nullptr;
  }
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_add_sequence(pa_block_manager* bm, const int64_t* tokens, int32_t n, int64_t* seq_id,
                       int32_t* cached_tokens) {
  return guarded([&]() -> int {
    if (!bm || !seq_id || (n > 0 && !tokens)) return PA_ERR_NULL;
    if (n < 0) return PA_ERR_SHAPE;
    const int32_t bs = bm->bs;
    const int32_t nfull = n / bs, nblocks = (n + bs - 1) / bs;
    // plan: leading cached blocks, and the keys of every full block
    std::vector<uint64_t> keys((size_t)nfull);
    std::vector<int32_t> reused;
    uint64_t parent = kNoParent;
    int32_t revive = 0;
    for (int32_t i = 0; i < nfull; ++i) {
      keys[i] = block_key(parent, tokens + (size_t)i * bs, bs);
      parent = keys[i];
      if ((int32_t)reused.size() == i) {
        const int32_t b = bm->lookup(keys[i], tokens + (size_t)i * bs);
        if (b >= 0) {
          reused.push_back(b);
          revive += bm->refs[b] == 0;
        }
      }
    }
    if (bm->nfree - revive < nblocks - (int32_t)reused.size()) return PA_ERR_NO_BLOCKS;
    Sequence s;
    s.tokens.assign(tokens, tokens + n);
    s.blocks.reserve((size_t)nblocks);
    for (int32_t b : reused) {
      if (bm->refs[b] == 0) bm->unlink(b);
      ++bm->refs[b];
      s.blocks.push_back(b);
    }
    for (int32_t i = (int32_t)reused.size(); i < nblocks; ++i) {
      const int32_t b = bm->take();
      if (i < nfull) bm->register_block(b, keys[i], tokens + (size_t)i * bs);
      s.blocks.push_back(b);
    }
    s.keys = std::move(keys);
    const int64_t id = bm->next_seq++;
    if (cached_tokens) *cached_tokens = (int32_t)reused.size() * bs;
    bm->seqs.emplace(id, std::move(s));
    *seq_id = id;
    return PA_OK;
  });
}

int pa_bm_append(pa_block_manager* bm, int64_t seq_id, int64_t token, int64_t* slot) {
  return guarded([&]() -> int {
    if (!bm || !slot) return PA_ERR_NULL;
    const auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
    Sequence& s = it->second;
    if (s.tokens.size() >= (size_t)INT32_MAX) return PA_ERR_TOO_LARGE;
    if (s.tokens.size() % (size_t)bm->bs == 0 && bm->nfree == 0) return PA_ERR_NO_BLOCKS;
    *slot = append_one(bm, s, token);
    return PA_OK;
  });
}

int pa_bm_append_batch(pa_block_manager* bm, const int64_t* seq_ids, const int64_t* tokens, int32_t n,
                       int64_t* slots) {
  return guarded([&]() -> int {
    if (!bm || (n > 0 && (!seq_ids || !tokens || !slots))) return PA_ERR_NULL;
    if (n < 0) return PA_ERR_SHAPE;
    // all or nothing: every id known and listed once (a stamp per call), blocks enough
    const uint64_t stamp = ++bm->batch_stamp;
    bm->batch.resize((size_t)n);
    int32_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
      const auto it = bm->seqs.find(seq_ids[i]);
      if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
      Sequence& s = it->second;
      if (s.stamp == stamp) return PA_ERR_SHAPE;
      s.stamp = stamp;
      if (s.tokens.size() >= (size_t)INT32_MAX) return PA_ERR_TOO_LARGE;
      need += s.tokens.size() % (size_t)bm->bs == 0;
      bm->batch[(size_t)i] = &s;
    }
    if (need > bm->nfree) return PA_ERR_NO_BLOCKS;
    for (int32_t i = 0; i < n; ++i) slots[i] = append_one(bm, *bm->batch[(size_t)i], tokens[i]);
    return PA_OK;
  });
}

int pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  const auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
  for (int32_t b : it->second.blocks)
    if (--bm->refs[b] == 0) bm->push_back(b);
  bm->seqs.erase(it);
  return PA_OK;
}

int32_t pa_bm_length(const pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  const auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? PA_ERR_NO_SEQUENCE : (int32_t)it->second.tokens.size();
}

int32_t pa_bm_num_free(const pa_block_manager* bm) { return bm ? bm->nfree : PA_ERR_NULL; }

int pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out, int32_t capacity,
                      int32_t* num_blocks) {
  if (!bm || !num_blocks || (capacity > 0 && !out)) return PA_ERR_NULL;
  const auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
  const std::vector<int32_t>& t = it->second.blocks;
  *num_blocks = (int32_t)t.size();
  if ((int32_t)t.size() > capacity) return PA_ERR_SHAPE;
  if (!t.empty()) memcpy(out, t.data(), sizeof(int32_t) * t.size());
  return PA_OK;
}

int pa_bm_slots(const pa_block_manager* bm, int64_t seq_id, int32_t start, int32_t count, int64_t* out) {
  if (!bm || (count > 0 && !out)) return PA_ERR_NULL;
  const auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
  const Sequence& s = it->second;
  if (start < 0 || count < 0 || (int64_t)start + count > (int64_t)s.tokens.size()) return PA_ERR_SHAPE;
  const int32_t bs = bm->bs;
  for (int32_t p = start; p < start + count; ++p) out[p - start] = (int64_t)s.blocks[p / bs] * bs + p % bs;
  return PA_OK;
}

int pa_bm_fill_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                      int32_t max_blocks_per_seq, int32_t fill, int32_t* block_tables,
                      int32_t* context_lens) {
  if (!bm || (num_seqs > 0 && (!seq_ids || !block_tables || !context_lens))) return PA_ERR_NULL;
  if (num_seqs < 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  for (int32_t i = 0; i < num_seqs; ++i)
    if (bm->seqs.find(seq_ids[i]) == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
  for (int32_t i = 0; i < num_seqs; ++i)
    if ((int32_t)bm->seqs.find(seq_ids[i])->second.blocks.size() > max_blocks_per_seq) return PA_ERR_SHAPE;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Sequence& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + (size_t)i * max_blocks_per_seq;
    const int32_t nbk = (int32_t)s.blocks.size();
    for (int32_t j = 0; j < max_blocks_per_seq; ++j) row[j] = j < nbk ? s.blocks[j] : fill;
    context_lens[i] = (int32_t)s.tokens.size();
  }
  return PA_OK;
}

}  // extern "C"
