// Host-side KV block manager: free list, reference counts, per-sequence
// block tables, copy-on-write planning, a prefix cache keyed by
// (parent registration, extra hash, tokens) and LRU eviction of unreferenced
// cached blocks.  Plain C++17; no device code.
#include "block_manager.h"

#include <algorithm>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

namespace {

// splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", 2014): a well-mixed 64-bit hash step.
inline uint64_t mix64(uint64_t z) {
  z += 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

uint64_t prefix_hash(uint64_t parent, uint64_t extra, const int32_t* tokens, int32_t n) {
  uint64_t h = mix64(parent ^ mix64(extra));
  for (int32_t i = 0; i < n; ++i) h = mix64(h ^ (uint32_t)tokens[i]);
  return h;
}

// First-in first-out queue of block ids in a ring sized once for every
// block, so queueing a released block never allocates.
struct BlockRing {
  std::vector<int32_t> buf;
  int64_t head = 0, count = 0;
  void init(int64_t capacity) { buf.assign((size_t)capacity, 0); }
  bool empty() const { return count == 0; }
  int64_t size() const { return count; }
  int32_t front() const { return buf[(size_t)head]; }
  void pop_front() {
    if (++head == (int64_t)buf.size()) head = 0;
    --count;
  }
  void push_back(int32_t b) {
    int64_t i = head + count;   // < 2 * capacity
    if (i >= (int64_t)buf.size()) i -= (int64_t)buf.size();
    buf[(size_t)i] = b;
    ++count;
  }
};

// Doubly linked list of block ids through per-block links, oldest first:
// appending, unlinking and taking the oldest never allocate.
struct BlockLru {
  std::vector<int32_t> prev, next;
  int32_t head = -1, tail = -1;
  int64_t count = 0;
  void init(int64_t n) {
    prev.assign((size_t)n, -1);
    next.assign((size_t)n, -1);
  }
  int64_t size() const { return count; }
  int32_t front() const { return head; }
  void push_back(int32_t b) {
    prev[(size_t)b] = tail;
    next[(size_t)b] = -1;
    if (tail >= 0) next[(size_t)tail] = b; else head = b;
    tail = b;
    ++count;
  }
  void erase(int32_t b) {
    const int32_t p = prev[(size_t)b], n = next[(size_t)b];
    if (p >= 0) next[(size_t)p] = n; else head = n;
    if (n >= 0) prev[(size_t)n] = p; else tail = p;
    prev[(size_t)b] = next[(size_t)b] = -1;
    --count;
  }
  void pop_front() { erase(head); }
};

struct Block {
  int32_t ref = 0;
  uint64_t last_access = 0;
  uint64_t serial = 0;             // registration of the cached prefix; 0 = none
  uint64_t parent = 0;             // parent block's registration (0 = first block)
  uint64_t extra = 0;
  uint64_t hash = 0;
  std::vector<int32_t> tokens;     // the block's tokens while registered
  bool in_lru = false;
};

struct Sequence {
  std::vector<int32_t> table;
  int32_t len = 0;
  uint64_t extra = 0;
  bool track = false;              // tokens known so far: full blocks get registered
  std::vector<int32_t> pending;    // tokens of the partial last block
};

}  // namespace

struct bm_manager {
  int64_t num_blocks = 0;
  int32_t bs = 0;
  bool prefix = false;
  std::vector<Block> blocks;
  BlockRing free_list;                              // unreferenced, no cached prefix
  BlockLru lru;                                     // unreferenced cached blocks, oldest first
  std::unordered_multimap<uint64_t, int32_t> index; // prefix hash -> registered block
  std::unordered_map<int64_t, Sequence> seqs;
  uint64_t clock = 0;
  uint64_t next_serial = 1;
  bm_stats_t st{};

  int64_t available() const { return free_list.size() + lru.size(); }

  void unregister(int32_t b) {
    Block& k = blocks[b];
    auto range = index.equal_range(k.hash);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        index.erase(it);
        break;
      }
    k.serial = 0;
    k.tokens.clear();
  }

  // A block with no references: the front of the free list, else the least
  // recently used cached block (evicted).  The caller has checked available().
  int32_t take() {
    int32_t b;
    if (!free_list.empty()) {
      b = free_list.front();
      free_list.pop_front();
    } else {
      b = lru.front();
      lru.pop_front();
      blocks[b].in_lru = false;
      unregister(b);
      ++st.evictions;
    }
    blocks[b].ref = 1;
    blocks[b].last_access = ++clock;
    ++st.allocations;
    return b;
  }

  void drop(int32_t b) {
    Block& k = blocks[b];
    if (--k.ref > 0) return;
    if (k.serial != 0) {
      k.last_access = ++clock;
      lru.push_back(b);
      k.in_lru = true;
    } else {
      free_list.push_back(b);
    }
  }

  // Another reference to a block (shared prefix): leaves the LRU list if it
  // was there.
  void acquire(int32_t b) {
    Block& k = blocks[b];
    if (k.in_lru) {
      lru.erase(b);
      k.in_lru = false;
    }
    ++k.ref;
    k.last_access = ++clock;
  }

  int32_t lookup(uint64_t parent, uint64_t extra, const int32_t* tokens) const {
    const uint64_t h = prefix_hash(parent, extra, tokens, bs);
    auto range = index.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const Block& k = blocks[it->second];
      if (k.parent == parent && k.extra == extra && std::equal(k.tokens.begin(), k.tokens.end(), tokens))
        return it->second;
    }
    return -1;
  }

  // Register the sequence's last block, which has just become full.
  void register_full(Sequence& s) {
    if (!prefix || !s.track) return;
    const size_t nb = s.table.size();
    uint64_t parent = 0;
    if (nb >= 2) {
      parent = blocks[s.table[nb - 2]].serial;
      if (parent == 0) {   // the chain is broken: nothing after it can be found
        s.track = false;
        return;
      }
    }
    if (lookup(parent, s.extra, s.pending.data()) >= 0) {   // the same prefix is held elsewhere
      s.track = false;
      return;
    }
    Block& k = blocks[s.table.back()];
    k.serial = next_serial++;
    k.parent = parent;
    k.extra = s.extra;
    k.tokens = s.pending;
    k.hash = prefix_hash(parent, s.extra, s.pending.data(), bs);
    index.emplace(k.hash, s.table.back());
  }

  // Blocks that appending `count` tokens to s takes (new logical blocks plus
  // one copy-on-write block).
  int64_t blocks_needed(const Sequence& s, int32_t count) const {
    if (count <= 0) return 0;
    const int64_t first = s.len, last = (int64_t)s.len + count - 1;
    int64_t need = last / bs - (first + bs - 1) / bs + 1;   // positions p in [first, last] with p % bs == 0
    if (need < 0) need = 0;
    if (first % bs != 0 && blocks[s.table.back()].ref > 1) ++need;
    return need;
  }

  // Append one token (capacity checked by the caller).
  void append_one(Sequence& s, const int32_t* token, int64_t* slot, int32_t* pair, int32_t* npairs) {
    const int32_t pos = s.len;
    const int32_t off = pos % bs;
    if (off == 0) {
      s.table.push_back(take());
      s.pending.clear();
    } else {
      const int32_t last = s.table.back();
      if (blocks[last].ref > 1) {
        const int32_t fresh = take();
        --blocks[last].ref;   // still >= 1: another sequence holds it
        s.table.back() = fresh;
        pair[0] = last;
        pair[1] = fresh;
        ++*npairs;
        ++st.cow_copies;
      }
    }
    s.len = pos + 1;
    *slot = (int64_t)s.table.back() * bs + off;
    if (s.track) {
      if (token) {
        s.pending.push_back(*token);
        if (off == bs - 1) register_full(s);
      } else {
        s.track = false;
      }
    }
  }
};

namespace {

bool valid_block_size(int32_t bs) { return bs > 0 && bs <= (1 << 20); }


}  // namespace

extern "C" kv_status_t bm_create(int64_t num_blocks, int32_t block_size, const int32_t* free_order,
                                 int32_t prefix_caching, bm_manager_t** out) {
  if (!out || num_blocks <= 0 || num_blocks > INT32_MAX || !valid_block_size(block_size)) return KV_ERR_INVALID_ARG;
  if ((int64_t)block_size * num_blocks > ((int64_t)1 << 62)) return KV_ERR_INVALID_ARG;
  *out = nullptr;
  bm_manager_t* bm = new (std::nothrow) bm_manager_t();
  if (!bm) return KV_ERR_OOM;
  try {
    bm->num_blocks = num_blocks;
    bm->bs = block_size;
    bm->prefix = prefix_caching != 0;
    bm->blocks.resize((size_t)num_blocks);
    bm->free_list.init(num_blocks);
    bm->lru.init(num_blocks);
    if (free_order) {
      std::vector<char> seen((size_t)num_blocks, 0);
      for (int64_t i = 0; i < num_blocks; ++i) {
        const int32_t b = free_order[i];
        if (b < 0 || b >= num_blocks || seen[(size_t)b]) {
          delete bm;
          return KV_ERR_INVALID_ARG;
        }
        seen[(size_t)b] = 1;
        bm->free_list.push_back(b);
      }
    } else {
      for (int64_t i = 0; i < num_blocks; ++i) bm->free_list.push_back((int32_t)i);
    }
  } catch (const std::bad_alloc&) {
    delete bm;
    return KV_ERR_OOM;
  }
  bm->st.num_blocks = num_blocks;
  *out = bm;
  return KV_OK;
}

extern "C" void bm_destroy(bm_manager_t* bm) { delete bm; }

extern "C" kv_status_t bm_add_sequence(bm_manager_t* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                                       uint64_t extra_hash, int64_t* slots, int32_t* num_cached) {
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !slots)) return KV_ERR_INVALID_ARG;
  if (bm->seqs.count(seq)) return KV_ERR_INVALID_ARG;
  const int32_t bs = bm->bs;
  try {
    // 1. leading full blocks found in the prefix cache (no side effects yet)
    std::vector<int32_t> hit;
    int64_t queries = 0;
    const bool track = bm->prefix && tokens != nullptr;
    if (track) {
      uint64_t parent = 0;
      for (int32_t k = 0; (int64_t)(k + 1) * bs <= num_tokens; ++k) {
        ++queries;
        const int32_t b = bm->lookup(parent, extra_hash, tokens + (int64_t)k * bs);
        if (b < 0) break;
        hit.push_back(b);
        parent = bm->blocks[b].serial;
      }
    }
    const int32_t cached = (int32_t)hit.size() * bs;
    int64_t in_lru = 0;
    for (int32_t b : hit) in_lru += bm->blocks[b].in_lru ? 1 : 0;
    const int64_t need = (num_tokens - cached + bs - 1) / bs;
    if (need > bm->available() - in_lru) return KV_ERR_NO_BLOCKS;

    // 2. commit
    Sequence& s = bm->seqs[seq];
    s.extra = extra_hash;
    s.track = track;
    for (int32_t b : hit) {
      bm->acquire(b);
      s.table.push_back(b);
    }
    s.len = cached;
    for (int32_t i = 0; i < cached; ++i)
      slots[i] = (int64_t)s.table[(size_t)(i / bs)] * bs + i % bs;
    int32_t pair[2];
    int32_t npairs = 0;
    for (int32_t i = cached; i < num_tokens; ++i)
      bm->append_one(s, tokens ? tokens + i : nullptr, slots + i, pair, &npairs);
    bm->st.prefix_queries += queries;
    bm->st.prefix_hits += (int64_t)hit.size();
    if (num_cached) *num_cached = cached;
  } catch (const std::bad_alloc&) {
    return KV_ERR_OOM;
  }
  return KV_OK;
}

extern "C" kv_status_t bm_fork(bm_manager_t* bm, int64_t parent, const int64_t* children, int32_t num_children) {
  if (!bm || num_children < 0 || (num_children > 0 && !children)) return KV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return KV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < num_children; ++i) {
    if (bm->seqs.count(children[i]) || children[i] == parent) return KV_ERR_INVALID_ARG;
    for (int32_t j = 0; j < i; ++j)
      if (children[j] == children[i]) return KV_ERR_INVALID_ARG;
  }
  try {
    const Sequence src = it->second;   // copy: inserting may rehash
    for (int32_t i = 0; i < num_children; ++i) {
      bm->seqs[children[i]] = src;
      for (int32_t b : src.table) ++bm->blocks[b].ref;
    }
  } catch (const std::bad_alloc&) {
    return KV_ERR_OOM;
  }
  return KV_OK;
}

extern "C" kv_status_t bm_append_slots(bm_manager_t* bm, int64_t seq, const int32_t* tokens, int32_t count,
                                       int64_t* slots, int32_t* copy_pairs, int32_t* num_pairs) {
  if (!bm || count < 0 || (count > 0 && (!slots || !copy_pairs)) || !num_pairs) return KV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return KV_ERR_INVALID_ARG;
  Sequence& s = it->second;
  if ((int64_t)s.len + count > INT32_MAX) return KV_ERR_INVALID_ARG;
  if (bm->blocks_needed(s, count) > bm->available()) return KV_ERR_NO_BLOCKS;
  *num_pairs = 0;
  try {
    for (int32_t i = 0; i < count; ++i) bm->append_one(s, tokens ? tokens + i : nullptr, slots + i, copy_pairs, num_pairs);
  } catch (const std::bad_alloc&) {
    return KV_ERR_OOM;
  }
  return KV_OK;
}

extern "C" kv_status_t bm_append_batch(bm_manager_t* bm, const int64_t* seqs, const int32_t* counts, int32_t n,
                                       const int32_t* tokens, int64_t* slots, int32_t* copy_pairs, int32_t* num_pairs) {
  if (!bm || n < 0 || !num_pairs || (n > 0 && (!seqs || !counts || !copy_pairs))) return KV_ERR_INVALID_ARG;
  try {
    // Validate and count the blocks the batch takes, in list order: a shared
    // last block costs a copy for every writer while its count is above one.
    std::vector<Sequence*> list((size_t)n);
    std::unordered_map<int64_t, int32_t> seen;
    std::unordered_map<int32_t, int32_t> ref_drop;
    int64_t need = 0, total = 0;
    const int32_t bs = bm->bs;
    for (int32_t i = 0; i < n; ++i) {
      auto it = bm->seqs.find(seqs[i]);
      if (it == bm->seqs.end() || counts[i] < 0 || !seen.emplace(seqs[i], i).second) return KV_ERR_INVALID_ARG;
      Sequence& s = it->second;
      if ((int64_t)s.len + counts[i] > INT32_MAX) return KV_ERR_INVALID_ARG;
      list[(size_t)i] = &s;
      total += counts[i];
      if (counts[i] == 0) continue;
      const int64_t first = s.len, last = first + counts[i] - 1;
      need += last / bs - (first + bs - 1) / bs + 1;
      if (first % bs != 0) {
        const int32_t b = s.table.back();
        if (bm->blocks[b].ref - ref_drop[b] > 1) {
          ++need;
          ++ref_drop[b];
        }
      }
    }
    if (total > 0 && !slots) return KV_ERR_INVALID_ARG;
    if (need > bm->available()) return KV_ERR_NO_BLOCKS;
    *num_pairs = 0;
    int64_t k = 0;
    for (int32_t i = 0; i < n; ++i)
      for (int32_t j = 0; j < counts[i]; ++j, ++k)
        bm->append_one(*list[(size_t)i], tokens ? tokens + k : nullptr, slots + k, copy_pairs + 2 * *num_pairs,
                       num_pairs);
  } catch (const std::bad_alloc&) {
    return KV_ERR_OOM;
  }
  return KV_OK;
}

// Releasing blocks only relinks them (free ring, LRU links), so this call
// allocates nothing and cannot fail part way.
extern "C" kv_status_t bm_free(bm_manager_t* bm, int64_t seq) {
  if (!bm) return KV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return KV_ERR_INVALID_ARG;
  const std::vector<int32_t>& t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b) bm->drop(*b);
  bm->seqs.erase(it);
  return KV_OK;
}

extern "C" kv_status_t bm_num_free_blocks(const bm_manager_t* bm, int64_t* n) {
  if (!bm || !n) return KV_ERR_INVALID_ARG;
  *n = bm->available();
  return KV_OK;
}

extern "C" kv_status_t bm_sequence_info(const bm_manager_t* bm, int64_t seq, int32_t* length, int32_t* num_blocks) {
  if (!bm) return KV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return KV_ERR_INVALID_ARG;
  if (length) *length = it->second.len;
  if (num_blocks) *num_blocks = (int32_t)it->second.table.size();
  return KV_OK;
}

extern "C" kv_status_t bm_block_table(const bm_manager_t* bm, int64_t seq, int32_t* out, int32_t capacity) {
  if (!bm || capacity < 0 || (capacity > 0 && !out)) return KV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return KV_ERR_INVALID_ARG;
  const std::vector<int32_t>& t = it->second.table;
  if ((int64_t)t.size() > capacity) return KV_ERR_INVALID_ARG;
  std::copy(t.begin(), t.end(), out);
  return KV_OK;
}

extern "C" kv_status_t bm_block_tables(const bm_manager_t* bm, const int64_t* seqs, int32_t n, int32_t max_blocks,
                                       int32_t* out, int32_t* context_lens) {
  if (!bm || n < 0 || max_blocks <= 0 || (n > 0 && (!seqs || !out))) return KV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end() || (int64_t)it->second.table.size() > max_blocks) return KV_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Sequence& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = out + (int64_t)i * max_blocks;
    std::fill(row, row + max_blocks, -1);
    std::copy(s.table.begin(), s.table.end(), row);
    if (context_lens) context_lens[i] = s.len;
  }
  return KV_OK;
}

extern "C" kv_status_t bm_ref_count(const bm_manager_t* bm, int32_t block, int32_t* ref) {
  if (!bm || !ref || block < 0 || block >= bm->num_blocks) return KV_ERR_INVALID_ARG;
  *ref = bm->blocks[(size_t)block].ref;
  return KV_OK;
}

extern "C" kv_status_t bm_stats(const bm_manager_t* bm, bm_stats_t* out) {
  if (!bm || !out) return KV_ERR_INVALID_ARG;
  bm_stats_t s = bm->st;
  s.num_blocks = bm->num_blocks;
  s.free_blocks = bm->free_list.size();
  s.cached_blocks = bm->lru.size();
  s.used_blocks = bm->num_blocks - s.free_blocks - s.cached_blocks;
  s.num_sequences = (int64_t)bm->seqs.size();
  s.tokens = 0;
  s.table_entries = 0;
  for (const auto& kv : bm->seqs) {
    s.tokens += kv.second.len;
    s.table_entries += (int64_t)kv.second.table.size();
  }
  *out = s;
  return KV_OK;
}
