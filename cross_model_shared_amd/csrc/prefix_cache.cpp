// Host-side page allocator with a prefix cache of full 16-token blocks, and the
// grouping of sessions that share leading pages (kvs_prefix_cache.h).
//
// Prefill-as-a-Service, component 3 (hybrid prefix cache pool): only
// block-aligned, full blocks are reused across requests.  A page is free,
// referenced (count > 0), or cached and unreferenced (evictable).  Cache
// entries are keyed by the whole token prefix up to the end of their block,
// through a chain of two independent 64-bit hashes; an entry keeps its parent
// key and its 16 tokens, which every lookup compares.
#include <stdint.h>
#include <string.h>

#include <new>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/kvs_prefix_cache.h"
#include "kvs_internal.h"

namespace {

constexpr int kBlock = 16;

struct Key {
  uint64_t h1, h2;
  bool operator==(const Key& o) const { return h1 == o.h1 && h2 == o.h2; }
};

struct KeyHash {
  size_t operator()(const Key& k) const { return size_t(k.h1 ^ (k.h2 * 0x9E3779B97F4A7C15ull)); }
};

// The key of the empty prefix.
constexpr Key kRoot{0x243F6A8885A308D3ull, 0x13198A2E03707344ull};

// splitmix64's finalizer (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", 2014).
inline uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xBF58476D1CE4E5B9ull;
  x ^= x >> 27;
  x *= 0x94D049BB133111EBull;
  x ^= x >> 31;
  return x;
}

// Key of a block: its parent's key chained with its 16 tokens, two ways.
Key block_key(const Key& parent, const int32_t* t) {
  uint64_t a = parent.h1, b = parent.h2 ^ 0xA4093822299F31D0ull;
  for (int i = 0; i < kBlock; ++i) {
    const uint64_t v = uint32_t(t[i]);
    a = mix64(a ^ (v + 0x9E3779B97F4A7C15ull * uint64_t(i + 1)));
    b = mix64((b + v) * 0xD6E8FEB86659FD93ull + uint64_t(i));
  }
  return Key{a, b};
}

struct Entry {
  int32_t page;
  Key parent;
  int32_t tokens[kBlock];
};

}  // namespace

struct kvs_prefix_cache {
  int32_t num_pages = 0;
  std::vector<int32_t> ref;           // references per page
  std::vector<uint8_t> has_entry;     // page holds a cache entry
  std::vector<Key> page_key;          // ... under this key
  std::vector<uint64_t> released_at;  // tick at which an evictable page lost its last reference
  std::set<int32_t> free_pages;       // lowest id first
  std::set<std::pair<uint64_t, int32_t>> evictable;  // (tick, page), earliest first
  std::unordered_map<Key, Entry, KeyHash> entries;
  uint64_t tick = 0;

  // Entry for block `t` under `parent`, if present and its tokens match.
  const Entry* find(const Key& key, const Key& parent, const int32_t* t) const {
    auto it = entries.find(key);
    if (it == entries.end()) return nullptr;
    const Entry& e = it->second;
    if (!(e.parent == parent) || memcmp(e.tokens, t, sizeof e.tokens) != 0) return nullptr;
    return &e;
  }
};

extern "C" {

kvs_prefix_cache* kvs_prefix_cache_create(int32_t num_pages) {
  if (num_pages <= 0) {
    kvs::set_error(KVS_EINVAL, "kvs_prefix_cache_create: num_pages must be positive");
    return nullptr;
  }
  kvs_prefix_cache* pc = new (std::nothrow) kvs_prefix_cache;
  if (!pc) return nullptr;
  try {
    pc->num_pages = num_pages;
    pc->ref.assign(num_pages, 0);
    pc->has_entry.assign(num_pages, 0);
    pc->page_key.assign(num_pages, Key{0, 0});
    pc->released_at.assign(num_pages, 0);
    for (int32_t p = 0; p < num_pages; ++p) pc->free_pages.insert(pc->free_pages.end(), p);
  } catch (...) {
    delete pc;
    return nullptr;
  }
  return pc;
}

void kvs_prefix_cache_destroy(kvs_prefix_cache* pc) { delete pc; }

int kvs_prefix_cache_admit(kvs_prefix_cache* pc, const int32_t* tokens, int32_t L, int32_t* bt_row,
                           int32_t* matched_pages) {
  if (!pc || !bt_row || !matched_pages || L < 0 || (L > 0 && !tokens))
    return kvs::set_error(KVS_EINVAL, "kvs_prefix_cache_admit: NULL argument or negative length");
  const int32_t nblocks = (L + kBlock - 1) / kBlock, full = L / kBlock;
  // 1. longest run of leading full blocks in the cache
  std::vector<int32_t> matched;
  Key prev = kRoot;
  for (int32_t i = 0; i < full; ++i) {
    const int32_t* t = tokens + int64_t(i) * kBlock;
    const Key key = block_key(prev, t);
    const Entry* e = pc->find(key, prev, t);
    if (!e) break;
    matched.push_back(e->page);
    prev = key;
  }
  // 2. room for the rest: free pages, then evictable ones not revived here
  const int32_t need = nblocks - int32_t(matched.size());
  int64_t revived = 0;
  for (int32_t p : matched) revived += pc->ref[p] == 0;
  const int64_t room = int64_t(pc->free_pages.size()) + int64_t(pc->evictable.size()) - revived;
  if (need > room)
    return kvs::set_error(KVS_ENOSPACE, "kvs_prefix_cache_admit: %d new pages needed, %lld available", need,
                          (long long)room);
  // 3. commit
  for (int32_t p : matched) {
    if (pc->ref[p] == 0) pc->evictable.erase({pc->released_at[p], p});
    ++pc->ref[p];
  }
  int32_t i = 0;
  for (; i < int32_t(matched.size()); ++i) bt_row[i] = matched[i];
  for (; i < nblocks; ++i) {
    int32_t p;
    if (!pc->free_pages.empty()) {
      p = *pc->free_pages.begin();
      pc->free_pages.erase(pc->free_pages.begin());
    } else {
      p = pc->evictable.begin()->second;
      pc->evictable.erase(pc->evictable.begin());
      pc->entries.erase(pc->page_key[p]);
      pc->has_entry[p] = 0;
    }
    pc->ref[p] = 1;
    bt_row[i] = p;
  }
  *matched_pages = int32_t(matched.size());
  return KVS_OK;
}

int kvs_prefix_cache_publish(kvs_prefix_cache* pc, const int32_t* tokens, int32_t L, const int32_t* bt_row) {
  if (!pc || L < 0 || (L >= kBlock && (!tokens || !bt_row)))
    return kvs::set_error(KVS_EINVAL, "kvs_prefix_cache_publish: NULL argument or negative length");
  const int32_t full = L / kBlock;
  for (int32_t i = 0; i < full; ++i) {
    const int32_t p = bt_row[i];
    if (p < 0 || p >= pc->num_pages || pc->ref[p] <= 0)
      return kvs::set_error(KVS_ERANGE, "kvs_prefix_cache_publish: block %d: page %d is not a referenced page", i,
                            p);
  }
  Key prev = kRoot;
  for (int32_t i = 0; i < full; ++i) {
    const int32_t* t = tokens + int64_t(i) * kBlock;
    const int32_t p = bt_row[i];
    const Key key = block_key(prev, t);
    if (pc->entries.find(key) == pc->entries.end() && !pc->has_entry[p]) {
      Entry e;
      e.page = p;
      e.parent = prev;
      memcpy(e.tokens, t, sizeof e.tokens);
      pc->entries.emplace(key, e);
      pc->has_entry[p] = 1;
      pc->page_key[p] = key;
    }
    prev = key;
  }
  return KVS_OK;
}

int kvs_prefix_cache_release(kvs_prefix_cache* pc, const int32_t* bt_row, int32_t npages) {
  if (!pc || npages < 0 || (npages > 0 && !bt_row))
    return kvs::set_error(KVS_EINVAL, "kvs_prefix_cache_release: NULL argument or negative count");
  std::unordered_map<int32_t, int32_t> drops;
  for (int32_t i = 0; i < npages; ++i) {
    const int32_t p = bt_row[i];
    if (p < 0 || p >= pc->num_pages)
      return kvs::set_error(KVS_ERANGE, "kvs_prefix_cache_release: page id %d outside the pool", p);
    if (++drops[p] > pc->ref[p])
      return kvs::set_error(KVS_ERANGE, "kvs_prefix_cache_release: page %d released more often than referenced", p);
  }
  for (int32_t i = 0; i < npages; ++i) {
    const int32_t p = bt_row[i];
    if (--pc->ref[p] > 0) continue;
    if (pc->has_entry[p]) {
      pc->released_at[p] = ++pc->tick;
      pc->evictable.insert({pc->released_at[p], p});
    } else {
      pc->free_pages.insert(p);
    }
  }
  return KVS_OK;
}

int kvs_prefix_cache_stats(const kvs_prefix_cache* pc, int32_t* free_pages, int32_t* evictable_pages,
                           int32_t* referenced_pages, int32_t* entries) {
  if (!pc) return kvs::set_error(KVS_EINVAL, "kvs_prefix_cache_stats: NULL handle");
  if (free_pages) *free_pages = int32_t(pc->free_pages.size());
  if (evictable_pages) *evictable_pages = int32_t(pc->evictable.size());
  if (referenced_pages)
    *referenced_pages = pc->num_pages - int32_t(pc->free_pages.size()) - int32_t(pc->evictable.size());
  if (entries) *entries = int32_t(pc->entries.size());
  return KVS_OK;
}

int kvs_prefix_cache_refcount(const kvs_prefix_cache* pc, int32_t page) {
  if (!pc) return kvs::set_error(KVS_EINVAL, "kvs_prefix_cache_refcount: NULL handle");
  if (page < 0 || page >= pc->num_pages)
    return kvs::set_error(KVS_ERANGE, "kvs_prefix_cache_refcount: page id %d outside the pool", page);
  return pc->ref[page];
}

int kvs_prefix_groups(const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                      int32_t* group_id, int32_t* group_prefix_pages) {
  if (batch < 0 || (batch > 0 && (!block_table || !seq_lens || !group_id || !group_prefix_pages)))
    return kvs::set_error(KVS_EINVAL, "kvs_prefix_groups: NULL argument or negative batch");
  for (int32_t b = 0; b < batch; ++b) {
    if (seq_lens[b] < 0) return kvs::set_error(KVS_EINVAL, "kvs_prefix_groups: seq_lens[%d] is negative", b);
    if (int64_t(seq_lens[b]) > int64_t(bt_stride) * kBlock)
      return kvs::set_error(KVS_ERANGE, "kvs_prefix_groups: seq_lens[%d] = %d exceeds bt_stride * 16", b,
                            seq_lens[b]);
  }
  auto row = [&](int32_t b) { return block_table + int64_t(b) * bt_stride; };
  int32_t b = 0;
  while (b < batch) {
    int32_t e = b + 1;
    if (seq_lens[b] >= kBlock)
      while (e < batch && seq_lens[e] >= kBlock && row(e)[0] == row(b)[0]) ++e;
    int32_t P = 0;
    if (e - b >= 2) {
      int32_t full = seq_lens[b] / kBlock;
      for (int32_t m = b + 1; m < e; ++m) full = seq_lens[m] / kBlock < full ? seq_lens[m] / kBlock : full;
      while (P < full) {
        bool same = true;
        for (int32_t m = b + 1; m < e && same; ++m) same = row(m)[P] == row(b)[P];
        if (!same) break;
        ++P;
      }
    }
    for (int32_t m = b; m < e; ++m) {
      group_id[m] = P > 0 ? b : -1;
      group_prefix_pages[m] = P;
    }
    b = e;
  }
  return KVS_OK;
}

}  // extern "C"
