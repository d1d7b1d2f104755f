// Host-only block pool manager: which physical blocks hold which cached
// document, under a block budget with least-recently-used eviction, for the
// three cache keys compared by the LazyAttention pages (position-agnostic,
// position-aware, prefix).  Nothing here touches a GPU.
#include <stddef.h>
#include <stdint.h>

#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "lazyattn.h"

namespace {

struct Key {
  int64_t a, b;
  bool operator==(const Key& o) const { return a == o.a && b == o.b; }
};

struct KeyHash {
  size_t operator()(const Key& k) const {
    uint64_t h = static_cast<uint64_t>(k.a) * 0x9E3779B97F4A7C15ull;
    h ^= static_cast<uint64_t>(k.b) + 0x7F4A7C159E3779B9ull + (h << 6) + (h >> 2);
    return static_cast<size_t>(h);
  }
};

struct Entry {
  std::vector<uint32_t> blocks;
  int32_t pins = 0;
  bool in_lru = false;
  std::list<Key>::iterator lru_pos;
};

}  // namespace

struct lazyattn_pool {
  int32_t policy = LAZYATTN_CACHE_POSITION_AGNOSTIC;
  std::vector<uint32_t> free_blocks;                 // a stack: the back is handed out next
  std::unordered_map<Key, Entry, KeyHash> cache;
  std::list<Key> lru;                                // front = least recently used, unpinned only
  std::unordered_map<Key, int64_t, KeyHash> prefix_nodes;   // (parent node, document) -> node
  int64_t next_node = 1;                             // node 0 is the empty prefix
  std::unordered_map<int64_t, std::vector<Key>> open; // ticket -> pinned keys, context order
  int64_t next_ticket = 1;
  lazyattn_pool_stats st{};
};

namespace {

void evict_lru(lazyattn_pool* p) {
  const Key k = p->lru.front();
  p->lru.pop_front();
  auto it = p->cache.find(k);
  Entry& e = it->second;
  // returned so that the next allocation hands them out in their old order
  for (size_t j = e.blocks.size(); j-- > 0;) p->free_blocks.push_back(e.blocks[j]);
  p->st.blocks_in_use -= static_cast<int64_t>(e.blocks.size());
  p->st.evictions += 1;
  p->cache.erase(it);
}

void pin(lazyattn_pool* p, Entry& e) {
  if (e.pins == 0 && e.in_lru) {
    p->lru.erase(e.lru_pos);
    e.in_lru = false;
  }
  e.pins += 1;
}

bool docs_valid(const int64_t* ids, const int32_t* lens, int64_t n) {
  for (int64_t k = 0; k < n; ++k)
    if (ids[k] < 0 || lens[k] < 1) return false;
  return true;
}

lazyattn_status admit(lazyattn_pool* p, const int64_t* ids, const int32_t* lens, int32_t n, uint32_t* blocks,
                      uint32_t* starts, int32_t max_entries, int32_t* num_entries, uint8_t* status,
                      int64_t* ticket) {
  int64_t need = 0;
  for (int32_t k = 0; k < n; ++k) need += (lens[k] + 15) / 16;
  if (need > max_entries) return LAZYATTN_EWORKSPACE;
  std::vector<Key> pinned;
  pinned.reserve(n);
  int64_t pos = 0, parent = 0;
  int32_t ne = 0;
  bool chain = true;
  for (int32_t k = 0; k < n; ++k) {
    const int32_t len = lens[k];
    const size_t nb = static_cast<size_t>((len + 15) / 16);
    Key key{ids[k], 0};
    if (p->policy == LAZYATTN_CACHE_POSITION_AWARE) {
      key.b = pos;
    } else if (p->policy == LAZYATTN_CACHE_PREFIX) {
      const Key edge{parent, ids[k]};
      auto nit = p->prefix_nodes.find(edge);
      if (nit == p->prefix_nodes.end()) nit = p->prefix_nodes.emplace(edge, p->next_node++).first;
      parent = nit->second;
      key = Key{parent, 0};
    }
    p->st.doc_accesses += 1;
    p->st.token_accesses += len;
    uint8_t s;
    Entry* e = nullptr;
    auto it = p->cache.find(key);
    if (it != p->cache.end()) {
      e = &it->second;
      s = (p->policy == LAZYATTN_CACHE_PREFIX && !chain) ? LAZYATTN_DOC_MISS : LAZYATTN_DOC_HIT;
      pin(p, *e);
    } else {
      while (p->free_blocks.size() < nb && !p->lru.empty()) evict_lru(p);
      if (p->free_blocks.size() >= nb) {
        Entry fresh;
        fresh.blocks.resize(nb);
        for (size_t j = 0; j < nb; ++j) {
          fresh.blocks[j] = p->free_blocks.back();
          p->free_blocks.pop_back();
        }
        e = &p->cache.emplace(key, std::move(fresh)).first->second;
        e->pins = 1;
        p->st.blocks_in_use += static_cast<int64_t>(nb);
        p->st.inserts += 1;
        s = LAZYATTN_DOC_MISS;
      } else {
        p->st.bypasses += 1;
        s = LAZYATTN_DOC_BYPASS;
      }
    }
    if (s == LAZYATTN_DOC_HIT) {
      p->st.doc_hits += 1;
      p->st.token_hits += len;
    } else {
      chain = false;
    }
    if (e) {
      pinned.push_back(key);
      for (size_t j = 0; j < nb; ++j) {
        if (blocks) blocks[ne] = e->blocks[j];
        if (starts) starts[ne] = static_cast<uint32_t>(pos + 16 * static_cast<int64_t>(j));
        ++ne;
      }
    }
    if (status) status[k] = s;
    pos += len;
  }
  if (num_entries) *num_entries = ne;
  const int64_t t = p->next_ticket++;
  p->open.emplace(t, std::move(pinned));
  p->st.open_requests += 1;
  if (ticket) *ticket = t;
  return LAZYATTN_OK;
}

lazyattn_status release(lazyattn_pool* p, int64_t ticket) {
  auto it = p->open.find(ticket);
  if (it == p->open.end()) return LAZYATTN_EINVAL;
  for (const Key& k : it->second) {
    Entry& e = p->cache.find(k)->second;       // pinned entries are never evicted
    e.pins -= 1;
    if (e.pins == 0) {
      e.lru_pos = p->lru.insert(p->lru.end(), k);
      e.in_lru = true;
    }
  }
  p->open.erase(it);
  p->st.open_requests -= 1;
  return LAZYATTN_OK;
}

}  // namespace

extern "C" {

lazyattn_status lazyattn_pool_create(int64_t num_blocks, int32_t policy, lazyattn_pool** out) {
  if (!out || num_blocks < 0 || num_blocks > 0xffffffffLL) return LAZYATTN_EINVAL;
  if (policy != LAZYATTN_CACHE_POSITION_AGNOSTIC && policy != LAZYATTN_CACHE_POSITION_AWARE &&
      policy != LAZYATTN_CACHE_PREFIX)
    return LAZYATTN_EINVAL;
  lazyattn_pool* p = new (std::nothrow) lazyattn_pool();
  if (!p) return LAZYATTN_EINVAL;
  p->policy = policy;
  p->free_blocks.reserve(static_cast<size_t>(num_blocks));
  for (int64_t b = num_blocks; b-- > 0;) p->free_blocks.push_back(static_cast<uint32_t>(b));   // 0 first out
  p->st.num_blocks = num_blocks;
  *out = p;
  return LAZYATTN_OK;
}

void lazyattn_pool_destroy(lazyattn_pool* pool) { delete pool; }

lazyattn_status lazyattn_pool_admit(lazyattn_pool* pool, const int64_t* doc_ids, const int32_t* doc_lens,
                                    int32_t n_docs, uint32_t* blocks, uint32_t* starts, int32_t max_entries,
                                    int32_t* num_entries, uint8_t* doc_status, int64_t* ticket) {
  if (!pool || n_docs < 0 || max_entries < 0 || !ticket || !num_entries) return LAZYATTN_EINVAL;
  if (n_docs > 0 && (!doc_ids || !doc_lens || !doc_status)) return LAZYATTN_EINVAL;
  if (max_entries > 0 && (!blocks || !starts)) return LAZYATTN_EINVAL;
  if (!docs_valid(doc_ids, doc_lens, n_docs)) return LAZYATTN_EINVAL;
  return admit(pool, doc_ids, doc_lens, n_docs, blocks, starts, max_entries, num_entries, doc_status, ticket);
}

lazyattn_status lazyattn_pool_release(lazyattn_pool* pool, int64_t ticket) {
  if (!pool) return LAZYATTN_EINVAL;
  return release(pool, ticket);
}

lazyattn_status lazyattn_pool_get_stats(const lazyattn_pool* pool, lazyattn_pool_stats* out) {
  if (!pool || !out) return LAZYATTN_EINVAL;
  *out = pool->st;
  return LAZYATTN_OK;
}

lazyattn_status lazyattn_pool_run_trace(lazyattn_pool* pool, const int64_t* doc_ids, const int32_t* doc_lens,
                                        const int64_t* req_offsets, int64_t n_requests) {
  if (!pool || n_requests < 0 || (n_requests > 0 && (!req_offsets || !doc_ids || !doc_lens)))
    return LAZYATTN_EINVAL;
  if (n_requests == 0) return LAZYATTN_OK;
  if (req_offsets[0] != 0) return LAZYATTN_EINVAL;
  for (int64_t i = 0; i < n_requests; ++i) {
    const int64_t n = req_offsets[i + 1] - req_offsets[i];
    if (n < 0 || n > 0x7fffffff) return LAZYATTN_EINVAL;
  }
  if (!docs_valid(doc_ids, doc_lens, req_offsets[n_requests])) return LAZYATTN_EINVAL;
  for (int64_t i = 0; i < n_requests; ++i) {
    const int64_t a = req_offsets[i];
    const int32_t n = static_cast<int32_t>(req_offsets[i + 1] - a);
    int64_t t;
    int32_t ne;
    const lazyattn_status s =
        admit(pool, doc_ids + a, doc_lens + a, n, nullptr, nullptr, 0x7fffffff, &ne, nullptr, &t);
    if (s != LAZYATTN_OK) return s;
    release(pool, t);
  }
  return LAZYATTN_OK;
}

}  // extern "C"
