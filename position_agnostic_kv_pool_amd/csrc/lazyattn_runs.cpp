// Host half of the shared-run decode: cutting a decode batch's tables into
// runs of entries that recur in several requests, and the work items over
// them (lazyattn_decode_runs_plan).  Nothing here touches a GPU.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <unordered_map>
#include <utility>
#include <vector>

#include "lazyattn_common.hpp"

namespace lazyattn {
namespace {

constexpr int kRunPiece = 64;   // entries per work item over a shared run at most
constexpr int kOwnPiece = 32;   // entries per work item over one request's unshared entries at most
constexpr int kXcds = 8;        // round-robin dispatch spreads consecutive work-group ids over 8 XCDs

struct Run {
  std::vector<uint32_t> blocks;
  int last_len = 0;
  std::vector<std::pair<int, int>> occ;   // (request, index of the run's first entry in its table)
};

struct Item {
  int word_begin, n_entries;
  std::vector<std::pair<int, int>> refs;  // (request, p - s)
};

}  // namespace

// An entry's identity for sharing: its block and valid length (a block used
// with two lengths forms two keys, so a run's entries read alike everywhere).
static inline uint64_t entry_key(uint32_t block, int len) {
  return (static_cast<uint64_t>(block) << 5) | static_cast<uint64_t>(len);
}

// An item's entry: block id in bits 31..0, key offset in bits 58..32, valid
// length (1..16) in bits 63..59.
static inline uint64_t item_word(uint32_t block, int offset, int len) {
  return static_cast<uint64_t>(block) | (static_cast<uint64_t>(offset) << 32) | (static_cast<uint64_t>(len) << 59);
}

static lazyattn_status build_run_items(const lazyattn_config* cfg, const uint64_t* tables, int R, int E,
                                       const int32_t* ne, const int32_t* ctx, std::vector<Item>& items,
                                       std::vector<uint64_t>& words) {
  auto entry_len = [&](int r, int e) -> int {
    const uint64_t* row = tables + static_cast<int64_t>(r) * E;
    const int64_t end = (e + 1 < ne[r]) ? static_cast<int64_t>(word_start(row[e + 1])) : ctx[r];
    return static_cast<int>(end - static_cast<int64_t>(word_start(row[e])));
  };
  auto key_of = [&](int r, int e) { return entry_key(word_block(tables[static_cast<int64_t>(r) * E + e]), entry_len(r, e)); };

  // every occurrence of every key, in (request, entry) order
  std::unordered_map<uint64_t, std::vector<std::pair<int, int>>> occ;
  for (int r = 0; r < R; ++r)
    for (int e = 0; e < ne[r]; ++e) occ[key_of(r, e)].emplace_back(r, e);

  // runs, in the order their first occurrence is met: a run grows while every
  // occurrence of its last entry is a whole block followed by the same next key,
  // and that key occurs nowhere else
  std::unordered_map<uint64_t, char> seen;
  std::vector<Run> runs;
  for (int r = 0; r < R; ++r) {
    for (int e = 0; e < ne[r]; ++e) {
      const uint64_t k = key_of(r, e);
      if (seen.count(k)) continue;
      seen[k] = 1;
      Run run;
      run.occ = occ[k];
      run.blocks.push_back(word_block(tables[static_cast<int64_t>(r) * E + e]));
      std::vector<std::pair<int, int>> cur = run.occ;
      for (;;) {
        bool ok = true;
        for (const auto& o : cur)
          if (entry_len(o.first, o.second) != kBlock || o.second + 1 >= ne[o.first]) {
            ok = false;
            break;
          }
        if (!ok) break;
        const uint64_t nk = key_of(cur[0].first, cur[0].second + 1);
        for (const auto& o : cur)
          if (key_of(o.first, o.second + 1) != nk) {
            ok = false;
            break;
          }
        if (!ok || seen.count(nk) || occ[nk].size() != cur.size()) break;
        seen[nk] = 1;
        for (auto& o : cur) ++o.second;
        run.blocks.push_back(word_block(tables[static_cast<int64_t>(cur[0].first) * E + cur[0].second]));
      }
      run.last_len = entry_len(cur[0].first, cur[0].second);
      runs.push_back(std::move(run));
    }
  }

  // Work items.  A run held by two or more occurrences is cut into pieces of at
  // most kRunPiece entries, each attended once per group of at most 16 / G
  // occurrences, with key offsets counted from the piece's first key; all items
  // of one piece go to the XCD queue with the least work so far.  The entries of
  // runs held once are gathered per request, in table order, into pieces of at
  // most kOwnPiece entries with one occurrence each and key offsets counted
  // from position 0 (their query turns by R(p)).
  const int per_item = std::max(1, 16 / (cfg->num_q_heads / cfg->num_kv_heads));
  std::vector<std::vector<Item>> queue(kXcds);
  std::vector<long long> load(kXcds, 0);
  auto least = [&]() { return static_cast<int>(std::min_element(load.begin(), load.end()) - load.begin()); };
  std::vector<std::vector<uint64_t>> own(static_cast<size_t>(R));   // (block, start, length) words
  for (const Run& run : runs) {
    const int n = static_cast<int>(run.blocks.size());
    if (run.occ.size() == 1) {
      const int rq = run.occ[0].first, e0 = run.occ[0].second;
      for (int k = 0; k < n; ++k) {
        const uint32_t s = word_start(tables[static_cast<int64_t>(rq) * E + e0 + k]);
        if (s >= (1u << 27)) return LAZYATTN_EUNSUPPORTED;   // past the word's offset field
        own[rq].push_back(item_word(run.blocks[k], static_cast<int>(s), k + 1 < n ? kBlock : run.last_len));
      }
      continue;
    }
    for (int c0 = 0; c0 < n; c0 += kRunPiece) {
      const int c1 = std::min(n, c0 + kRunPiece);
      const int word_begin = static_cast<int>(words.size());
      for (int k = c0; k < c1; ++k)
        words.push_back(item_word(run.blocks[k], kBlock * (k - c0), k + 1 < n ? kBlock : run.last_len));
      const int x = least();
      const int n_occ = static_cast<int>(run.occ.size());
      for (int j0 = 0; j0 < n_occ; j0 += per_item) {
        Item it;
        it.word_begin = word_begin;
        it.n_entries = c1 - c0;
        for (int j = j0; j < std::min(n_occ, j0 + per_item); ++j) {
          const int rq = run.occ[j].first;
          const int s = static_cast<int>(word_start(tables[static_cast<int64_t>(rq) * E + run.occ[j].second + c0]));
          it.refs.emplace_back(rq, (ctx[rq] - 1) - s);
        }
        load[x] += c1 - c0;
        queue[x].push_back(std::move(it));
      }
    }
  }
  for (int r = 0; r < R; ++r) {
    const int n = static_cast<int>(own[r].size());
    for (int c0 = 0; c0 < n; c0 += kOwnPiece) {
      const int c1 = std::min(n, c0 + kOwnPiece);
      Item it;
      it.word_begin = static_cast<int>(words.size());
      it.n_entries = c1 - c0;
      words.insert(words.end(), own[r].begin() + c0, own[r].begin() + c1);
      it.refs.emplace_back(r, ctx[r] - 1);
      const int x = least();
      load[x] += c1 - c0;
      queue[x].push_back(std::move(it));
    }
  }
  // A work-group takes four items, one per wave, and work-group m runs on XCD
  // m % 8: queue x's items 4 k .. 4 k + 3 form work-group 8 k + x.  The queues
  // are first evened out to a common length, a multiple of 4 (items past it
  // move from the back of the longer queues to the shorter ones; the rest is
  // padded with empty items), and each is ordered by size, longest first, so
  // that the four waves of a work-group carry similar work.
  size_t total = 0;
  for (const auto& q : queue) total += q.size();
  const size_t per = ((total + kXcds - 1) / kXcds + 3) / 4 * 4;
  std::vector<Item> spill;
  for (auto& q : queue)
    while (q.size() > per) {
      spill.push_back(std::move(q.back()));
      q.pop_back();
    }
  for (auto& q : queue)
    while (q.size() < per && !spill.empty()) {
      q.push_back(std::move(spill.back()));
      spill.pop_back();
    }
  for (auto& q : queue)
    std::stable_sort(q.begin(), q.end(), [](const Item& a, const Item& b) { return a.n_entries > b.n_entries; });
  items.clear();
  for (size_t k = 0; k < per; k += 4)
    for (int x = 0; x < kXcds; ++x)
      for (size_t w = 0; w < 4; ++w) {
        if (k + w < queue[x].size()) {
          items.push_back(std::move(queue[x][k + w]));
        } else {
          Item empty{0, 0, {}};
          items.push_back(std::move(empty));
        }
      }
  return LAZYATTN_OK;
}

}  // namespace lazyattn

using namespace lazyattn;

extern "C" {

lazyattn_status lazyattn_decode_runs_plan(const lazyattn_config* cfg, const uint64_t* tables_h, int32_t num_reqs,
                                          int32_t max_entries, const int32_t* num_entries_h,
                                          const int32_t* ctx_lens_h, int64_t num_blocks, int32_t capacity_items,
                                          int32_t capacity_words, int32_t capacity_refs, int32_t* items_h,
                                          uint64_t* words_h, int32_t* refs_h, int32_t* req_ref_begin_h,
                                          int32_t* req_refs_h, int32_t* num_items, int32_t* num_words,
                                          int32_t* num_refs) {
  if (!num_items || !num_words || !num_refs) return LAZYATTN_EINVAL;
  *num_items = *num_words = *num_refs = 0;
  int32_t bad_r = -1, bad_e = -1;
  lazyattn_status st = lazyattn_validate_tables(cfg, tables_h, num_reqs, max_entries, num_entries_h, ctx_lens_h,
                                                num_blocks, &bad_r, &bad_e);
  if (st != LAZYATTN_OK) return st;
  if (cfg->dtype != LAZYATTN_BF16 || cfg->num_q_heads / cfg->num_kv_heads > 16) return LAZYATTN_EUNSUPPORTED;
  std::vector<Item> items;
  std::vector<uint64_t> words;
  st = build_run_items(cfg, tables_h, num_reqs, max_entries, num_entries_h, ctx_lens_h, items, words);
  if (st != LAZYATTN_OK) return st;
  long long n_refs = 0;
  for (const Item& it : items) n_refs += static_cast<long long>(it.refs.size());
  if (items.size() > 0x7fffffffULL || words.size() > 0x7fffffffULL || n_refs > 0x7fffffffLL)
    return LAZYATTN_EUNSUPPORTED;
  *num_items = static_cast<int32_t>(items.size());
  *num_words = static_cast<int32_t>(words.size());
  *num_refs = static_cast<int32_t>(n_refs);
  if (capacity_items < *num_items || capacity_words < *num_words || capacity_refs < *num_refs) return LAZYATTN_EWORKSPACE;
  if ((*num_items > 0 && !items_h) || (*num_words > 0 && !words_h) || (*num_refs > 0 && (!refs_h || !req_refs_h)) ||
      (num_reqs > 0 && !req_ref_begin_h))
    return LAZYATTN_EINVAL;
  std::vector<int32_t> count(static_cast<size_t>(num_reqs) + 1, 0);
  int32_t ref = 0;
  for (size_t i = 0; i < items.size(); ++i) {
    const Item& it = items[i];
    int32_t* row = items_h + i * LAZYATTN_RUN_ITEM_INTS;
    row[0] = it.word_begin;
    row[1] = it.n_entries;
    row[2] = ref;
    row[3] = static_cast<int32_t>(it.refs.size());
    for (const auto& o : it.refs) {
      refs_h[2 * ref] = o.first;
      refs_h[2 * ref + 1] = o.second;
      ++count[static_cast<size_t>(o.first) + 1];
      ++ref;
    }
  }
  std::copy(words.begin(), words.end(), words_h);
  for (int32_t r = 0; r < num_reqs; ++r) count[static_cast<size_t>(r) + 1] += count[r];
  if (num_reqs >= 0 && req_ref_begin_h) std::copy(count.begin(), count.end(), req_ref_begin_h);
  std::vector<int32_t> fill(count.begin(), count.end() - 1);
  for (int32_t k = 0; k < ref; ++k) req_refs_h[fill[refs_h[2 * k]]++] = k;
  return LAZYATTN_OK;
}

size_t lazyattn_decode_runs_workspace_size(const lazyattn_config* cfg, int32_t num_refs) {
  if (check_config(cfg) != LAZYATTN_OK || num_refs < 0) return 0;
  const size_t rows = static_cast<size_t>(num_refs) * cfg->num_q_heads;
  return rows * (static_cast<size_t>(cfg->head_dim) * sizeof(uint16_t) + 2 * sizeof(float));
}

}  // extern "C"
