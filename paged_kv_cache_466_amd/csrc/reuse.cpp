// Host-side block reuse: a prefix cache over the block pool, and the H2O
// retention rule.
//
// "KV Cache Engineering for LLM Serving", section 11 "Prefix reuse": a
// completed block is stored under a key made of the whole token prefix up to
// its end, so a block is shared only when everything before it matches too.
// Here the key is kept as a chain: an entry is (its parent entry, the
// block's own tokens), and a lookup walks the chain from the root, comparing
// the tokens in full - the same keys as whole prefixes, with no false match
// and no hash collisions.  The cache holds one pool reference per cached
// block; a lookup hands the caller one more reference per matched block.
// Eviction drops least-recently-used entries that have no cached children
// and whose block nobody else holds.
//
// Section 9 "Eviction" (H2O): under a budget of positions the latest ones
// are kept, and the rest of the budget goes to the older positions with the
// largest accumulated attention scores; equal scores keep the earlier
// position.
#include <algorithm>
#include <cstring>
#include <map>
#include <new>
#include <numeric>
#include <utility>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

struct pkv_prefix_cache {
  struct Entry {
    int32_t block;
    int parent;                   // entry index, -1 for the root
    std::vector<int32_t> tokens;  // the block's own tokens
    uint64_t last_use;
    int children;                 // cached entries under this one
    bool live;
  };
  pkv_pool* pool;
  int block_size;
  uint64_t clock = 0;
  std::vector<Entry> entries;     // entry 0 is the root (no block)
  std::vector<int> free_slots;
  std::map<std::pair<int, std::vector<int32_t>>, int> child;   // (parent, tokens) -> entry
  int live_count = 0;
};

namespace {

int find_child(const pkv_prefix_cache* c, int parent, const int32_t* tokens) {
  std::vector<int32_t> key(tokens, tokens + c->block_size);
  auto it = c->child.find({parent, key});
  return it == c->child.end() ? -1 : it->second;
}

}  // namespace

extern "C" pkv_prefix_cache* pkv_prefix_cache_create(pkv_pool* pool, int block_size) {
  if (!pool || block_size <= 0) {
    pkv::set_error("pkv_prefix_cache_create: null pool or block_size <= 0");
    return nullptr;
  }
  pkv_prefix_cache* c = new (std::nothrow) pkv_prefix_cache;
  if (!c) {
    pkv::set_error("pkv_prefix_cache_create: out of host memory");
    return nullptr;
  }
  c->pool = pool;
  c->block_size = block_size;
  c->entries.push_back({-1, -1, {}, 0, 0, true});
  return c;
}

extern "C" void pkv_prefix_cache_destroy(pkv_prefix_cache* c) {
  if (!c) return;
  for (size_t i = 1; i < c->entries.size(); ++i)
    if (c->entries[i].live) (void)pkv_pool_decref(c->pool, c->entries[i].block);
  delete c;
}

extern "C" pkv_status pkv_prefix_cache_match(pkv_prefix_cache* c, const int32_t* tokens, int n_tokens,
                                             int32_t* blocks_out, int max_blocks, int* n_matched) {
  if (!c || !n_matched || n_tokens < 0 || max_blocks < 0 || (n_tokens > 0 && !tokens) ||
      (max_blocks > 0 && !blocks_out))
    return pkv::fail(PKV_EINVAL, "pkv_prefix_cache_match: bad argument");
  *n_matched = 0;
  const uint64_t now = ++c->clock;
  int node = 0;
  const int full = n_tokens / c->block_size;
  for (int b = 0; b < full && b < max_blocks; ++b) {
    const int e = find_child(c, node, tokens + (size_t)b * c->block_size);
    if (e < 0) break;
    pkv_status st = pkv_pool_incref(c->pool, c->entries[e].block);
    if (st != PKV_OK) return st;
    c->entries[e].last_use = now;
    blocks_out[b] = c->entries[e].block;
    ++*n_matched;
    node = e;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_prefix_cache_insert(pkv_prefix_cache* c, const int32_t* tokens, int n_tokens,
                                              const int32_t* blocks, int n_blocks, int* n_added) {
  if (!c || n_tokens < 0 || n_blocks < 0 || (n_tokens > 0 && !tokens) || (n_blocks > 0 && !blocks))
    return pkv::fail(PKV_EINVAL, "pkv_prefix_cache_insert: bad argument");
  int added = 0;
  const uint64_t now = ++c->clock;
  int node = 0;
  const int full = n_tokens / c->block_size;
  for (int b = 0; b < full && b < n_blocks; ++b) {
    const int32_t* tk = tokens + (size_t)b * c->block_size;
    int e = find_child(c, node, tk);
    if (e < 0) {
      // a new entry: the cache takes a reference to the caller's block
      pkv_status st = pkv_pool_incref(c->pool, blocks[b]);
      if (st != PKV_OK) {
        if (n_added) *n_added = added;
        return st;
      }
      pkv_prefix_cache::Entry en{blocks[b], node, std::vector<int32_t>(tk, tk + c->block_size), now, 0, true};
      if (!c->free_slots.empty()) {
        e = c->free_slots.back();
        c->free_slots.pop_back();
        c->entries[e] = std::move(en);
      } else {
        e = (int)c->entries.size();
        c->entries.push_back(std::move(en));
      }
      c->child[{node, c->entries[e].tokens}] = e;
      c->entries[node].children++;
      c->live_count++;
      ++added;
    } else {
      c->entries[e].last_use = now;
    }
    node = e;
  }
  if (n_added) *n_added = added;
  return PKV_OK;
}

extern "C" pkv_status pkv_prefix_cache_evict(pkv_prefix_cache* c, int n_wanted, int* n_evicted) {
  if (!c || n_wanted < 0) return pkv::fail(PKV_EINVAL, "pkv_prefix_cache_evict: bad argument");
  int done = 0;
  while (done < n_wanted) {
    // the least recently used leaf whose block only the cache holds
    int best = -1;
    for (size_t i = 1; i < c->entries.size(); ++i) {
      const auto& e = c->entries[i];
      if (!e.live || e.children != 0 || pkv_pool_refcount(c->pool, e.block) != 1) continue;
      if (best < 0 || e.last_use < c->entries[best].last_use) best = (int)i;
    }
    if (best < 0) break;
    auto& e = c->entries[best];
    pkv_status st = pkv_pool_decref(c->pool, e.block);
    if (st != PKV_OK) return st;
    c->child.erase({e.parent, e.tokens});
    c->entries[e.parent].children--;
    e.live = false;
    e.tokens.clear();
    c->free_slots.push_back(best);
    c->live_count--;
    ++done;
  }
  if (n_evicted) *n_evicted = done;
  return PKV_OK;
}

extern "C" int pkv_prefix_cache_size(const pkv_prefix_cache* c) { return c ? c->live_count : -1; }

extern "C" pkv_status pkv_h2o_retain(const float* scores, int n, int budget, int recent_count, int32_t* kept_out,
                                     int* n_kept) {
  if (n < 0 || budget < 0 || recent_count < 0 || !n_kept || (n > 0 && (!scores || !kept_out)))
    return pkv::fail(PKV_EINVAL, "pkv_h2o_retain: bad argument");
  for (int i = 0; i < n; ++i)
    if (scores[i] != scores[i]) return pkv::fail(PKV_EINVAL, "pkv_h2o_retain: NaN score at %d", i);
  if (budget >= n) {
    for (int i = 0; i < n; ++i) kept_out[i] = i;
    *n_kept = n;
    return PKV_OK;
  }
  const int r = std::min(recent_count, budget);
  const int older = n - r;
  std::vector<int32_t> idx(older);
  std::iota(idx.begin(), idx.end(), 0);
  // largest score first, earlier position first among equal scores
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return scores[a] > scores[b]; });
  idx.resize(budget - r);
  for (int i = older; i < n; ++i) idx.push_back(i);
  std::sort(idx.begin(), idx.end());
  std::copy(idx.begin(), idx.end(), kept_out);
  *n_kept = (int)idx.size();
  return PKV_OK;
}
