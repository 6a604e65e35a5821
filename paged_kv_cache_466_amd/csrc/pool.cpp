// Host block pool: FIFO free list of physical block ids with reference counts.
//
// "KV Cache Engineering for LLM Serving", section 10 "Paging": requests take
// blocks from the front of a shared free list and finished requests return
// theirs to the back.  "Chapter 18", "How PagedAttention Works": a new block
// is taken when the current one is full.  Learning-AI topic t13_4,
// copy-on-write paragraph: a block shared by several sequences is duplicated
// when one of them writes into it.
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

struct pkv_pool {
  std::deque<int32_t> free_list;
  std::vector<int32_t> refcount;
};

extern "C" pkv_pool* pkv_pool_create(int num_blocks, const int32_t* initial_order) {
  if (num_blocks < 0) {
    pkv::set_error("pkv_pool_create: num_blocks < 0");
    return nullptr;
  }
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) {
    pkv::set_error("pkv_pool_create: out of host memory");
    return nullptr;
  }
  p->refcount.assign(num_blocks, 0);
  if (initial_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      int32_t b = initial_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        pkv::set_error("pkv_pool_create: initial_order is not a permutation of 0..num_blocks-1");
        return nullptr;
      }
      seen[b] = 1;
      p->free_list.push_back(b);
    }
  } else {
    for (int i = 0; i < num_blocks; ++i) p->free_list.push_back(i);
  }
  return p;
}

extern "C" void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

extern "C" pkv_status pkv_pool_alloc(pkv_pool* pool, int32_t* block_out) {
  if (!pool || !block_out) return pkv::fail(PKV_EINVAL, "pkv_pool_alloc: null argument");
  if (pool->free_list.empty()) return pkv::fail(PKV_ENOMEM, "pkv_pool_alloc: block pool exhausted");
  int32_t b = pool->free_list.front();
  pool->free_list.pop_front();
  pool->refcount[b] = 1;
  *block_out = b;
  return PKV_OK;
}

static bool in_use(const pkv_pool* pool, int32_t b) {
  return b >= 0 && b < (int32_t)pool->refcount.size() && pool->refcount[b] > 0;
}

extern "C" pkv_status pkv_pool_incref(pkv_pool* pool, int32_t block) {
  if (!pool) return pkv::fail(PKV_EINVAL, "pkv_pool_incref: null pool");
  if (!in_use(pool, block)) return pkv::fail(PKV_EINVAL, "pkv_pool_incref: block is free or out of range");
  pool->refcount[block] += 1;
  return PKV_OK;
}

extern "C" pkv_status pkv_pool_decref(pkv_pool* pool, int32_t block) {
  if (!pool) return pkv::fail(PKV_EINVAL, "pkv_pool_decref: null pool");
  if (!in_use(pool, block)) return pkv::fail(PKV_EINVAL, "pkv_pool_decref: block is free or out of range");
  if (--pool->refcount[block] == 0) pool->free_list.push_back(block);
  return PKV_OK;
}

extern "C" int32_t pkv_pool_refcount(const pkv_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= (int32_t)pool->refcount.size()) return -1;
  return pool->refcount[block];
}

extern "C" pkv_status pkv_pool_allocate_sequence(pkv_pool* pool, int32_t num_tokens, int block_size,
                                                 int32_t* table_out, int32_t table_capacity, int32_t* n_out) {
  if (!pool || !n_out) return pkv::fail(PKV_EINVAL, "pkv_pool_allocate_sequence: null argument");
  if (block_size <= 0 || num_tokens < 0 || table_capacity < 0)
    return pkv::fail(PKV_EINVAL, "pkv_pool_allocate_sequence: bad block_size, num_tokens or capacity");
  const int64_t n = ((int64_t)num_tokens + block_size - 1) / block_size;
  if (n > table_capacity) return pkv::fail(PKV_EINVAL, "pkv_pool_allocate_sequence: table capacity exceeded");
  if (n > 0 && !table_out) return pkv::fail(PKV_EINVAL, "pkv_pool_allocate_sequence: null table");
  if (n > (int64_t)pool->free_list.size())
    return pkv::fail(PKV_ENOMEM, "pkv_pool_allocate_sequence: %lld blocks needed, %zu free", (long long)n,
                     pool->free_list.size());
  for (int64_t i = 0; i < n; ++i) {
    const int32_t b = pool->free_list.front();
    pool->free_list.pop_front();
    pool->refcount[b] = 1;
    table_out[i] = b;
  }
  *n_out = (int32_t)n;
  return PKV_OK;
}

// Occurrences of each block in table[0 .. n) that is in use; false when some
// entry is free or out of range.
static bool count_in_use(const pkv_pool* pool, const int32_t* table, int32_t n,
                         std::unordered_map<int32_t, int32_t>& uses) {
  for (int32_t i = 0; i < n; ++i) {
    if (!in_use(pool, table[i])) return false;
    ++uses[table[i]];
  }
  return true;
}

extern "C" pkv_status pkv_pool_fork(pkv_pool* pool, const int32_t* table, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !table)) return pkv::fail(PKV_EINVAL, "pkv_pool_fork: bad argument");
  std::unordered_map<int32_t, int32_t> uses;
  if (!count_in_use(pool, table, n, uses)) return pkv::fail(PKV_EINVAL, "pkv_pool_fork: table names a free block");
  for (int32_t i = 0; i < n; ++i) pool->refcount[table[i]] += 1;
  return PKV_OK;
}

extern "C" pkv_status pkv_pool_release(pkv_pool* pool, const int32_t* table, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !table)) return pkv::fail(PKV_EINVAL, "pkv_pool_release: bad argument");
  std::unordered_map<int32_t, int32_t> uses;
  if (!count_in_use(pool, table, n, uses))
    return pkv::fail(PKV_EINVAL, "pkv_pool_release: table names a free block");
  for (const auto& kv : uses)
    if (pool->refcount[kv.first] < kv.second)
      return pkv::fail(PKV_EINVAL, "pkv_pool_release: block %d listed more often than it is referenced", kv.first);
  // in table order, so that blocks freed here reach the back of the free
  // list in that order
  for (int32_t i = 0; i < n; ++i)
    if (--pool->refcount[table[i]] == 0) pool->free_list.push_back(table[i]);
  return PKV_OK;
}

extern "C" pkv_status pkv_pool_append(pkv_pool* pool, int32_t* table, int32_t table_capacity,
                                      int32_t* table_len, int32_t seq_len, int block_size,
                                      int32_t* slot_out, int32_t* cow_src, int32_t* cow_dst) {
  if (!pool || !table || !table_len || !slot_out || !cow_src || !cow_dst)
    return pkv::fail(PKV_EINVAL, "pkv_pool_append: null argument");
  if (block_size <= 0 || seq_len < 0) return pkv::fail(PKV_EINVAL, "pkv_pool_append: bad block_size or seq_len");
  const int32_t n = *table_len;
  if (n != (seq_len + block_size - 1) / block_size)
    return pkv::fail(PKV_EINVAL, "pkv_pool_append: table length does not cover seq_len tokens");
  *cow_src = -1;
  *cow_dst = -1;
  const int32_t logical = seq_len / block_size;
  const int32_t offset = seq_len % block_size;
  if (offset == 0) {
    // the last block is full (or the sequence is empty): take a new block
    if (n >= table_capacity) return pkv::fail(PKV_EINVAL, "pkv_pool_append: table capacity exceeded");
    int32_t b;
    pkv_status st = pkv_pool_alloc(pool, &b);
    if (st != PKV_OK) return st;
    table[n] = b;
    *table_len = n + 1;
  } else {
    int32_t b = table[logical];
    if (!in_use(pool, b)) return pkv::fail(PKV_EINVAL, "pkv_pool_append: table names a free block");
    if (pool->refcount[b] > 1) {
      // copy-on-write: the writer gets its own copy of the shared block
      int32_t nb;
      pkv_status st = pkv_pool_alloc(pool, &nb);
      if (st != PKV_OK) return st;
      pool->refcount[b] -= 1;
      table[logical] = nb;
      *cow_src = b;
      *cow_dst = nb;
    }
  }
  *slot_out = table[logical] * block_size + offset;
  return PKV_OK;
}

extern "C" pkv_status pkv_pool_stats(const pkv_pool* pool, int32_t* free_blocks, int32_t* used_blocks,
                                     int32_t* shared_blocks) {
  if (!pool) return pkv::fail(PKV_EINVAL, "pkv_pool_stats: null pool");
  int32_t used = 0, shared = 0;
  for (int32_t r : pool->refcount) {
    used += r > 0;
    shared += r > 1;
  }
  if (free_blocks) *free_blocks = (int32_t)pool->free_list.size();
  if (used_blocks) *used_blocks = used;
  if (shared_blocks) *shared_blocks = shared;
  return PKV_OK;
}

extern "C" pkv_status pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n) {
  if (!pool || !n) return pkv::fail(PKV_EINVAL, "pkv_pool_free_list: null argument");
  int32_t i = 0;
  for (int32_t b : pool->free_list) {
    if (i < cap && out) out[i] = b;
    ++i;
  }
  *n = i;
  return PKV_OK;
}
