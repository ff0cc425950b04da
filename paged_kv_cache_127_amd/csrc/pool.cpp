// Host block pool: free list + reference counts, and block-table helpers for one sequence.
//
// "PagedAttention: Virtual Memory for the KV Cache": a request takes one more block only when
// a token enters a new logical block ("Growing a request"); sharers of a partially filled
// block get a private copy before writing ("Sharing a prefix and copying a partial block").
// "KV Cache Optimization and Management": a block goes back to the free pool only when its
// reference count reaches zero (answer A6).
// Allocation order is not fixed by the pages; the pool hands out the lowest free id.
#include <cstdio>
#include <new>
#include <set>
#include <vector>

#include "pagedkv.h"

struct pkv_pool {
  std::vector<int32_t> ref;
  std::set<int32_t> free_ids;
};

namespace {
bool in_range(const pkv_pool* p, int32_t b) { return b >= 0 && (size_t)b < p->ref.size(); }
}  // namespace

extern "C" {

pkv_pool* pkv_pool_create(int num_blocks) {
  if (num_blocks <= 0) return nullptr;
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return nullptr;
  try {
    p->ref.assign((size_t)num_blocks, 0);
    for (int32_t b = 0; b < num_blocks; ++b) p->free_ids.insert(p->free_ids.end(), b);
  } catch (...) {
    delete p;
    return nullptr;
  }
  return p;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

int pkv_pool_alloc(pkv_pool* pool, int32_t* out_block) {
  if (!pool || !out_block) return PKV_ERR_INVALID_ARG;
  if (pool->free_ids.empty()) return PKV_ERR_POOL_EXHAUSTED;
  const int32_t b = *pool->free_ids.begin();
  pool->free_ids.erase(pool->free_ids.begin());
  pool->ref[b] = 1;
  *out_block = b;
  return PKV_OK;
}

int pkv_pool_claim(pkv_pool* pool, int32_t block) {
  if (!pool || !in_range(pool, block)) return PKV_ERR_INVALID_ARG;
  if (pool->ref[block] != 0) return PKV_ERR_REFCOUNT;
  pool->free_ids.erase(block);
  pool->ref[block] = 1;
  return PKV_OK;
}

int pkv_pool_incref(pkv_pool* pool, int32_t block) {
  if (!pool || !in_range(pool, block)) return PKV_ERR_INVALID_ARG;
  if (pool->ref[block] == 0) return PKV_ERR_REFCOUNT;
  ++pool->ref[block];
  return PKV_OK;
}

int pkv_pool_decref(pkv_pool* pool, int32_t block, int* freed) {
  if (!pool || !in_range(pool, block)) return PKV_ERR_INVALID_ARG;
  if (pool->ref[block] == 0) return PKV_ERR_REFCOUNT;
  const bool now_free = --pool->ref[block] == 0;
  if (now_free) pool->free_ids.insert(block);
  if (freed) *freed = now_free ? 1 : 0;
  return PKV_OK;
}

int pkv_pool_refcount(const pkv_pool* pool, int32_t block) {
  if (!pool || !in_range(pool, block)) return PKV_ERR_INVALID_ARG;
  return pool->ref[block];
}

int pkv_pool_num_free(const pkv_pool* pool) {
  if (!pool) return PKV_ERR_INVALID_ARG;
  return (int)pool->free_ids.size();
}

int pkv_seq_prepare_write(pkv_pool* pool, int32_t* table_row, int max_blocks, int length,
                          int block_size, int32_t* block, int32_t* offset, int32_t* cow_src,
                          int32_t* cow_dst, int32_t* cow_n) {
  if (!pool || !table_row || !block || !offset || !cow_src || !cow_dst || !cow_n ||
      max_blocks <= 0 || length < 0 || block_size <= 0)
    return PKV_ERR_INVALID_ARG;
  const int j = length / block_size;
  const int r = length % block_size;
  if (j >= max_blocks) return PKV_ERR_INVALID_ARG;
  *cow_src = *cow_dst = -1;
  *cow_n = -1;
  if (r == 0) {
    // a new logical block: an entry the caller already placed (>= 0, live) is kept
    const int32_t pre = table_row[j];
    if (!(in_range(pool, pre) && pool->ref[pre] > 0)) {
      int32_t b;
      const int rc = pkv_pool_alloc(pool, &b);
      if (rc != PKV_OK) return rc;
      table_row[j] = b;
    }
  } else {
    const int32_t old = table_row[j];
    if (!in_range(pool, old) || pool->ref[old] == 0) return PKV_ERR_REFCOUNT;
    if (pool->ref[old] > 1) {
      int32_t b;
      const int rc = pkv_pool_alloc(pool, &b);
      if (rc != PKV_OK) return rc;
      table_row[j] = b;
      --pool->ref[old];   // > 0 remains: another sequence still holds it
      *cow_src = old;
      *cow_dst = b;
      *cow_n = r;
    }
  }
  *block = table_row[j];
  *offset = r;
  return PKV_OK;
}

int pkv_seq_fork(pkv_pool* pool, const int32_t* src_row, int32_t* dst_row, int num_blocks_used) {
  if (!pool || !src_row || !dst_row || num_blocks_used < 0) return PKV_ERR_INVALID_ARG;
  for (int j = 0; j < num_blocks_used; ++j)
    if (!in_range(pool, src_row[j]) || pool->ref[src_row[j]] == 0) return PKV_ERR_REFCOUNT;
  for (int j = 0; j < num_blocks_used; ++j) {
    ++pool->ref[src_row[j]];
    dst_row[j] = src_row[j];
  }
  return PKV_OK;
}

int pkv_seq_release(pkv_pool* pool, const int32_t* table_row, int num_blocks_used) {
  if (!pool || !table_row || num_blocks_used < 0) return PKV_ERR_INVALID_ARG;
  for (int j = 0; j < num_blocks_used; ++j)
    if (!in_range(pool, table_row[j]) || pool->ref[table_row[j]] == 0) return PKV_ERR_REFCOUNT;
  int freed = 0;
  for (int j = 0; j < num_blocks_used; ++j) {
    int f = 0;
    pkv_pool_decref(pool, table_row[j], &f);
    freed += f;
  }
  return freed;
}

}  // extern "C"
