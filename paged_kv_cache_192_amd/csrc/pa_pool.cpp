// Host block pool: a stack of free physical block ids plus a reference count
// per block.  Sequences take blocks one at a time as they grow and give
// them back when they finish or are cancelled; a shared prefix is held by
// several sequences at once and returns to the pool when the last one lets
// go ("Cache KV en production", section on paging; glossary "PagedAttention
// & Gestion du KV-Cache", sections 3 and 4).
#include <cstdint>
#include <new>
#include <vector>

#include "pa_internal.h"

struct pa_pool {
  int32_t num_blocks;
  std::vector<int32_t> free_stack;  // top = back(): the next id handed out
  std::vector<int32_t> refcount;
  std::vector<int32_t> scratch;     // per-call occurrence counts (all zero between calls)
};

using pa::fail;

extern "C" {

pa_status pa_pool_create(int32_t num_blocks, const int32_t* initial_order, pa_pool** out) {
  if (!out) return fail(PA_ERR_INVALID, "pa_pool_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0) return fail(PA_ERR_INVALID, "pa_pool_create: num_blocks must be positive");
  pa_pool* p = new (std::nothrow) pa_pool;
  if (!p) return fail(PA_ERR_OOM, "pa_pool_create: host allocation failed");
  try {
    p->num_blocks = num_blocks;
    p->refcount.assign(num_blocks, 0);
    p->scratch.assign(num_blocks, 0);
    p->free_stack.resize(num_blocks);
    if (initial_order) {
      // must be a permutation of 0..num_blocks-1
      for (int32_t i = 0; i < num_blocks; ++i) {
        int32_t id = initial_order[i];
        if (id < 0 || id >= num_blocks || p->scratch[id]) {
          delete p;
          return fail(PA_ERR_INVALID, "pa_pool_create: initial_order is not a permutation of 0..%d",
                      num_blocks - 1);
        }
        p->scratch[id] = 1;
      }
      for (int32_t i = 0; i < num_blocks; ++i) p->scratch[i] = 0;
    }
    // the first id handed out is initial_order[0], so it sits on top
    for (int32_t i = 0; i < num_blocks; ++i)
      p->free_stack[num_blocks - 1 - i] = initial_order ? initial_order[i] : i;
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(PA_ERR_OOM, "pa_pool_create: host allocation failed");
  }
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool* p) { delete p; }

pa_status pa_block_alloc(pa_pool* p, int32_t n, int32_t* out_ids) {
  if (!p) return fail(PA_ERR_INVALID, "pa_block_alloc: pool is NULL");
  if (n < 0) return fail(PA_ERR_INVALID, "pa_block_alloc: n < 0");
  if (n == 0) return PA_OK;
  if (!out_ids) return fail(PA_ERR_INVALID, "pa_block_alloc: out_ids is NULL");
  if ((size_t)n > p->free_stack.size())
    return fail(PA_ERR_OOM, "pa_block_alloc: %d blocks asked, %zu free", n, p->free_stack.size());
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = p->free_stack.back();
    p->free_stack.pop_back();
    p->refcount[id] = 1;
    out_ids[i] = id;
  }
  return PA_OK;
}

// Checks the whole call before anything changes.  need_held: each id must be
// held at least as many times as it occurs (free); otherwise each id must be
// held at all (share).
static pa_status validate(pa_pool* p, int32_t n, const int32_t* ids, bool need_held, const char* fn) {
  // range first, so an id outside the pool is reported before any state error
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= p->num_blocks)
      return fail(PA_ERR_INVALID, "%s: block id %d outside [0, %d)", fn, ids[i], p->num_blocks);
  pa_status st = PA_OK;
  int32_t i = 0;
  for (; i < n; ++i) {
    const int32_t id = ids[i];
    const int32_t c = ++p->scratch[id];
    if (p->refcount[id] == 0 || (need_held && c > p->refcount[id])) {
      st = fail(PA_ERR_STATE, "%s: block %d is held %d time(s), used %d time(s) in this call", fn, id,
                p->refcount[id], c);
      ++i;
      break;
    }
  }
  for (int32_t k = 0; k < i; ++k) p->scratch[ids[k]] = 0;
  return st;
}

pa_status pa_block_share(pa_pool* p, int32_t n, const int32_t* ids) {
  if (!p) return fail(PA_ERR_INVALID, "pa_block_share: pool is NULL");
  if (n < 0) return fail(PA_ERR_INVALID, "pa_block_share: n < 0");
  if (n == 0) return PA_OK;
  if (!ids) return fail(PA_ERR_INVALID, "pa_block_share: ids is NULL");
  pa_status st = validate(p, n, ids, false, "pa_block_share");
  if (st != PA_OK) return st;
  for (int32_t i = 0; i < n; ++i) ++p->refcount[ids[i]];
  return PA_OK;
}

pa_status pa_block_free(pa_pool* p, int32_t n, const int32_t* ids) {
  if (!p) return fail(PA_ERR_INVALID, "pa_block_free: pool is NULL");
  if (n < 0) return fail(PA_ERR_INVALID, "pa_block_free: n < 0");
  if (n == 0) return PA_OK;
  if (!ids) return fail(PA_ERR_INVALID, "pa_block_free: ids is NULL");
  pa_status st = validate(p, n, ids, true, "pa_block_free");
  if (st != PA_OK) return st;
  for (int32_t i = 0; i < n; ++i)
    if (--p->refcount[ids[i]] == 0) p->free_stack.push_back(ids[i]);
  return PA_OK;
}

int32_t pa_block_refcount(const pa_pool* p, int32_t id) {
  if (!p || id < 0 || id >= p->num_blocks) return -1;
  return p->refcount[id];
}

int32_t pa_pool_num_free(const pa_pool* p) { return p ? (int32_t)p->free_stack.size() : -1; }

int32_t pa_pool_num_blocks(const pa_pool* p) { return p ? p->num_blocks : -1; }

}  // extern "C"
