// Host-side index of the position-free KV pool: which physical blocks hold which document,
// how many live requests use each document, and which cached documents may be evicted.
//
// Technical summary of LazyAttention (arXiv 2606.04302), "Core Concept" and "Problem
// Statement": because cached keys carry no position, one physical copy of a document's
// blocks serves every request that contains the document, at any offset. The index is
// therefore keyed by document alone (never by document and position); a request that finds
// its document cached reuses the same block ids, and only missing documents take new
// blocks. Under a block budget, documents no live request uses are kept in LRU order and
// evicted oldest first when an allocation needs room.
#include "lazyattn.h"

#include <cstdint>
#include <list>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

namespace {

enum BlockState : uint8_t { kFree = 0, kDoc = 1, kPrivate = 2 };

struct Doc {
  std::vector<int32_t> blocks;
  int32_t n_tokens = 0;
  int32_t refs = 0;
  std::list<uint64_t>::iterator lru;   // valid while refs == 0
};

struct PoolIndex {
  int32_t num_blocks, block_size;
  std::vector<int32_t> free_stack;     // top = back; ids handed out in ascending order at first
  std::vector<uint8_t> state;
  std::unordered_map<uint64_t, Doc> docs;
  std::list<uint64_t> lru;             // unreferenced cached documents, oldest first
  int64_t evictable_blocks = 0;        // blocks of the documents in `lru`
  int64_t hits = 0, misses = 0, evictions = 0, evicted_blocks = 0;
  int32_t private_blocks = 0, pinned_docs = 0;
  std::mutex mu;

  PoolIndex(int32_t n, int32_t b) : num_blocks(n), block_size(b), state(n, kFree) {
    free_stack.reserve(n);
    for (int32_t i = n - 1; i >= 0; --i) free_stack.push_back(i);
  }

  // make `need` blocks free by evicting unreferenced documents, oldest first; false (and no
  // eviction) if even evicting all of them would not be enough
  bool make_room(int64_t need) {
    if ((int64_t)free_stack.size() + evictable_blocks < need) return false;
    while ((int64_t)free_stack.size() < need) {
      const uint64_t key = lru.front();
      lru.pop_front();
      auto it = docs.find(key);
      for (int32_t b : it->second.blocks) {
        state[b] = kFree;
        free_stack.push_back(b);
      }
      evictable_blocks -= (int64_t)it->second.blocks.size();
      evicted_blocks += (int64_t)it->second.blocks.size();
      ++evictions;
      docs.erase(it);
    }
    return true;
  }

  void take(int32_t n, std::vector<int32_t>& out, BlockState st) {
    for (int32_t i = 0; i < n; ++i) {
      const int32_t b = free_stack.back();
      free_stack.pop_back();
      state[b] = st;
      out.push_back(b);
    }
  }
};

}  // namespace

extern "C" {

int lazyattn_pool_create(int32_t num_blocks, int32_t block_size, void** pool_out) {
  if (!pool_out) return LAZYATTN_ERR_NULL;
  *pool_out = nullptr;
  if (num_blocks <= 0 || num_blocks > (1 << LAZYATTN_ID_BITS) || block_size <= 0)
    return LAZYATTN_ERR_ARG;
  PoolIndex* p = new (std::nothrow) PoolIndex(num_blocks, block_size);
  if (!p) return LAZYATTN_ERR_NOSPACE;
  *pool_out = p;
  return LAZYATTN_OK;
}

int lazyattn_pool_destroy(void* pool) {
  if (!pool) return LAZYATTN_ERR_NULL;
  delete static_cast<PoolIndex*>(pool);
  return LAZYATTN_OK;
}

int lazyattn_pool_acquire(void* pool, uint64_t doc_key, int32_t n_tokens, int32_t* blocks_out,
                          int32_t blocks_cap, int32_t* n_blocks_out, int32_t* hit_out) {
  if (!pool || !blocks_out || !n_blocks_out || !hit_out) return LAZYATTN_ERR_NULL;
  PoolIndex& P = *static_cast<PoolIndex*>(pool);
  if (n_tokens <= 0) return LAZYATTN_ERR_ARG;
  std::lock_guard<std::mutex> g(P.mu);
  const int64_t need = ((int64_t)n_tokens + P.block_size - 1) / P.block_size;
  *n_blocks_out = (int32_t)need;
  auto it = P.docs.find(doc_key);
  if (it != P.docs.end()) {
    Doc& d = it->second;
    if (d.n_tokens != n_tokens) return LAZYATTN_ERR_STATE;
    if (blocks_cap < (int32_t)d.blocks.size()) return LAZYATTN_ERR_ARG;
    if (d.refs == 0) {
      P.lru.erase(d.lru);
      P.evictable_blocks -= (int64_t)d.blocks.size();
      ++P.pinned_docs;
    }
    ++d.refs;
    ++P.hits;
    for (size_t i = 0; i < d.blocks.size(); ++i) blocks_out[i] = d.blocks[i];
    *hit_out = 1;
    return LAZYATTN_OK;
  }
  if (blocks_cap < need) return LAZYATTN_ERR_ARG;
  if (!P.make_room(need)) return LAZYATTN_ERR_NOSPACE;
  Doc d;
  d.n_tokens = n_tokens;
  d.refs = 1;
  P.take((int32_t)need, d.blocks, kDoc);
  for (int64_t i = 0; i < need; ++i) blocks_out[i] = d.blocks[i];
  P.docs.emplace(doc_key, std::move(d));
  ++P.misses;
  ++P.pinned_docs;
  *hit_out = 0;
  return LAZYATTN_OK;
}

int lazyattn_pool_release(void* pool, uint64_t doc_key) {
  if (!pool) return LAZYATTN_ERR_NULL;
  PoolIndex& P = *static_cast<PoolIndex*>(pool);
  std::lock_guard<std::mutex> g(P.mu);
  auto it = P.docs.find(doc_key);
  if (it == P.docs.end() || it->second.refs <= 0) return LAZYATTN_ERR_STATE;
  Doc& d = it->second;
  if (--d.refs == 0) {
    d.lru = P.lru.insert(P.lru.end(), doc_key);
    P.evictable_blocks += (int64_t)d.blocks.size();
    --P.pinned_docs;
  }
  return LAZYATTN_OK;
}

int lazyattn_pool_alloc_private(void* pool, int32_t n_blocks, int32_t* blocks_out) {
  if (!pool || !blocks_out) return LAZYATTN_ERR_NULL;
  PoolIndex& P = *static_cast<PoolIndex*>(pool);
  if (n_blocks <= 0) return LAZYATTN_ERR_ARG;
  std::lock_guard<std::mutex> g(P.mu);
  if (!P.make_room(n_blocks)) return LAZYATTN_ERR_NOSPACE;
  std::vector<int32_t> got;
  got.reserve(n_blocks);
  P.take(n_blocks, got, kPrivate);
  for (int32_t i = 0; i < n_blocks; ++i) blocks_out[i] = got[i];
  P.private_blocks += n_blocks;
  return LAZYATTN_OK;
}

int lazyattn_pool_free_private(void* pool, const int32_t* blocks, int32_t n_blocks) {
  if (!pool || (!blocks && n_blocks > 0)) return LAZYATTN_ERR_NULL;
  PoolIndex& P = *static_cast<PoolIndex*>(pool);
  if (n_blocks < 0) return LAZYATTN_ERR_ARG;
  std::lock_guard<std::mutex> g(P.mu);
  for (int32_t i = 0; i < n_blocks; ++i) {                 // all or nothing
    const int32_t b = blocks[i];
    if (b < 0 || b >= P.num_blocks || P.state[b] != kPrivate) return LAZYATTN_ERR_STATE;
    for (int32_t k = 0; k < i; ++k)
      if (blocks[k] == b) return LAZYATTN_ERR_STATE;      // freed twice in one call
  }
  for (int32_t i = 0; i < n_blocks; ++i) {
    P.state[blocks[i]] = kFree;
    P.free_stack.push_back(blocks[i]);
  }
  P.private_blocks -= n_blocks;
  return LAZYATTN_OK;
}

int lazyattn_pool_stats(void* pool, LazyattnPoolStats* out) {
  if (!pool || !out) return LAZYATTN_ERR_NULL;
  PoolIndex& P = *static_cast<PoolIndex*>(pool);
  std::lock_guard<std::mutex> g(P.mu);
  out->hits = P.hits;
  out->misses = P.misses;
  out->evictions = P.evictions;
  out->evicted_blocks = P.evicted_blocks;
  out->num_blocks = P.num_blocks;
  out->free_blocks = (int32_t)P.free_stack.size();
  out->cached_docs = (int32_t)P.docs.size();
  out->pinned_docs = P.pinned_docs;
  out->private_blocks = P.private_blocks;
  out->evictable_blocks = (int32_t)P.evictable_blocks;
  return LAZYATTN_OK;
}

}  // extern "C"
