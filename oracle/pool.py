"""Reference statements of the pool side of the method (test infrastructure only).

  ingest          new tokens' keys and values written into their pool slots exactly as
                  given (technical summary, "Core Concept": the cache keeps content-only
                  keys, so nothing is rotated on the way in) -- a plain numpy scatter.
  PoolIndexModel  the block index of the position-free pool, keyed by document alone
                  ("Core Concept" / "Problem Statement": one physical copy serves every
                  request at any offset). The pages fix no replacement policy; the library
                  documents LRU among documents no live request uses, and this model
                  restates that documented behaviour step by step in plain Python
                  (dictionary, ordered dictionary, list), including the order in which
                  free block ids are handed out (a stack, ids 0, 1, 2, ... first; freed
                  blocks are pushed in the order the document listed them).
"""
from collections import OrderedDict

import numpy as np


def ingest(k_pool, v_pool, k_new, v_new, slot_mapping, B):
    """Return copies of (k_pool, v_pool) [num_blocks, Hkv, B, D] with token i's rows
    k_new[i], v_new[i] ([n, Hkv, D]) at block slot_mapping[i] // B, slot slot_mapping[i] % B;
    tokens with a negative slot or a block past the pool are not written."""
    k_out, v_out = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    num_blocks = k_pool.shape[0]
    for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0 or s // B >= num_blocks:
            continue
        k_out[s // B, :, s % B, :] = k_new[i]
        v_out[s // B, :, s % B, :] = v_new[i]
    return k_out, v_out


class PoolIndexModel:
    """Plain model of the pool index: same results as lazyattn_pool_* for the same calls."""

    def __init__(self, num_blocks, block_size):
        self.num_blocks, self.B = num_blocks, block_size
        self.free = list(range(num_blocks - 1, -1, -1))       # top of the stack = end
        self.docs = {}                                        # key -> [blocks, n_tokens, refs]
        self.lru = OrderedDict()                              # unreferenced docs, oldest first
        self.private = set()
        self.hits = self.misses = self.evictions = self.evicted_blocks = 0

    def _evictable(self):
        return sum(len(self.docs[k][0]) for k in self.lru)

    def _make_room(self, need):
        if len(self.free) + self._evictable() < need:
            return False
        while len(self.free) < need:
            key, _ = self.lru.popitem(last=False)
            blocks = self.docs.pop(key)[0]
            self.free.extend(blocks)
            self.evictions += 1
            self.evicted_blocks += len(blocks)
        return True

    def acquire(self, key, n_tokens):
        """-> (blocks, hit) or the string 'nospace' / 'state'."""
        need = -(-n_tokens // self.B)
        if key in self.docs:
            d = self.docs[key]
            if d[1] != n_tokens:
                return "state"
            if d[2] == 0:
                del self.lru[key]
            d[2] += 1
            self.hits += 1
            return list(d[0]), True
        if not self._make_room(need):
            return "nospace"
        blocks = [self.free.pop() for _ in range(need)]
        self.docs[key] = [blocks, n_tokens, 1]
        self.misses += 1
        return list(blocks), False

    def release(self, key):
        if key not in self.docs or self.docs[key][2] <= 0:
            return "state"
        self.docs[key][2] -= 1
        if self.docs[key][2] == 0:
            self.lru[key] = True
        return None

    def alloc_private(self, n):
        if not self._make_room(n):
            return "nospace"
        blocks = [self.free.pop() for _ in range(n)]
        self.private.update(blocks)
        return blocks

    def free_private(self, blocks):
        if len(set(blocks)) != len(blocks) or any(b not in self.private for b in blocks):
            return "state"
        for b in blocks:
            self.private.discard(b)
            self.free.append(b)
        return None

    def stats(self):
        return dict(hits=self.hits, misses=self.misses, evictions=self.evictions,
                    evicted_blocks=self.evicted_blocks, num_blocks=self.num_blocks,
                    free_blocks=len(self.free), cached_docs=len(self.docs),
                    pinned_docs=sum(1 for d in self.docs.values() if d[2] > 0),
                    private_blocks=len(self.private), evictable_blocks=self._evictable())
