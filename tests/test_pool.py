"""Pool side of the method on the host: the ingest scatter reference, the pool-index model
pinned on hand-worked traces, the native pool index (liblazyattn.so, host code) against
that model, and the hit-rate simulator against closed forms."""
import os

import numpy as np
import pytest

from oracle.pool import ingest, PoolIndexModel
from workload.cachesim import zipf_trace, simulate, entry_keys, _Model, POLICIES


# ------------------------------------------------------------------ ingest reference

def test_ingest_reference_hand_example():
    # 3 blocks of B = 2 slots, 1 KV head, D = 2; tokens go to slots 5, 0, -1 (skipped),
    # 9 (block 4: past the pool, skipped) and 2
    k_pool = np.full((3, 1, 2, 2), 7, np.uint16)
    v_pool = np.full((3, 1, 2, 2), 8, np.uint16)
    k_new = np.array([[[1, 2]], [[3, 4]], [[5, 6]], [[9, 9]], [[10, 11]]], np.uint16)
    v_new = k_new + 100
    slots = np.array([5, 0, -1, 9, 2], np.int32)
    k, v = ingest(k_pool, v_pool, k_new, v_new, slots, 2)
    want_k = np.array([[[[3, 4], [7, 7]]], [[[10, 11], [7, 7]]], [[[7, 7], [1, 2]]]], np.uint16)
    assert np.array_equal(k, want_k)
    assert np.array_equal(v, np.where(want_k == 7, 8, want_k + 100))
    assert np.array_equal(k_pool, np.full((3, 1, 2, 2), 7, np.uint16))   # inputs untouched


# ------------------------------------------------------------------ pool-index model

def test_model_textbook_lru_trace():
    """4 blocks, documents of 2 blocks (32 tokens, B = 16); worked by hand."""
    m = PoolIndexModel(4, 16)
    assert m.acquire("A", 32) == ([0, 1], False)
    assert m.release("A") is None
    assert m.acquire("B", 32) == ([2, 3], False)
    assert m.release("B") is None
    assert m.acquire("A", 32) == ([0, 1], True)           # hit; A becomes most recent
    assert m.release("A") is None                         # LRU order now: B, A
    # C needs 2 blocks, none free: B (least recently used) is evicted; its blocks [2, 3]
    # are pushed back in order, so C pops 3 first, then 2
    assert m.acquire("C", 17) == ([3, 2], False)
    assert m.stats()["evictions"] == 1 and "B" not in m.docs
    assert m.acquire("A", 32) == ([0, 1], True)           # A pinned by this reference
    assert m.acquire("D", 1) == "nospace"                 # C and A are both referenced
    assert m.release("C") is None
    assert m.acquire("D", 1) == ([2], False)              # evicts C ([3, 2] pushed); 3 spare
    assert m.free == [3] and m.stats()["evicted_blocks"] == 4
    assert m.acquire("A", 31) == "state"                  # same key, other length
    assert m.release("B") == "state"                      # evicted: unknown
    assert m.alloc_private(2) == "nospace"                # 1 free, nothing evictable
    assert m.release("D") is None
    assert m.alloc_private(2) == [2, 3]                   # evicts D: free stack [3, 2]
    assert m.free_private([2, 2]) == "state" and m.free_private([0]) == "state"
    assert m.free_private([2, 3]) is None
    st = m.stats()
    assert (st["hits"], st["misses"], st["evictions"], st["free_blocks"]) == (2, 4, 3, 2)


# ------------------------------------------------------------------ native index vs model

@pytest.fixture(scope="module")
def native():
    import position_agnostic_kv_paged_amd as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built")
    L.lib()
    return L


def _native_call(idx, op, *args):
    from position_agnostic_kv_paged_amd._lib import LazyAttnError, ERR_NOSPACE, ERR_STATE
    try:
        r = getattr(idx, op)(*args)
    except LazyAttnError as e:
        return {ERR_NOSPACE: "nospace", ERR_STATE: "state"}[e.code]
    if op == "acquire":
        return list(r[0]), r[1]
    if op == "alloc_private":
        return list(r)
    return r


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_native_pool_index_equals_model(native, seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(8, 40))
    idx, m = native.PoolIndex(nb, 16), PoolIndexModel(nb, 16)
    held, priv = [], []
    lengths = {}
    for step in range(600):
        r = rng.random()
        if r < 0.45:
            key = int(rng.integers(1, 25))
            n = lengths.setdefault(key, int(rng.integers(1, 6 * 16)))
            if rng.random() < 0.03:
                n += 1                                    # wrong length: STATE
            a, b = _native_call(idx, "acquire", key, n), m.acquire(key, n)
            assert a == (tuple(b) if isinstance(b, tuple) else b) or a == b, (step, a, b)
            if isinstance(b, tuple):
                held.append(key)
        elif r < 0.8:
            key = held.pop(int(rng.integers(len(held)))) if held and rng.random() < 0.9 \
                else int(rng.integers(1, 25))
            assert _native_call(idx, "release", key) == m.release(key), step
        elif r < 0.9:
            n = int(rng.integers(1, 4))
            a, b = _native_call(idx, "alloc_private", n), m.alloc_private(n)
            assert a == b, (step, a, b)
            if isinstance(b, list):
                priv.append(b)
        else:
            blocks = priv.pop() if priv and rng.random() < 0.85 else [int(rng.integers(nb))]
            assert _native_call(idx, "free_private", blocks) == m.free_private(blocks), step
        assert idx.stats() == m.stats(), step


# ------------------------------------------------------------------ hit-rate simulator

def _first_seen_hits(keys):
    seen, hits = set(), 0
    for k in keys:
        hits += k in seen
        seen.add(k)
    return hits


@pytest.mark.parametrize("s", [0.7, 1.1])
def test_simulator_unlimited_budget_closed_forms(native, s):
    """Without evictions an entry misses exactly on first use: hit rate = 1 - distinct
    keys / draws, with keys = documents, (document, offset) or prefixes."""
    trace = zipf_trace(300, 400, 5, s, seed=3, start_jitter=0)
    budget = 400 * 5 * 4                                  # room for every key ever used
    for policy in POLICIES:
        keys = [k for start, docs in trace for k in entry_keys(policy, start, docs, 64)]
        res = simulate(trace, policy, budget, 64)
        assert res["hit_rate"] == pytest.approx(_first_seen_hits(keys) / len(keys), abs=0)
        assert res["evictions"] == 0
    docs = [d for _, ds in trace for d in ds]
    agn = simulate(trace, "position-agnostic", budget, 64)["hit_rate"]
    assert agn == pytest.approx(1 - len(set(docs)) / len(docs), abs=0)


def test_simulator_single_document_requests_coincide(native):
    """One document per request, same start: the three keys identify the same entries."""
    trace = zipf_trace(200, 500, 1, 1.0, seed=4)
    rates = [simulate(trace, p, 40 * 4, 64)["hit_rate"] for p in POLICIES]
    assert rates[0] == rates[1] == rates[2]


def test_simulator_native_equals_model(native):
    trace = zipf_trace(150, 300, 6, 0.9, seed=5, start_jitter=64)
    for p in POLICIES:
        a = simulate(trace, p, 120, 48)
        b = simulate(trace, p, 120, 48, index=_Model(PoolIndexModel(120, 16)))
        assert a == b


def test_simulator_ordering(native):
    """The pages' comparison: position-agnostic >= position-aware >= prefix."""
    for s in (0.8, 1.2):
        trace = zipf_trace(400, 600, 6, s, seed=6)
        for budget in (200, 800, 400 * 4):
            r = {p: simulate(trace, p, budget, 64)["hit_rate"] for p in POLICIES}
            assert r["position-agnostic"] >= r["position-aware"] >= r["prefix"], (s, budget, r)
            assert r["position-agnostic"] > r["prefix"]
