"""Cache hit-rate simulator for RAG requests over a block-budgeted KV pool.

Technical summary of LazyAttention (arXiv 2606.04302), "Problem Statement" and "Key
Contributions": a position-aware KV cache can reuse a document only where it sits at the
same position, prefix caching only where the whole preceding prompt is identical, and a
position-agnostic cache wherever the document appears; under skewed (Zipf) document
access and a bounded cache this raises the hit ratio (the pages report 7.5x over prefix
caching and 2.86x over position-aware caching for their own traces and budgets, which are
not available here, so these numbers are not reproduced -- only the comparison is).

Model (synthetic, seeded):
  * n_docs documents of doc_tokens tokens each; a request retrieves docs_per_request
    distinct documents drawn from a finite Zipf(s) over document ranks (a seeded
    permutation maps ranks to document ids), in draw order, placed back to back after a
    prompt start that is the same for every request (start_jitter > 0 draws it per
    request instead);
  * the cache is a pool of budget_blocks blocks of block_size tokens, managed by the
    library's pool index (lazyattn_pool_*): a document entry takes ceil(doc_tokens /
    block_size) blocks; entries no live request uses are evicted least recently used first;
  * requests run one at a time: every document of a request is acquired (hit or miss),
    then released when the request ends;
  * the three caches differ only in the key an entry is stored under:
        position-agnostic   the document
        position-aware      the document and its offset in the prompt
        prefix              the document and every document before it (and the start)
  * hit rate = document blocks served from the cache / document blocks requested.
Prefix caching is modelled per document-sized entry (a real prefix cache evicts leaf
blocks first); entries are independent here.

  python -m workload.cachesim     prints one JSON line per (skew, budget) setting.
"""
import hashlib
import json
import sys

import numpy as np

from .rag import zipf_ranks, _zipf_cdf

POLICIES = ("position-agnostic", "position-aware", "prefix")


def zipf_trace(n_docs, n_requests, docs_per_request, s, seed, start_jitter=0):
    """[(start, [doc, ...]), ...] -- documents distinct within a request."""
    rng = np.random.default_rng((seed, 21))
    rank_to_doc = rng.permutation(n_docs)
    cdf = _zipf_cdf(n_docs, s)
    out = []
    for _ in range(n_requests):
        docs, seen = [], set()
        while len(docs) < docs_per_request:
            d = int(rank_to_doc[zipf_ranks(rng, 1, n_docs, s, cdf)[0] - 1])
            if d not in seen:
                seen.add(d)
                docs.append(d)
        start = int(rng.integers(0, start_jitter + 1)) if start_jitter > 0 else 0
        out.append((start, docs))
    return out


def _h64(*parts):
    """Deterministic 64-bit key of a tuple of integers."""
    b = np.asarray(parts, dtype=np.int64).tobytes()
    return int.from_bytes(hashlib.blake2b(b, digest_size=8).digest(), "little")


def entry_keys(policy, start, docs, doc_tokens):
    """Cache key of every document of one request under `policy`."""
    if policy == "position-agnostic":
        return [_h64(0, d) for d in docs]
    if policy == "position-aware":
        return [_h64(1, d, start + i * doc_tokens) for i, d in enumerate(docs)]
    if policy == "prefix":
        return [_h64(2, start, *docs[: i + 1]) for i in range(len(docs))]
    raise ValueError(policy)


class _Model:
    """Adapter giving the plain pool-index model (oracle side) the PoolIndex interface."""

    def __init__(self, model):
        self.m = model

    def acquire(self, key, n_tokens):
        r = self.m.acquire(key, n_tokens)
        if isinstance(r, str):
            raise RuntimeError(r)
        return r

    def release(self, key):
        if self.m.release(key) is not None:
            raise RuntimeError("state")

    def stats(self):
        return self.m.stats()


def simulate(trace, policy, budget_blocks, doc_tokens, block_size=16, index=None):
    """Hit statistics of one policy on a trace. `index` is a fresh pool index with
    budget_blocks blocks (default: the library's native one)."""
    if index is None:
        from position_agnostic_kv_paged_amd import PoolIndex
        index = PoolIndex(budget_blocks, block_size)
    bpd = -(-doc_tokens // block_size)
    hit_blocks = req_blocks = 0
    for start, docs in trace:
        keys = entry_keys(policy, start, docs, doc_tokens)
        held = []
        for k in keys:
            _, hit = index.acquire(k, doc_tokens)
            held.append(k)
            req_blocks += bpd
            hit_blocks += bpd if hit else 0
        for k in held:
            index.release(k)
    st = index.stats()
    return {"policy": policy, "hit_rate": hit_blocks / max(req_blocks, 1),
            "hits": st["hits"], "misses": st["misses"], "evictions": st["evictions"]}


def main(argv=None):
    import argparse
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--docs", type=int, default=2000)
    ap.add_argument("--doc-tokens", type=int, default=1024)
    ap.add_argument("--docs-per-request", type=int, default=8)
    ap.add_argument("--requests", type=int, default=4000)
    ap.add_argument("--skews", default="0.6,0.8,1.0,1.2")
    ap.add_argument("--budgets", default="0.02,0.05,0.1,0.25,1.0",
                    help="cache size as a fraction of all documents' blocks")
    ap.add_argument("--start-jitter", type=int, default=0)
    ap.add_argument("--seed", type=int, default=1)
    a = ap.parse_args(argv)
    bpd = -(-a.doc_tokens // 16)
    for s in [float(x) for x in a.skews.split(",")]:
        trace = zipf_trace(a.docs, a.requests, a.docs_per_request, s, a.seed, a.start_jitter)
        for frac in [float(x) for x in a.budgets.split(",")]:
            budget = max(int(frac * a.docs * bpd), a.docs_per_request * bpd)
            res = {p: simulate(trace, p, budget, a.doc_tokens)["hit_rate"] for p in POLICIES}
            line = {"zipf_s": s, "budget_fraction": frac, "budget_blocks": budget,
                    "hit_rate": res,
                    "agnostic_over_prefix": res["position-agnostic"] / max(res["prefix"], 1e-12),
                    "agnostic_over_aware": res["position-agnostic"] / max(res["position-aware"], 1e-12)}
            print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
