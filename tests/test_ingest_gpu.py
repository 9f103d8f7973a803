"""Ingest of new keys/values into the position-free pool, on the GPU (through the C ABI):
bit-exact against the reference scatter, and a serving-loop check -- documents placed by
the pool index, written by the ingest kernel, reused across requests at other offsets and
evicted under a small budget -- with every request's attention compared to the float64
oracle over a host pool built independently (reference scatter, model of the index)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from oracle.pool import ingest as ingest_ref, PoolIndexModel  # noqa: E402
from workload import f32_to_bf16_bits, BF16_NAN  # noqa: E402
from tests.gpu_util import compare, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import position_agnostic_kv_paged_amd as L
    L.lib()


def _bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("D,Hkv,n", [(128, 8, 1000), (64, 2, 37), (128, 1, 1), (128, 3, 333),
                                      (64, 5, 1531)])
def test_ingest_bit_exact(D, Hkv, n):
    import position_agnostic_kv_paged_amd as L
    rng = np.random.default_rng(D + Hkv + n)
    nb = 96
    say(f"ingest D={D} Hkv={Hkv} tokens={n}")
    k0 = np.full((nb, Hkv, 16, D), np.uint16(BF16_NAN & 0xFFFF), np.uint16)
    v0 = k0.copy()
    kn, vn = _bits(rng, (n, Hkv, D)), _bits(rng, (n, Hkv, D))
    slots = rng.permutation(nb * 16)[:n].astype(np.int32)   # distinct slots
    slots[rng.random(n) < 0.1] = -1                          # unmapped tokens
    if n > 3:
        slots[1] = nb * 16 + 5                               # block past the pool
    kp, vp = _dev(k0), _dev(v0)
    L.ingest_kv(_dev(kn), _dev(vn), torch.from_numpy(slots).cuda(), kp, vp)
    torch.cuda.synchronize()
    want_k, want_v = ingest_ref(k0, v0, kn, vn, slots, 16)
    assert np.array_equal(kp.view(torch.int16).cpu().numpy().view(np.uint16), want_k)
    assert np.array_equal(vp.view(torch.int16).cpu().numpy().view(np.uint16), want_v)


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_serving_loop_ingest_reuse_evict(kind):
    """Requests of 3 Zipf-drawn documents (48 tokens) at a per-request start plus a private
    question, one at a time, over a 20-block pool: hits reuse the same blocks at other
    offsets, misses ingest, evictions overwrite blocks of unreferenced documents."""
    import position_agnostic_kv_paged_amd as L
    rng = np.random.default_rng(41 if kind == "prefill" else 42)
    Hq, Hkv, D, B, nb, base = 8, 2, 128, 16, 20, 10000.0
    n_docs, doc_tok, q_tok = 7, 48, 20
    doc_k = [_bits(rng, (doc_tok, Hkv, D)) for _ in range(n_docs)]
    doc_v = [_bits(rng, (doc_tok, Hkv, D)) for _ in range(n_docs)]
    nan = np.uint16(BF16_NAN & 0xFFFF)
    host_k = np.full((nb, Hkv, B, D), nan, np.uint16)
    host_v = host_k.copy()
    dev_k, dev_v = _dev(host_k), _dev(host_v)
    idx, model = L.PoolIndex(nb, B), PoolIndexModel(nb, B)
    p = 1.0 / np.arange(1, n_docs + 1) ** 1.1
    hits = evictions = 0
    for r in range(12):
        docs = list(rng.choice(n_docs, size=3, replace=False, p=p / p.sum()))
        start = int(rng.integers(0, 300))
        ids, offs, writes = [], [], []
        pos = start
        for d in docs:
            blocks, hit = idx.acquire(d + 1, doc_tok)
            mblocks, mhit = model.acquire(d + 1, doc_tok)    # oracle-side layout
            assert list(blocks) == mblocks and hit == mhit
            hits += hit
            if not hit:
                slots = np.array([blocks[t // B] * B + t % B for t in range(doc_tok)], np.int32)
                writes.append((doc_k[d], doc_v[d], slots))
            ids += list(mblocks)
            offs += [pos + B * i for i in range(len(mblocks))]
            pos += doc_tok
        qk, qv = _bits(rng, (q_tok, Hkv, D)), _bits(rng, (q_tok, Hkv, D))
        pblocks = idx.alloc_private(2)
        assert list(pblocks) == model.alloc_private(2)
        writes.append((qk, qv, np.array([pblocks[t // B] * B + t % B for t in range(q_tok)],
                                        np.int32)))
        ids += list(pblocks)
        offs += [pos, pos + B]
        for k, v, slots in writes:                              # both pools, same writes
            L.ingest_kv(_dev(k), _dev(v), torch.from_numpy(slots).cuda(), dev_k, dev_v)
            host_k, host_v = ingest_ref(host_k, host_v, k, v, slots, B)
        kv_len = pos + q_tok - start
        nq = q_tok if kind == "prefill" else 1
        q_pos = np.arange(pos + q_tok - nq, pos + q_tok, dtype=np.int32)
        q = _bits(rng, (nq, Hq, D))
        bt = np.array([0, len(ids)], np.int32)
        words = L.encode_meta(np.array(ids, np.int32), np.array(offs, np.int64), bt)
        fn = L.prefill if kind == "prefill" else L.decode
        out = fn(_dev(q), dev_k, dev_v, torch.from_numpy(bt).cuda(),
                 torch.from_numpy(words.view(np.int32)).cuda(),
                 torch.tensor([kv_len], dtype=torch.int32, device="cuda"),
                 torch.tensor([0, nq], dtype=torch.int32, device="cuda"),
                 torch.from_numpy(q_pos).cuda(), base, len(ids))
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        want = oracle.lazy_attention(q, host_k, host_v, [np.array(ids)], [np.array(offs)],
                                     np.array([kv_len]), np.array([0, nq]), q_pos, base, B)
        compare(got, want, f"serving request {r} via {kind} (docs {docs}, start {start})")
        for d in docs:
            idx.release(d + 1)
            model.release(d + 1)
        idx.free_private(pblocks)
        model.free_private(list(pblocks))
        assert idx.stats() == model.stats()
    st = idx.stats()
    say(f"  hits {hits} evictions {st['evictions']}")
    assert hits > 0 and st["evictions"] > 0
