"""Seeded workload generator: determinism, Zipf statistics, layout structure (CPU)."""
import hashlib

import numpy as np
import pytest

from workload import make, zipf_ranks, harmonic, f32_to_bf16_bits, CONFIGS
from workload.rag import _to_bf16_fast


def _digest(wl):
    h = hashlib.sha256()
    for a in [wl.q_bits, wl.k_bits, wl.v_bits, wl.pool_ids, wl.kv_lens, wl.q_pos,
              wl.flat_block_ids, wl.flat_offsets]:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_deterministic():
    a = make("decode-32q8kv-b64-ctx4161")
    b = make("decode-32q8kv-b64-ctx4161")
    assert _digest(a) == _digest(b)
    c = make("decode-32q8kv-b64-ctx4161", seed=99)
    assert _digest(a) != _digest(c)


@pytest.mark.parametrize("N,s", [(1000, 1.1), (4000, 1.2), (2000, 1.1)])
def test_zipf_rank1_frequency(N, s):
    rng = np.random.default_rng(123)
    n = 200000
    r = zipf_ranks(rng, n, N, s)
    p1 = 1.0 / harmonic(N, s)
    f1 = np.mean(r == 1)
    assert abs(f1 - p1) < 4 * np.sqrt(p1 * (1 - p1) / n)
    p2 = 2.0 ** (-s) / harmonic(N, s)
    assert abs(np.mean(r == 2) - p2) < 4 * np.sqrt(p2 * (1 - p2) / n)
    assert r.min() >= 1 and r.max() <= N


def test_bf16_rounding_paths_agree():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0,
                                  1e-40, 3.0e38], dtype=np.float32)])
    assert np.array_equal(_to_bf16_fast(x), f32_to_bf16_bits(x))
    # ties to even: 1 + 2^-8 -> 1.0 (0x3F80); 1 + 3*2^-8 -> 1 + 2^-6 (0x3F82)
    assert f32_to_bf16_bits(np.float32(1.0 + 2**-8)) == 0x3F80
    assert f32_to_bf16_bits(np.float32(1.0 + 3 * 2**-8)) == 0x3F82


def test_tiny_layout():
    wl = make("tiny-prefill-4q1kv-d64")
    assert wl.num_seqs == 1 and wl.total_q == 32 and int(wl.kv_lens[0]) == 160
    assert list(wl.seq_offsets[0]) == [0, 16, 32, 48, 64, 80, 96, 112, 128, 144]
    assert list(wl.q_pos) == list(range(128, 160))
    assert wl.num_blocks == 10 and sorted(wl.pool_ids) == list(range(10))
    d = make("tiny-prefill-4q1kv-d64", decode_variant=True)
    assert int(d.kv_lens[0]) == 161 and list(d.q_pos) == [160]
    assert np.all(d.k_bits[np.searchsorted(d.pool_ids, d.seq_block_ids[0][-1]), :, 1:] == 0x7FC0)


def test_decode_layout_back_to_back():
    wl = make("decode-32q8kv-b64-ctx4161")
    assert wl.num_seqs == 64 and np.all(wl.kv_lens == 4161)
    for s in range(wl.num_seqs):
        offs = wl.seq_offsets[s]
        assert len(offs) == 261
        delta = offs - 16 * np.arange(len(offs))
        assert np.all(delta == delta[0]) and 0 <= delta[0] <= 511
        assert wl.q_pos[s] == offs[-1]            # decode token at the last slot
    assert wl.num_blocks == 32000 + 64 * 5


def test_prefill_layout_gaps_and_queries():
    wl = make("prefill-32q8kv-b16-ctx5376")
    assert wl.num_seqs == 16 and wl.total_q == 16 * 256 and np.all(wl.kv_lens == 5376)
    for s in range(wl.num_seqs):
        offs = wl.seq_offsets[s]
        assert len(offs) == 336
        assert np.all(np.diff(offs) >= 16)
        qp = wl.q_pos[wl.q_indptr[s]: wl.q_indptr[s + 1]]
        assert np.array_equal(qp, offs[320] + np.arange(256))


def test_long_decode_repeats_documents():
    wl = make("decode-32q8kv-b8-ctx32769")
    assert np.all(wl.kv_lens == 32769)
    repeats = [len(x) - len(np.unique(x)) for x in wl.seq_block_ids]
    assert max(repeats) > 0                   # same physical block at several offsets


def test_mixed_layout():
    cfg = CONFIGS["mixed-64q8kv-4p96d"]
    assert cfg.Hq == 64 and cfg.Hkv == 8
    wl = make("mixed-64q8kv-4p96d")
    qlen = np.diff(wl.q_indptr)
    assert list(qlen[:4]) == [512] * 4 and np.all(qlen[4:] == 1) and wl.num_seqs == 100
    assert np.all(wl.kv_lens[:4] == 16 * 1024 + 512) and np.all(wl.kv_lens[4:] == 12 * 1024 + 1)


def test_no_reuse_control_has_distinct_documents():
    """The no-reuse control keeps the shape (requests, documents per request, lengths) and
    references every pool block at most once (private blocks are unique anyway)."""
    base = make("decode-32q8kv-b64-ctx4161")
    ctl = make("decode-32q8kv-b64-ctx4161", no_reuse=True)
    assert ctl.num_seqs == base.num_seqs
    assert np.array_equal(ctl.kv_lens, base.kv_lens)
    assert np.array_equal(ctl.q_indptr, base.q_indptr)
    ids = np.concatenate([ctl.seq_block_ids[s] for s in range(ctl.num_seqs)])
    assert len(np.unique(ids)) == len(ids)
    base_ids = np.concatenate([base.seq_block_ids[s] for s in range(base.num_seqs)])
    assert len(np.unique(base_ids)) < len(base_ids)          # the Zipf batch does reuse
