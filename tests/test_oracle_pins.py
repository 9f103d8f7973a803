"""Pins of the float64 oracle to things other than itself (CPU only).

Each test targets a plausible mistake: a wrong frequency exponent, a swapped
pair convention or sign, a dropped scale, a wrong GQA head map, a mask on table
order instead of logical position, a materialisation that depends on block ids,
or a packing error.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import rope, meta, overhead
from tests.brute import brute_attention, rope_matrix
from tests.util import small, oracle_out, dense_request, rel
from workload import Segment, RequestLayout, build

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- RoPE

def test_inv_freq_closed_form():
    assert np.allclose(rope.inv_freq(4, 10000.0), [1.0, 0.01], rtol=0, atol=1e-15)
    assert np.allclose(rope.inv_freq(8, 100.0),
                       [1.0, 0.31622776601683794, 0.1, 0.031622776601683794], rtol=1e-15)


def test_rotate_two_dims_is_plane_rotation():
    # D = 2: theta_0 = 1 rad per position, (1, 0) rotated by n = 1
    y = rope.rotate(np.array([1.0, 0.0]), 1, 10000.0)
    assert abs(y[0] - 0.5403023058681398) < 1e-15 and abs(y[1] - 0.8414709848078965) < 1e-15


def test_rotate_matches_complex_form():
    rng = np.random.default_rng(0)
    D, base = 16, 10000.0
    x = rng.standard_normal((5, D))
    pos = np.array([0, 1, 17, 4096, 35001])
    z = x[:, : D // 2] + 1j * x[:, D // 2:]
    th = base ** (-np.arange(D // 2) * 2.0 / D)
    zr = z * np.exp(1j * pos[:, None] * th[None, :])
    want = np.concatenate([zr.real, zr.imag], axis=1)
    got = rope.rotate(x, pos, base)
    assert np.max(np.abs(got - want)) < 1e-11


def test_rotate_matches_explicit_matrix():
    rng = np.random.default_rng(1)
    for D in (8, 64, 128):
        x = rng.standard_normal(D)
        for n in (0, 3, 511, 20000):
            assert np.max(np.abs(rope.rotate(x, n, 10000.0) - rope_matrix(n, D, 10000.0) @ x)) < 1e-11


def test_rotation_group_identities():
    rng = np.random.default_rng(2)
    D, base = 128, 10000.0
    x = rng.standard_normal(D)
    assert np.array_equal(rope.rotate(x, 0, base), x)
    for a, b in [(3, 5), (1000, -77), (123456, 654321)]:
        lhs = rope.rotate(rope.rotate(x, b, base), a, base)
        assert np.max(np.abs(lhs - rope.rotate(x, a + b, base))) < 1e-8
        assert abs(np.linalg.norm(rope.rotate(x, a, base)) - np.linalg.norm(x)) < 1e-12


def test_relative_position_identity():
    """<R(a) q, R(b) k> = <R(a - b) q, k> (the relative-offset property)."""
    rng = np.random.default_rng(3)
    D, base = 128, 10000.0
    for _ in range(50):
        q, k = rng.standard_normal(D), rng.standard_normal(D)
        a, b = rng.integers(-10**6, 10**6, size=2)
        lhs = rope.rotate(q, a, base) @ rope.rotate(k, b, base)
        rhs = rope.rotate(q, a - b, base) @ k
        assert abs(lhs - rhs) < 1e-8 * max(1.0, abs(rhs))


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("Hq,Hkv,D", [(4, 2, 16), (4, 1, 8), (2, 2, 16), (8, 1, 8)])
def test_oracle_equals_brute_force(Hq, Hkv, D):
    wl = small(Hq=Hq, Hkv=Hkv, D=D, seed=11 + Hq + D)
    got = oracle_out(wl)
    want = brute_attention(wl)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) < 1e-12


def test_brute_force_with_gaps_overlap_and_partial_block():
    # overlapping documents, a gap, an unaligned start, 5-token partial tail,
    # and a query set spanning all of them
    segs = [Segment("doc", 3, doc=1), Segment("doc", 20, doc=0),
            Segment("doc", 100, doc=1), Segment("private", 140, tokens=21)]
    wl = small(segs=segs, q_len=21, seed=5, q_scale=4.0)
    assert np.max(np.abs(oracle_out(wl) - brute_attention(wl))) < 1e-12


def test_sdpa_special_case_dense_from_zero():
    """Dense layout from position 0 equals torch SDPA (causal) over eagerly rotated q, k."""
    torch = pytest.importorskip("torch")
    Hq, Hkv, D, n = 8, 2, 32, 45
    wl = build("dense", Hq, Hkv, D, 16, 10000.0, 1, 16, [dense_request(n)], seed=9)
    got = oracle_out(wl)
    q = oracle.bf16_bits_to_f64(wl.q_bits)                       # [n, Hq, D]
    ids = wl.compact_ids(0)
    k = np.concatenate([oracle.bf16_bits_to_f64(wl.k_bits[i]) for i in ids], axis=1)[:, :n]
    v = np.concatenate([oracle.bf16_bits_to_f64(wl.v_bits[i]) for i in ids], axis=1)[:, :n]
    th = 10000.0 ** (-np.arange(D // 2) * 2.0 / D)
    pos = np.arange(n)

    def crot(x):  # complex-form RoPE over the token axis (second to last)
        z = x[..., : D // 2] + 1j * x[..., D // 2:]
        z = z * np.exp(1j * pos[:, None] * th[None, :])
        return np.concatenate([z.real, z.imag], axis=-1)
    qt = torch.from_numpy(crot(q.transpose(1, 0, 2)))             # [Hq, n, D]
    kt = torch.from_numpy(crot(k)).repeat_interleave(Hq // Hkv, dim=0)
    vt = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    ref = ref.numpy().transpose(1, 0, 2)
    assert np.max(np.abs(got - ref)) < 1e-12


# ---------------------------------------------------------------- partial rotary

def test_partial_rotate_matches_complex_form():
    """rotary_dim r: z_k = x_k + i x_{k+r/2} times exp(i n base^(-2k/r)) for k < r/2, the
    other dims untouched (a frequency exponent over D instead of r, or pairs k, k + D/2,
    would fail)."""
    rng = np.random.default_rng(40)
    base = 10000.0
    for D, r in ((64, 16), (128, 32), (128, 64), (16, 2)):
        x = rng.standard_normal((4, D))
        pos = np.array([0, 3, 777, 40001])
        z = x[:, : r // 2] + 1j * x[:, r // 2: r]
        th = np.exp(-np.log(base) * 2.0 * np.arange(r // 2) / r)
        zr = z * np.exp(1j * pos[:, None] * th[None, :])
        want = np.concatenate([zr.real, zr.imag, x[:, r:]], axis=1)
        got = rope.rotate(x, pos, base, rotary_dim=r)
        assert np.max(np.abs(got - want)) < 1e-11
        assert np.array_equal(got[:, r:], x[:, r:])
    x = rng.standard_normal(32)
    assert np.array_equal(rope.rotate(x, 99, base, rotary_dim=32), rope.rotate(x, 99, base))


def test_partial_rotary_relative_identity():
    """<R(a) q, R(b) k> = <R(a - b) q, k> also with partial rotary: the pass-through dims
    add the same plain product on both sides."""
    rng = np.random.default_rng(41)
    for r in (16, 48):
        q, k = rng.standard_normal(64), rng.standard_normal(64)
        for a, b in ((5, 2), (100000, 31), (7, 900000)):
            lhs = rope.rotate(q, a, 500000.0, r) @ rope.rotate(k, b, 500000.0, r)
            rhs = rope.rotate(q, a - b, 500000.0, r) @ k
            assert abs(lhs - rhs) < 1e-9 * (1 + abs(lhs))


def test_partial_rotary_sdpa_dense_from_zero():
    """Dense layout from position 0 with rotary_dim 16 of 64 equals torch SDPA over q, k
    rotated in complex form on their first 16 dims (both q and k see the partial rotation,
    the scale stays 1/sqrt(D))."""
    torch = pytest.importorskip("torch")
    Hq, Hkv, D, r, n = 4, 2, 64, 16, 37
    wl = build("dense", Hq, Hkv, D, 16, 10000.0, 1, 16, [dense_request(n)], seed=45)
    got = oracle_out(wl, rotary_dim=r)
    q = oracle.bf16_bits_to_f64(wl.q_bits)
    ids = wl.compact_ids(0)
    k = np.concatenate([oracle.bf16_bits_to_f64(wl.k_bits[i]) for i in ids], axis=1)[:, :n]
    v = np.concatenate([oracle.bf16_bits_to_f64(wl.v_bits[i]) for i in ids], axis=1)[:, :n]
    th = 10000.0 ** (-np.arange(r // 2) * 2.0 / r)
    pos = np.arange(n)

    def crot(x):
        z = x[..., : r // 2] + 1j * x[..., r // 2: r]
        z = z * np.exp(1j * pos[:, None] * th[None, :])
        return np.concatenate([z.real, z.imag, x[..., r:]], axis=-1)
    qt = torch.from_numpy(crot(q.transpose(1, 0, 2)))
    kt = torch.from_numpy(crot(k)).repeat_interleave(Hq // Hkv, dim=0)
    vt = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    assert np.max(np.abs(got - ref.numpy().transpose(1, 0, 2))) < 1e-12
    assert np.max(np.abs(got - oracle_out(wl))) > 1e-3      # differs from full rotary


# ---------------------------------------------------------------- document-rotated pool

def _docrot_wl():
    segs = [Segment("doc", 5, doc=0), Segment("doc", 40, doc=2), Segment("doc", 200, doc=0),
            Segment("private", 300, tokens=21)]
    return small(Hq=4, Hkv=2, D=32, segs=segs, q_len=21, seed=51)


def test_doc_rotated_pool_equals_lazy_attention():
    """Keys stored with RoPE at their positions inside their document (float64, no
    rounding): undoing the stored rotation and applying the logical one gives the lazy
    oracle's output on the un-rotated pool (doc 0 appears twice at different offsets)."""
    from oracle.docrot import doc_rotated_attention
    from tests.util import doc_stored_offsets, doc_rotated_pool
    wl = _docrot_wl()
    st = doc_stored_offsets(wl)
    kd = doc_rotated_pool(wl, st, as_bits=False)
    got = doc_rotated_attention(wl.q_bits, kd, wl.v_bits,
                                [wl.compact_ids(s) for s in range(wl.num_seqs)],
                                wl.seq_offsets, st, wl.kv_lens, wl.q_indptr, wl.q_pos,
                                wl.rope_base, wl.B)
    assert np.max(np.abs(got - oracle_out(wl))) < 1e-12
    bad = [x.copy() for x in st]
    bad[0][2] += 1                                   # one block's stored offset off by one
    worse = doc_rotated_attention(wl.q_bits, kd, wl.v_bits,
                                  [wl.compact_ids(s) for s in range(wl.num_seqs)],
                                  wl.seq_offsets, bad, wl.kv_lens, wl.q_indptr, wl.q_pos,
                                  wl.rope_base, wl.B)
    assert np.max(np.abs(worse - got)) > 1e-4


def test_doc_rotated_translation_invariance():
    """Shifting every logical offset and query position by c (stored offsets fixed) leaves
    the output unchanged: only L - p and the stored rotation enter."""
    from oracle.docrot import doc_rotated_attention
    from tests.util import doc_stored_offsets, doc_rotated_pool
    wl = _docrot_wl()
    st = doc_stored_offsets(wl)
    kd = doc_rotated_pool(wl, st)
    ids = [wl.compact_ids(s) for s in range(wl.num_seqs)]
    a = doc_rotated_attention(wl.q_bits, kd, wl.v_bits, ids, wl.seq_offsets, st, wl.kv_lens,
                              wl.q_indptr, wl.q_pos, wl.rope_base, wl.B)
    c = 123457
    b = doc_rotated_attention(wl.q_bits, kd, wl.v_bits, ids, [o + c for o in wl.seq_offsets],
                              st, wl.kv_lens, wl.q_indptr, wl.q_pos + c, wl.rope_base, wl.B)
    assert np.max(np.abs(a - b)) < 1e-10


def test_single_visible_key_returns_its_value():
    segs = [Segment("private", 10, tokens=16)]
    wl = small(segs=segs, q_len=1, q_pos=np.array([10]))
    out = oracle_out(wl)
    blk = wl.compact_ids(0)[0]
    v0 = oracle.bf16_bits_to_f64(wl.v_bits[blk, :, 0, :])           # [Hkv, D]
    G = wl.Hq // wl.Hkv
    for h in range(wl.Hq):
        assert np.array_equal(out[0, h], v0[h // G])


def test_zero_keys_give_mean_of_visible_values():
    wl = small(seed=13)
    wl.k_bits[:] = 0                                                # all scores 0
    out = oracle_out(wl)
    G = wl.Hq // wl.Hkv
    for r in range(wl.total_q):
        p = wl.q_pos[r]
        vals, pos = [], []
        for t, (bid, off) in enumerate(zip(wl.compact_ids(0), wl.seq_offsets[0])):
            n_t = 16 if t < len(wl.seq_offsets[0]) - 1 else wl.kv_lens[0] - 16 * t
            for j in range(n_t):
                if off + j <= p:
                    vals.append(oracle.bf16_bits_to_f64(wl.v_bits[bid, :, j, :]))
        mean = np.mean(vals, axis=0)
        for h in range(wl.Hq):
            assert np.max(np.abs(out[r, h] - mean[h // G])) < 1e-13


def test_no_visible_key_outputs_zero():
    segs = [Segment("doc", 50, doc=0), Segment("private", 90, tokens=3)]
    wl = small(segs=segs, q_len=2, q_pos=np.array([0, 49]))
    assert np.array_equal(oracle_out(wl), np.zeros_like(oracle_out(wl)))


def test_sequence_without_entries_outputs_zero():
    """A sequence with no block-table entries has no key, so its rows are 0; the other
    sequences of the batch are unaffected (each equals its own single-request oracle)."""
    r1 = RequestLayout([Segment("doc", 5, doc=0), Segment("private", 40, tokens=20)], 20)
    empty = RequestLayout([], 3, np.array([7, 8, 9]))
    both = build("small", 4, 2, 64, 16, 10000.0, 3, 32, [r1, empty], 11)
    alone = build("small", 4, 2, 64, 16, 10000.0, 3, 32, [r1], 11)
    out = oracle_out(both)
    assert both.kv_lens[1] == 0 and both.block_table[2] == both.block_table[1]
    assert np.array_equal(out[20:], np.zeros_like(out[20:]))
    assert np.array_equal(out[:20], oracle_out(alone))


def test_reuse_equals_copies():
    """One physical block at two offsets == two physical copies (each used once)."""
    lay_reuse = RequestLayout([Segment("doc", 0, doc=0), Segment("doc", 77, doc=0),
                               Segment("private", 140, tokens=9)], 9)
    wl = build("reuse", 4, 2, 16, 16, 10000.0, 2, 32, [lay_reuse], seed=21)
    out_reuse = oracle_out(wl)
    # copy: second placement reads doc 1, made an exact copy of doc 0
    lay_copy = RequestLayout([Segment("doc", 0, doc=0), Segment("doc", 77, doc=1),
                              Segment("private", 140, tokens=9)], 9)
    wc = build("copy", 4, 2, 16, 16, 10000.0, 2, 32, [lay_copy], seed=21)
    ids0 = wc.compact_ids(0)
    wc.k_bits[ids0[2:4]] = wc.k_bits[ids0[0:2]]
    wc.v_bits[ids0[2:4]] = wc.v_bits[ids0[0:2]]
    assert np.array_equal(oracle_out(wc), out_reuse)
    assert np.max(np.abs(brute_attention(wc) - out_reuse)) < 1e-12


def test_rotated_pool_baseline_equals_lazy():
    """The materialised baseline -- a pool whose keys already carry R(L) at the position
    they are referenced at, read as stored -- gives the same attention as the position-free
    pool with rotation applied ("Mathematical Equivalence"); checked against the
    independent brute force too."""
    segs = [Segment("doc", 3, doc=0), Segment("doc", 47, doc=1), Segment("private", 90, tokens=12)]
    wl = small(segs=segs, q_len=12, seed=23, q_scale=3.0)
    ids = [wl.compact_ids(s) for s in range(wl.num_seqs)]
    kp = oracle.rotated_pool(wl.k_bits, ids, wl.seq_offsets, wl.kv_lens, wl.B, wl.rope_base)
    base_out = oracle.lazy_attention(wl.q_bits, kp, wl.v_bits, ids, wl.seq_offsets, wl.kv_lens,
                                     wl.q_indptr, wl.q_pos, wl.rope_base, wl.B, rotate_keys=False)
    assert np.max(np.abs(base_out - oracle_out(wl))) < 1e-12
    assert np.max(np.abs(base_out - brute_attention(wl))) < 1e-12
    # and the baseline really depends on where the rotation was applied
    wrong = oracle.lazy_attention(wl.q_bits, kp, wl.v_bits, ids, wl.seq_offsets, wl.kv_lens,
                                  wl.q_indptr, wl.q_pos, wl.rope_base, wl.B)
    assert np.max(np.abs(wrong - base_out)) > 1e-3


def test_translation_invariance():
    wl = small(seed=31, q_scale=4.0)
    base_out = oracle_out(wl)
    for c in (1, 12345, 100000):
        wl2 = small(seed=31, q_scale=4.0)
        wl2.seq_offsets = [o + c for o in wl2.seq_offsets]
        wl2.q_pos = wl2.q_pos + c
        assert np.max(np.abs(oracle_out(wl2) - base_out)) < 1e-9


def test_block_table_permutation_invariance():
    segs = [Segment("doc", 0, doc=0), Segment("doc", 64, doc=1), Segment("doc", 96, doc=2),
            Segment("private", 128, tokens=32)]
    wl = small(segs=segs, q_len=32, seed=41)
    out = oracle_out(wl)
    perm = np.array([5, 0, 3, 1, 4, 2, 7, 6])      # all entries are full blocks
    wl.seq_block_ids = [wl.seq_block_ids[0][perm]]
    wl.seq_offsets = [wl.seq_offsets[0][perm]]
    assert np.max(np.abs(oracle_out(wl) - out)) < 1e-12


def test_position_matters():
    """Negative control: moving one document changes the output."""
    wl = small(seed=51, q_scale=4.0)
    out = oracle_out(wl)
    wl.seq_offsets = [wl.seq_offsets[0] + np.array([1, 1, 0, 0, 0, 0])]
    assert np.max(np.abs(oracle_out(wl) - out)) > 1e-3


# ---------------------------------------------------------------- packed words

def _golden_words():
    with open(os.path.join(GOLDEN, "packed_words.json")) as f:
        return json.load(f)


def test_packed_word_golden_bits():
    g = _golden_words()
    for c in g["cases"]:
        t = c["t"]
        ids = [0] * t + [c["block_id"]]
        offs = [16 * i for i in range(t)] + [c["offset"]]
        bt = np.array([0, t + 1])
        w = meta.encode_meta(ids, offs, bt, g["B"])
        assert int(w[-1]) == int(c["word"], 16), c
        dids, doffs = meta.decode_meta(w, bt, g["B"])
        assert int(dids[-1]) == c["block_id"] and int(doffs[-1]) == c["offset"]


def test_packed_word_roundtrip_and_range():
    rng = np.random.default_rng(4)
    bt = np.array([0, 300, 301, 1000])
    t = np.concatenate([np.arange(300), [0], np.arange(699)])
    ids = rng.integers(0, 1 << 17, size=1000)
    offs = t * 16 + rng.integers(-16384, 16384, size=1000)
    w = meta.encode_meta(ids, offs, bt, 16)
    di, do = meta.decode_meta(w, bt, 16)
    assert np.array_equal(di, ids) and np.array_equal(do, offs)
    with pytest.raises(ValueError):
        meta.encode_meta([1 << 17], [0], [0, 1], 16)
    with pytest.raises(ValueError):
        meta.encode_meta([0], [16384], [0, 1], 16)
    with pytest.raises(ValueError):
        meta.encode_meta([0], [-16385], [0, 1], 16)


# ---------------------------------------------------------------- overhead

def test_rotation_overhead_printed_value():
    with open(os.path.join(GOLDEN, "rotation_overhead.json")) as f:
        g = json.load(f)
    pct = 100.0 * overhead.rotation_overhead(g["M"])
    assert round(pct, g["printed_digits"]) == g["overhead_percent_printed"]
    assert abs(overhead.rotation_overhead(g["M"]) - 3.0 / (4 * g["M"])) < 1e-15
    # rotating twice (reset to zero, then to the target) would not match the printed figure
    twice = 100.0 * overhead.rotation_overhead(g["M"], rotations_per_key=2)
    assert round(twice, 2) != g["overhead_percent_printed"]


# ------------------------------------------------------------------ RoPE frequency tables

def test_frequency_table_equals_base_form():
    """Passing the table theta_k = base^(-2k/D) explicitly gives the same rotation."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    pos = np.array([0, 1, 77, 4000, 40000])
    assert np.array_equal(rope.rotate(x, pos, rope.inv_freq(64, 10000.0)),
                          rope.rotate(x, pos, 10000.0))


def test_zero_frequency_pairs_are_unrotated():
    theta = rope.inv_freq(32, 10000.0).copy()
    theta[::2] = 0.0
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 32))
    y = rope.rotate(x, np.array([5, 900, 31000]), theta)
    k = np.arange(0, 16, 2)
    assert np.array_equal(y[:, k], x[:, k]) and np.array_equal(y[:, k + 16], x[:, k + 16])
    assert not np.allclose(y[:, k + 1], x[:, k + 1])


def test_llama31_scaling_bands_and_continuity():
    """High frequencies (wavelength < 8192/4) unchanged, low (> 8192/1) divided by 8, the
    band between interpolated continuously; the 128-dim, base 500000 table has all three."""
    t_hi = 2 * np.pi / np.array([2047.0, 100.0, 2 * np.pi])      # w < 2048
    t_lo = 2 * np.pi / np.array([8193.0, 1e5, 3e6])              # w > 8192
    assert np.array_equal(rope.llama31_scale(t_hi), t_hi)
    assert np.array_equal(rope.llama31_scale(t_lo), t_lo / 8)
    for w in (2048.0, 8192.0):                                  # band edges: continuous
        t = 2 * np.pi / np.array([w * (1 - 1e-12), w, w * (1 + 1e-12)])
        v = rope.llama31_scale(t)
        assert np.allclose(v, v[1], rtol=1e-9)
    mid = 2 * np.pi / 4096.0                                    # r = 2: s = 1/3
    assert np.isclose(rope.llama31_scale([mid])[0], (2 / 3) * mid / 8 + (1 / 3) * mid, rtol=1e-15)
    th = rope.inv_freq(128, 500000.0)
    sc = rope.llama31_scale(th)
    w = 2 * np.pi / th
    assert (sc == th)[w < 2048].all() and (sc == th / 8)[w > 8192].all()
    assert ((w >= 2048) & (w <= 8192)).any() and (np.diff(sc) < 0).all()


def test_package_llama31_table_equals_oracle():
    from position_agnostic_kv_paged_amd.api import llama31_inv_freq
    for D in (64, 128):
        want = rope.llama31_scale(rope.inv_freq(D, 500000.0))
        assert np.allclose(llama31_inv_freq(D), want, rtol=1e-15, atol=0)


# ------------------------------------------------------------------ ALiBi

def _alibi_out(wl, slopes):
    from oracle.alibi import alibi_attention
    return alibi_attention(wl.q_bits, wl.k_bits, wl.v_bits,
                           [wl.compact_ids(s) for s in range(wl.num_seqs)], wl.seq_offsets,
                           wl.kv_lens, wl.q_indptr, wl.q_pos, slopes, wl.B)


def test_alibi_slopes_published_values():
    from oracle.alibi import alibi_slopes
    assert np.array_equal(alibi_slopes(8), 2.0 ** -np.arange(1, 9))        # 1/2 .. 1/256
    assert np.allclose(alibi_slopes(4), [2 ** -2, 2 ** -4, 2 ** -6, 2 ** -8], rtol=0, atol=0)
    s12 = alibi_slopes(12)                    # 8 of H = 8, then slopes 1, 3, 5, 7 of H = 16
    assert np.array_equal(s12[:8], alibi_slopes(8))
    assert np.allclose(s12[8:], 2.0 ** (-np.array([1, 3, 5, 7]) * 0.5), rtol=1e-15)


def test_alibi_equals_sdpa_with_explicit_bias():
    """A layout with gaps, reuse and a partial tail against torch's scaled_dot_product_attention
    given the bias -m_h (p - L) and the causal mask as an explicit additive matrix."""
    torch = pytest.importorskip("torch")
    from oracle.alibi import alibi_slopes
    segs = [Segment("doc", 3, doc=1), Segment("doc", 40, doc=0), Segment("doc", 100, doc=1),
            Segment("private", 140, tokens=21)]
    wl = small(Hq=8, Hkv=2, D=32, segs=segs, q_len=21, seed=13)
    sl = alibi_slopes(8) * 3.0
    got = _alibi_out(wl, sl)
    ids = wl.compact_ids(0)
    T = len(ids)
    n_t = [16] * (T - 1) + [int(wl.kv_lens[0]) - 16 * (T - 1)]
    k = np.concatenate([oracle.bf16_bits_to_f64(wl.k_bits[ids[t]][:, :n_t[t]]) for t in range(T)], 1)
    v = np.concatenate([oracle.bf16_bits_to_f64(wl.v_bits[ids[t]][:, :n_t[t]]) for t in range(T)], 1)
    L = np.concatenate([wl.seq_offsets[0][t] + np.arange(n_t[t]) for t in range(T)])
    p = wl.q_pos.astype(np.int64)
    bias = np.where(L[None, :] <= p[:, None], -(p[:, None] - L[None, :]).astype(float), -np.inf)
    q = torch.from_numpy(oracle.bf16_bits_to_f64(wl.q_bits).transpose(1, 0, 2).copy())
    kt = torch.from_numpy(k).repeat_interleave(4, dim=0)
    vt = torch.from_numpy(v).repeat_interleave(4, dim=0)
    mask = torch.from_numpy(sl[:, None, None] * bias[None])
    ref = torch.nn.functional.scaled_dot_product_attention(q, kt, vt, attn_mask=mask)
    assert np.max(np.abs(got - ref.numpy().transpose(1, 0, 2))) < 1e-12


def test_alibi_translation_invariance_and_limits():
    from oracle.alibi import alibi_slopes
    segs = [Segment("doc", 10, doc=0), Segment("doc", 60, doc=2), Segment("private", 95, tokens=9)]
    wl = small(Hq=4, Hkv=1, D=16, segs=segs, q_len=9, seed=14)
    shifted = [Segment(s.kind, s.start + 5000, doc=s.doc, tokens=s.tokens) for s in segs]
    wl2 = small(Hq=4, Hkv=1, D=16, segs=shifted, q_len=9, seed=14)
    sl = alibi_slopes(4)
    assert np.allclose(_alibi_out(wl, sl), _alibi_out(wl2, sl), rtol=0, atol=1e-13)
    # zero slopes: plain causal attention without position (independent of any placement
    # that keeps the visible set)
    assert np.allclose(_alibi_out(wl, np.zeros(4)), _alibi_out(wl2, np.zeros(4)), atol=1e-13)
    # a very steep slope: each row returns the value of its nearest visible key, the
    # private token at the row's own position
    out = _alibi_out(wl, np.full(4, 60.0))
    ids, offs = wl.compact_ids(0), wl.seq_offsets[0]
    for r, p in enumerate(wl.q_pos):
        t = max(i for i in range(len(offs)) if offs[i] <= p)
        want = oracle.bf16_bits_to_f64(wl.v_bits[ids[t], 0, p - offs[t]])
        assert np.allclose(out[r], want[None, :], atol=1e-12)
