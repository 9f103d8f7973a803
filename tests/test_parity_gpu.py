"""Parity of the HIP path (through the C ABI) with the float64 oracle on the same inputs.

Tolerance on bf16 outputs: max |diff| <= 2e-2 and mean |diff| <= 2e-3; packed-word
decoding bit-exact. Every case, the full-size workloads included, compares every output
element (all rows, heads and dims) with the oracle; unreferenced pool blocks and padding
slots hold NaN, so a stray read shows up as a non-finite output.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from workload import make, Segment, RequestLayout, build  # noqa: E402
from tests.util import small, oracle_out  # noqa: E402
from tests.gpu_util import run_hip, compare, say, words_for, MAX_ABS  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import position_agnostic_kv_paged_amd as L
    L.lib()


def _oracle_rows(wl, seq, rows):
    return oracle_out(wl, rows=rows, seq=seq)


# ------------------------------------------------------------------ packed words

def test_device_word_decode_bit_exact():
    import position_agnostic_kv_paged_amd as L
    wl = make("decode-32q8kv-b8-ctx32769")
    words = words_for(wl)
    bt = wl.block_table
    say("device decode of words: long-decode workload")
    ids, offs = L.debug_decode_meta(torch.from_numpy(words.view(np.int32)).cuda(),
                                    torch.from_numpy(bt).cuda())
    torch.cuda.synchronize()
    want_ids, want_offs = oracle.decode_meta(words, bt, 16)
    assert np.array_equal(ids.cpu().numpy(), want_ids)
    assert np.array_equal(offs.cpu().numpy(), want_offs)
    # boundary words
    cases_ids = np.array([0, 1, 131071, 5, 0, 131071], np.int32)
    cases_off = np.array([0, 16 - 16384, 32 + 16383, 48 - 1, 64 + 7, 80], np.int64)
    bt2 = np.array([0, 6], np.int32)
    w2 = L.encode_meta(cases_ids, cases_off, bt2)
    ids, offs = L.debug_decode_meta(torch.from_numpy(w2.view(np.int32)).cuda(),
                                    torch.from_numpy(bt2).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), cases_ids)
    assert np.array_equal(offs.cpu().numpy(), cases_off)


# ------------------------------------------------------------------ tiny configuration

@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_tiny_prefill_config(kind):
    wl = make("tiny-prefill-4q1kv-d64")
    say(f"tiny prefill config via {kind}")
    compare(run_hip(wl, kind), oracle_out(wl), f"tiny/{kind}")


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_tiny_decode_variant(kind):
    wl = make("tiny-prefill-4q1kv-d64", decode_variant=True)
    say(f"tiny decode variant via {kind}")
    compare(run_hip(wl, kind), oracle_out(wl), f"tiny-decode/{kind}")


# ------------------------------------------------------------------ adversarial mini-cases

def _mini_cases():
    cases = []
    for D in (64, 128):
        for Hq, Hkv in ((4, 4), (4, 2), (8, 2), (8, 1)):
            cases.append((f"gaps-D{D}-G{Hq // Hkv}", dict(Hq=Hq, Hkv=Hkv, D=D, seed=D + Hq)))
    segs_overlap = [Segment("doc", 3, doc=1), Segment("doc", 20, doc=0),
                    Segment("doc", 100, doc=1), Segment("private", 140, tokens=21)]
    cases.append(("overlap-repeat-partial", dict(Hq=8, Hkv=2, D=128, segs=segs_overlap,
                                                 q_len=21, seed=3, q_scale=4.0)))
    # 550 two-block placements back-to-back from 16000 (delta = 16000 stays in the word's
    # 15-bit range): key and query positions run past 2^15
    segs_far = [Segment("doc", 16000 + 32 * i, doc=i % 3) for i in range(550)] + \
        [Segment("private", 16000 + 32 * 550, tokens=37)]
    cases.append(("positions-above-2^15", dict(Hq=4, Hkv=1, D=128, segs=segs_far, q_len=37,
                                               seed=4, q_scale=4.0)))
    segs_zero = [Segment("doc", 50, doc=0), Segment("private", 90, tokens=3)]
    cases.append(("no-visible-key", dict(Hq=4, Hkv=2, D=64, segs=segs_zero, q_len=2,
                                         q_pos=np.array([0, 49]), seed=5)))
    segs_long = [Segment("doc", 7 + 32 * i, doc=i % 3) for i in range(9)] + \
        [Segment("private", 7 + 32 * 9, tokens=150)]
    cases.append(("many-tiles-ragged", dict(Hq=8, Hkv=2, D=128, segs=segs_long, q_len=150,
                                            seed=6)))
    # 16 query heads per KV head (decode: heads in the 16 MFMA columns, q' set per block)
    cases.append(("gaps-D128-G16", dict(Hq=16, Hkv=1, D=128, seed=21)))
    cases.append(("gaps-D64-G16", dict(Hq=32, Hkv=2, D=64, seed=22)))
    cases.append(("overlap-repeat-partial-G16", dict(Hq=16, Hkv=1, D=128, segs=segs_overlap,
                                                     q_len=21, seed=23, q_scale=4.0)))
    cases.append(("positions-above-2^15-G16", dict(Hq=16, Hkv=1, D=128, segs=segs_far,
                                                   q_len=37, seed=24, q_scale=4.0)))
    cases.append(("many-tiles-ragged-G16", dict(Hq=32, Hkv=2, D=128, segs=segs_long,
                                                q_len=150, seed=25)))
    # more than 16 query heads per KV head (multi-query attention): each KV head is split
    # into 16-head groups that read the same pool head
    cases.append(("gaps-D128-G32", dict(Hq=32, Hkv=1, D=128, seed=41)))
    cases.append(("gaps-D64-G32-2kv", dict(Hq=64, Hkv=2, D=64, seed=42)))
    cases.append(("overlap-repeat-partial-G64", dict(Hq=64, Hkv=1, D=128, segs=segs_overlap,
                                                     q_len=21, seed=43, q_scale=4.0)))
    cases.append(("many-tiles-ragged-G48", dict(Hq=48, Hkv=1, D=128, segs=segs_long,
                                                q_len=150, seed=44)))
    return cases


@pytest.mark.parametrize("kind", ["prefill", "decode"])
@pytest.mark.parametrize("name,kw", _mini_cases(), ids=[c[0] for c in _mini_cases()])
def test_mini_cases(name, kw, kind):
    wl = small(**kw)
    say(f"mini case {name} via {kind}")
    compare(run_hip(wl, kind), oracle_out(wl), f"{name}/{kind}")


def _freq_tables(D):
    """name -> (table given to the HIP entry point, table given to the oracle). The Llama
    3.1 table comes from the library's host helper on the HIP side and from the oracle's own
    scaling on the oracle side, so the two sides share no arithmetic."""
    import position_agnostic_kv_paged_amd as L
    half_zero = oracle.rope.inv_freq(D, 10000.0).copy()
    half_zero[::2] = 0.0                                 # every other pair unrotated
    interp = oracle.rope.inv_freq(D, 10000.0) / 4.0      # position interpolation by 4
    llama = oracle.rope.llama31_scale(oracle.rope.inv_freq(D, 500000.0))
    return {"llama31": (L.llama31_inv_freq(D), llama), "half-zero": (half_zero, half_zero),
            "interp4": (interp, interp)}


@pytest.mark.parametrize("kind", ["prefill", "decode"])
@pytest.mark.parametrize("table", ["llama31", "half-zero", "interp4"])
@pytest.mark.parametrize("name", ["gaps-D128-G4", "gaps-D64-G2", "positions-above-2^15",
                                  "many-tiles-ragged"])
def test_frequency_tables(name, table, kind):
    """lazyattn_*_freqs with frequency-scaled RoPE tables against the oracle with the same
    table (Llama 3.1 scaling at base 500000, zero-frequency pairs, position interpolation)."""
    kw = dict(_mini_cases())[name]
    wl = small(**kw)
    th_hip, th_oracle = _freq_tables(wl.D)[table]
    say(f"frequency table {table} on {name} via {kind}")
    compare(run_hip(wl, kind, inv_freq=th_hip), oracle_out(wl, base=th_oracle),
            f"{name}/{table}/{kind}")


_PARTIAL = [("gaps-D128-G4", 32), ("gaps-D128-G4", 64), ("gaps-D128-G4", 112),
            ("gaps-D64-G2", 16), ("gaps-D64-G2", 48), ("positions-above-2^15", 16),
            ("many-tiles-ragged", 64), ("overlap-repeat-partial", 32), ("gaps-D128-G16", 32),
            ("gaps-D128-G32", 64)]


@pytest.mark.parametrize("kind", ["prefill", "decode"])
@pytest.mark.parametrize("name,r", _PARTIAL, ids=[f"{n}-r{r}" for n, r in _PARTIAL])
def test_partial_rotary(name, r, kind):
    """lazyattn_*_partial (rotate-half inside the first r dims, the rest unrotated) against
    the oracle's partial rotary on the same workload."""
    wl = small(**dict(_mini_cases())[name])
    say(f"partial rotary r = {r} on {name} via {kind}")
    compare(run_hip(wl, kind, rotary_dim=r), oracle_out(wl, rotary_dim=r),
            f"{name}/r{r}/{kind}")


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_partial_rotary_full_size(kind):
    """Partial rotary (r = 32 of 128) on the full-size Zipf batches, every row."""
    wl = make("decode-32q8kv-b64-ctx4161" if kind == "decode" else "prefill-32q8kv-b16-ctx5376")
    say(f"partial rotary r = 32 on {wl.name} via {kind}")
    _full_check(wl, kind, f"{wl.name}/r32", rotary_dim=32)


_DOCROT = ["gaps-D128-G4", "gaps-D64-G2", "overlap-repeat-partial", "positions-above-2^15",
           "many-tiles-ragged", "gaps-D128-G16", "many-tiles-ragged-G16", "gaps-D128-G32",
           "gaps-D128-G1"]


def _docrot_case(wl, stored):
    """(workload whose K pool holds keys rotated at the stored offsets, oracle output)."""
    import dataclasses
    from oracle.docrot import doc_rotated_attention
    from tests.util import doc_rotated_pool
    kd = doc_rotated_pool(wl, stored)
    want = doc_rotated_attention(wl.q_bits, kd, wl.v_bits,
                                 [wl.compact_ids(s) for s in range(wl.num_seqs)],
                                 wl.seq_offsets, stored, wl.kv_lens, wl.q_indptr, wl.q_pos,
                                 wl.rope_base, wl.B)
    return dataclasses.replace(wl, k_bits=kd), want


@pytest.mark.parametrize("kind", ["prefill", "decode"])
@pytest.mark.parametrize("name", _DOCROT)
def test_doc_rotated_pool(name, kind):
    """lazyattn_*_doc_rotated over a pool whose document keys carry RoPE at their positions
    inside the document (block b at 16 b) and private keys at their logical positions."""
    from tests.util import doc_stored_offsets
    wl = small(**dict(_mini_cases())[name])
    st = doc_stored_offsets(wl)
    wd, want = _docrot_case(wl, st)
    say(f"document-rotated pool on {name} via {kind}")
    compare(run_hip(wd, kind, stored=st), want, f"{name}/docrot/{kind}")


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_doc_rotated_pool_at_logical_offsets(kind):
    """Stored offsets equal to the logical offsets (every block rotated where it is used):
    the materialised pool, through the document-rotated entry points."""
    wl = small(**dict(_mini_cases())["gaps-D128-G4"])      # every block referenced once
    st = [np.asarray(o, dtype=np.int64) for o in wl.seq_offsets]
    wd, want = _docrot_case(wl, st)
    compare(run_hip(wd, kind, stored=st), want, f"docrot-logical/{kind}")
    assert np.max(np.abs(want - oracle_out(wl))) < 1e-2          # the same attention


def test_doc_rotated_pool_full_size_decode():
    """Document-rotated pool on the 64-request decode batch (Zipf documents reused at
    per-request offsets), every row."""
    from tests.util import doc_stored_offsets
    wl = make("decode-32q8kv-b64-ctx4161")
    st = doc_stored_offsets(wl)
    wd, want = _docrot_case(wl, st)
    say("document-rotated pool on decode-32q8kv-b64-ctx4161 via decode")
    compare(run_hip(wd, "decode", stored=st), want, "decode-b64/docrot")


@pytest.mark.parametrize("variant", ["partial-r32", "doc-rotated"])
def test_variants_mixed_batch_with_empty_sequences(variant):
    """Partial rotary and the document-rotated pool in one call holding prefill, decode,
    zero-query and entry-less requests (through lazyattn_prefill_*, which routes single-row
    requests to the decode kernel)."""
    segs = [Segment("doc", 11, doc=0), Segment("doc", 60, doc=1),
            Segment("private", 100, tokens=70)]
    reqs = [RequestLayout([], 1, np.array([3])),
            RequestLayout(segs, 70),
            RequestLayout([Segment("doc", 0, doc=2), Segment("private", 32, tokens=5)], 1),
            RequestLayout([Segment("doc", 0, doc=1), Segment("private", 32, tokens=2)], 0),
            RequestLayout([], 2, np.array([0, 5]))]
    wl = build("mixed-empty", 16, 2, 128, 16, 10000.0, 3, 32, reqs, seed=61)
    say(f"{variant} on a mixed batch with empty requests")
    if variant == "partial-r32":
        got, want = run_hip(wl, "prefill", rotary_dim=32), oracle_out(wl, rotary_dim=32)
    else:
        from tests.util import doc_stored_offsets
        st = doc_stored_offsets(wl)
        wd, want = _docrot_case(wl, st)
        got = run_hip(wd, "prefill", stored=st)
    compare(got, want, f"mixed-empty/{variant}")
    for s in (0, 4):
        r0, r1 = int(wl.q_indptr[s]), int(wl.q_indptr[s + 1])
        assert np.array_equal(got[r0:r1], np.zeros_like(got[r0:r1]))


def _alibi_ref(wl, slopes):
    from oracle.alibi import alibi_attention
    return alibi_attention(wl.q_bits, wl.k_bits, wl.v_bits,
                           [wl.compact_ids(s) for s in range(wl.num_seqs)], wl.seq_offsets,
                           wl.kv_lens, wl.q_indptr, wl.q_pos, slopes, wl.B)


@pytest.mark.parametrize("kind", ["prefill", "decode"])
@pytest.mark.parametrize("name,kw", _mini_cases(), ids=[c[0] for c in _mini_cases()])
def test_alibi_mini_cases(name, kw, kind):
    """lazyattn_*_alibi over the position-free pool against the float64 ALiBi definition:
    the paper's slopes, four times steeper on the peaky (x4 query scale) cases."""
    from oracle.alibi import alibi_slopes
    wl = small(**kw)
    sl = alibi_slopes(wl.Hq) * (4.0 if kw.get("q_scale", 1.0) > 1.0 else 1.0)
    say(f"ALiBi mini case {name} via {kind}")
    compare(run_hip(wl, kind, slopes=sl), _alibi_ref(wl, sl), f"alibi/{name}/{kind}")


def test_alibi_mixed_batch_and_zero_slopes():
    """A mixed batch through lazyattn_prefill_alibi, and zero slopes (no positional term)."""
    from oracle.alibi import alibi_slopes
    reqs = [RequestLayout([Segment("doc", 11, doc=0), Segment("doc", 60, doc=1),
                           Segment("private", 100, tokens=70)], 70),
            RequestLayout([Segment("doc", 0, doc=2), Segment("private", 32, tokens=5)], 1),
            RequestLayout([Segment("doc", 500, doc=2), Segment("doc", 5, doc=0),
                           Segment("private", 600, tokens=17)], 1)]
    wl = build("mixed-small", 8, 2, 128, 16, 10000.0, 3, 32, reqs, seed=18)
    for sl in (alibi_slopes(8), np.zeros(8)):
        say(f"ALiBi mixed batch, slopes {sl[:2]}")
        compare(run_hip(wl, "prefill", slopes=sl), _alibi_ref(wl, sl), "alibi/mixed/prefill")
        compare(run_hip(wl, "decode", slopes=sl), _alibi_ref(wl, sl), "alibi/mixed/decode")


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_sequences_without_entries(kind):
    """Sequences with no block-table entries (first, middle and last of the batch) give 0
    rows and leave the others exact; the last one's table starts at the end of the words."""
    segs = [Segment("doc", 5, doc=0), Segment("doc", 40, doc=2),
            Segment("private", 72, tokens=20)]
    nq = 20 if kind == "prefill" else 1
    ne = 2 if kind == "prefill" else 1
    full = RequestLayout(segs, nq)
    empty = RequestLayout([], ne, np.array([7, 9][:ne]))
    wl = build("small", 8, 2, 128, 16, 10000.0, 3, 32, [empty, full, empty, full, empty], 12)
    say(f"sequences without entries via {kind}")
    assert wl.kv_lens[-1] == 0 and wl.block_table[-1] == wl.block_table[-2]
    got, want = run_hip(wl, kind), oracle_out(wl)
    compare(got, want, f"empty-sequences/{kind}")
    for s in (0, 2, 4):
        r0, r1 = int(wl.q_indptr[s]), int(wl.q_indptr[s + 1])
        assert np.array_equal(got[r0:r1], np.zeros_like(got[r0:r1]))


def test_mixed_batch_small():
    """One call with prefill (q_len > 1), decode (q_len = 1) and empty (q_len = 0) requests."""
    reqs = [RequestLayout([Segment("doc", 11, doc=0), Segment("doc", 60, doc=1),
                           Segment("private", 100, tokens=70)], 70),
            RequestLayout([Segment("doc", 0, doc=2), Segment("private", 32, tokens=5)], 1),
            RequestLayout([Segment("doc", 0, doc=1), Segment("private", 32, tokens=2)], 0),
            RequestLayout([Segment("doc", 500, doc=2), Segment("doc", 5, doc=0),
                           Segment("private", 600, tokens=17)], 1)]
    wl = build("mixed-small", 8, 1, 128, 16, 10000.0, 3, 32, reqs, seed=8)
    say("mixed small batch via prefill")
    compare(run_hip(wl, "prefill"), oracle_out(wl), "mixed-small/prefill")
    compare(run_hip(wl, "decode"), oracle_out(wl), "mixed-small/decode")


@pytest.mark.parametrize("Hkv,G", [(3, 4), (6, 2)])
def test_kv_heads_straddling_xcd_ranges(Hkv, G):
    """Decode items are numbered head-major and cut into eight contiguous ranges, one per XCD
    (the mixed kernel cuts its decode chunks the same way). With 3 or 6 KV heads the ranges
    start inside heads. Every row against the oracle: a decode batch, and the same rows with
    prefill requests between them in one mixed call."""
    dec = [RequestLayout([Segment("doc", 5 + i, doc=i % 4), Segment("doc", 100 + 2 * i, doc=(i + 1) % 4),
                          Segment("private", 240 + 3 * i, tokens=3 + i % 5)], 1) for i in range(40)]
    pre = RequestLayout([Segment("doc", 17, doc=2), Segment("private", 90, tokens=20)], 20)
    for name, reqs, kind in (("decode", dec, "decode"),
                             ("mixed", [pre] + dec[:20] + [pre] + dec[20:], "prefill")):
        wl = build(f"straddle-{Hkv}kv-{name}", Hkv * G, Hkv, 128, 16, 10000.0, 4, 48, reqs,
                   seed=31 + Hkv)
        say(f"KV heads {Hkv}, {name} batch via {kind}")
        compare(run_hip(wl, kind), oracle_out(wl), f"straddle-{Hkv}kv/{name}")


def _distinct_cases():
    """Layouts in which every pool block is referenced once (a rotated pool can hold it)."""
    segs = [Segment("doc", 7 + 32 * i + 3 * (i % 2), doc=i) for i in range(9)] + \
        [Segment("private", 7 + 32 * 9 + 5, tokens=150)]
    one = dict(Hq=8, Hkv=2, D=128, n_docs=9, segs=segs, q_len=150, seed=12, q_scale=3.0)
    reqs = [RequestLayout([Segment("doc", 11, doc=0), Segment("doc", 60, doc=1),
                           Segment("private", 100, tokens=9)], 1),
            RequestLayout([Segment("doc", 400, doc=2), Segment("doc", 3, doc=3),
                           Segment("private", 700, tokens=33)], 1),
            RequestLayout([Segment("doc", 1000, doc=4), Segment("private", 1040, tokens=5)], 5)]
    multi = dict(Hq=4, Hkv=1, D=64, n_docs=5, requests=reqs, seed=13)
    return [("distinct-one-request-D128", one), ("distinct-multi-request-D64", multi)]


@pytest.mark.parametrize("kind", ["prefill", "decode"])
@pytest.mark.parametrize("name,kw", _distinct_cases(), ids=[c[0] for c in _distinct_cases()])
def test_rotated_pool_baseline(name, kw, kind):
    """The materialised-baseline entry points over a pool that holds every key rotated to
    the position it is referenced at (built on the host in float64, rounded to bf16)
    against the oracle reading that pool as stored."""
    import torch
    import oracle
    import position_agnostic_kv_paged_amd as L
    from workload import f32_to_bf16_bits
    wl = small(**kw)
    ids = [wl.compact_ids(s) for s in range(wl.num_seqs)]
    kp = oracle.rotated_pool(wl.k_bits, ids, wl.seq_offsets, wl.kv_lens, wl.B, wl.rope_base)
    kp_bits = wl.k_bits.copy()                  # unreferenced slots keep their NaN fill
    fin = np.isfinite(kp)
    kp_bits[fin] = f32_to_bf16_bits(kp[fin].astype(np.float32))
    want = oracle.lazy_attention(wl.q_bits, kp_bits, wl.v_bits, ids, wl.seq_offsets,
                                 wl.kv_lens, wl.q_indptr, wl.q_pos, wl.rope_base, wl.B,
                                 rotate_keys=False)
    t = wl.to_device("cuda")
    t["k_pool"] = torch.from_numpy(kp_bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    meta = torch.from_numpy(np.ascontiguousarray(words_for(wl)).view(np.int32)).to("cuda")
    fn = L.prefill_rotated_pool if kind == "prefill" else L.decode_rotated_pool
    say(f"rotated-pool baseline {name} via {kind}")
    out = fn(t["q"], t["k_pool"], t["v_pool"], t["block_table"], meta, t["kv_lens"],
             t["q_indptr"], t["q_pos"], wl.rope_base, max(len(x) for x in wl.seq_block_ids))
    torch.cuda.synchronize()
    compare(out.float().cpu().numpy().astype(np.float64), want, f"{name}/{kind}-baseline")


def _materialize_cases():
    segs_overlap = [Segment("doc", 3, doc=1), Segment("doc", 20, doc=0),
                    Segment("doc", 100, doc=1), Segment("private", 140, tokens=21)]
    return _distinct_cases() + [
        ("overlap-repeat-partial", dict(Hq=8, Hkv=2, D=128, segs=segs_overlap, q_len=21,
                                        seed=3, q_scale=4.0))]


@pytest.mark.parametrize("name,kw", _materialize_cases(), ids=[c[0] for c in _materialize_cases()])
def test_materialize_rotated(name, kw):
    """lazyattn_materialize_rotated writes, for every entry, its keys rotated to their
    logical positions (within one bf16 ulp of the oracle's float64 rotation), its values
    (bit for bit) and a word naming the private block; attention over that copy through the
    baseline entry points matches the oracle on the original position-free inputs (blocks
    reused at several offsets get one copy per placement)."""
    import torch
    import oracle
    import position_agnostic_kv_paged_amd as L
    from oracle.attention import bf16_bits_to_f64
    from workload import f32_to_bf16_bits
    wl = small(**kw)
    t = wl.to_device("cuda")
    words = words_for(wl)
    meta = torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to("cuda")
    n = int(wl.block_table[-1])
    say(f"materialize {name}: {n} entries")
    dk, dv, dm = L.materialize_rotated(t["k_pool"], t["v_pool"], t["block_table"], meta,
                                       t["kv_lens"], wl.rope_base, n)
    torch.cuda.synchronize()
    got_k = dk.view(torch.int16).cpu().numpy().view(np.uint16)
    got_v = dv.view(torch.int16).cpu().numpy().view(np.uint16)
    got_m = dm.cpu().numpy().view(np.uint32)
    # expected, from the oracle's definitions (host only)
    exp_k = np.zeros_like(got_k)
    exp_v = np.zeros_like(got_v)
    for s_ in range(wl.num_seqs):
        ids = wl.compact_ids(s_)
        T = len(ids)
        for t_ in range(T):
            e = int(wl.block_table[s_]) + t_
            n_t = wl.B if t_ < T - 1 else int(wl.kv_lens[s_]) - (T - 1) * wl.B
            pos = int(wl.seq_offsets[s_][t_]) + np.arange(n_t)
            kk = bf16_bits_to_f64(wl.k_bits[ids[t_]][:, :n_t, :])
            rot = oracle.rope.rotate(kk, pos[None, :], wl.rope_base)
            exp_k[e, :, :n_t] = f32_to_bf16_bits(rot.astype(np.float32))
            exp_v[e, :, :n_t] = wl.v_bits[ids[t_]][:, :n_t, :]
    diff = np.abs(got_k.astype(np.int32) - exp_k.astype(np.int32))
    say(f"  keys: {np.count_nonzero(diff)} of {diff.size} bit patterns differ, max {diff.max()}")
    assert diff.max() <= 1 and np.count_nonzero(diff) <= 1e-3 * diff.size
    assert np.array_equal(got_v, exp_v)
    exp_m = oracle.encode_meta(np.arange(n), np.concatenate(wl.seq_offsets), wl.block_table, wl.B)
    assert np.array_equal(got_m, np.asarray(exp_m, dtype=np.uint32))
    # attention over the copy: to parity with the oracle reading the host-built copy as
    # stored; against LazyAttention's definition the copy's bf16 rounding of rotated keys
    # (8 mantissa bits, where the lazy kernels keep rotated keys in fp16) costs up to about
    # 2.5e-2 on the x4-query stress layout, so that comparison gets a looser bound
    host_copy_k = exp_k
    want_copy = oracle.lazy_attention(wl.q_bits, host_copy_k, exp_v, [np.arange(n)[int(wl.block_table[s_]):int(wl.block_table[s_ + 1])] for s_ in range(wl.num_seqs)],
                                      wl.seq_offsets, wl.kv_lens, wl.q_indptr, wl.q_pos,
                                      wl.rope_base, wl.B, rotate_keys=False)
    want_lazy = oracle_out(wl)
    for kind, fn in (("prefill", L.prefill_rotated_pool), ("decode", L.decode_rotated_pool)):
        out = fn(t["q"], dk, dv, t["block_table"], dm, t["kv_lens"], t["q_indptr"], t["q_pos"],
                 wl.rope_base, max(len(x) for x in wl.seq_block_ids))
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        compare(got, want_copy, f"{name}/copy+{kind}")
        d = float(np.abs(got - want_lazy).max())
        say(f"  {name}/copy+{kind} vs the position-free definition: max_abs={d:.3e}")
        assert d <= 3 * MAX_ABS


# ------------------------------------------------------------------ properties

def test_reuse_equals_copy_bitwise_on_gpu():
    lay_reuse = RequestLayout([Segment("doc", 0, doc=0), Segment("doc", 77, doc=0),
                               Segment("private", 140, tokens=9)], 9)
    lay_copy = RequestLayout([Segment("doc", 0, doc=0), Segment("doc", 77, doc=1),
                              Segment("private", 140, tokens=9)], 9)
    w1 = build("reuse", 8, 2, 128, 16, 10000.0, 2, 32, [lay_reuse], seed=21)
    w2 = build("copy", 8, 2, 128, 16, 10000.0, 2, 32, [lay_copy], seed=21)
    ids = w2.compact_ids(0)
    w2.k_bits[ids[2:4]] = w2.k_bits[ids[0:2]]
    w2.v_bits[ids[2:4]] = w2.v_bits[ids[0:2]]
    for kind in ("prefill", "decode"):
        say(f"reuse vs copy via {kind}")
        a, b = run_hip(w1, kind), run_hip(w2, kind)
        assert np.array_equal(a, b)
        compare(a, oracle_out(w1), f"reuse/{kind}")


def test_run_to_run_bitwise_determinism():
    wl = make("prefill-32q8kv-b16-ctx5376")
    say("determinism: prefill workload twice")
    a, b = run_hip(wl, "prefill", repeat=2)
    assert np.array_equal(a, b)
    wd = make("decode-32q8kv-b64-ctx4161")
    say("determinism: decode workload twice")
    a, b = run_hip(wd, "decode", repeat=2)
    assert np.array_equal(a, b)
    wm = make("mixed-64q8kv-4p96d")                   # G = 8, prefill tiles and decode rows
    say("determinism: mixed batch three times (one call)")
    outs = run_hip(wm, "prefill", repeat=3)
    assert all(np.array_equal(outs[0], x) for x in outs[1:])


def test_shifted_document_is_detected():
    """The comparison sees a one-position error in a document placement."""
    wl = small(Hq=8, Hkv=2, D=128, seed=77, q_scale=4.0)
    good = oracle_out(wl)
    wl.seq_offsets = [wl.seq_offsets[0] + np.array([1, 1, 0, 0, 0, 0])]
    got = run_hip(wl, "prefill")
    assert np.max(np.abs(got - good)) > 2e-2


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_negative_control_rotation_compiled_out(kind):
    """Negative control: the kernels with the key rotation compiled out (the materialised
    baseline's entry points, which expect every key already rotated to its position) run on
    the position-free pool must fail the tolerance against the oracle. The parity bar can
    therefore see a missing rotation. The same call with the rotation passes."""
    import torch
    import position_agnostic_kv_paged_amd as L
    wl = small(Hq=8, Hkv=2, D=128, seed=91, q_scale=4.0)
    want = oracle_out(wl)
    t = wl.to_device("cuda")
    meta = torch.from_numpy(np.ascontiguousarray(words_for(wl)).view(np.int32)).to("cuda")
    fn = L.prefill_rotated_pool if kind == "prefill" else L.decode_rotated_pool
    say(f"negative control: rotation compiled out via {kind}")
    out = fn(t["q"], t["k_pool"], t["v_pool"], t["block_table"], meta, t["kv_lens"],
             t["q_indptr"], t["q_pos"], wl.rope_base, max(len(x) for x in wl.seq_block_ids))
    torch.cuda.synchronize()
    bad = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(bad))
    assert np.max(np.abs(bad - want)) > 2e-2 or np.mean(np.abs(bad - want)) > 2e-3
    compare(run_hip(wl, kind), want, f"negative-control-reference/{kind}")


# ------------------------------------------------------------------ full-size workloads

def _full_check(wl, kind, label, inv_freq=None, oracle_base=None, slopes=None,
                rotary_dim=None):
    """Every output element of a full-size call against the oracle on the same inputs."""
    got = run_hip(wl, kind, inv_freq=inv_freq, slopes=slopes, rotary_dim=rotary_dim)
    if slopes is not None:
        want = _alibi_ref(wl, slopes)
    else:
        want = oracle_out(wl, base=oracle_base, rotary_dim=rotary_dim)
    return compare(got, want, label)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("q_scale", [1.0, 4.0])
def test_decode_llama8b_batch64(q_scale):
    wl = make("decode-32q8kv-b64-ctx4161", q_scale=q_scale)
    say(f"{wl.name} via decode, every row")
    _full_check(wl, "decode", wl.name)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("q_scale", [1.0, 4.0])
def test_prefill_llama8b_batch16(q_scale):
    wl = make("prefill-32q8kv-b16-ctx5376", q_scale=q_scale)
    say(f"{wl.name} via prefill, every row")
    _full_check(wl, "prefill", wl.name)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("q_scale", [1.0, 4.0])
def test_long_decode_batch8(q_scale):
    wl = make("decode-32q8kv-b8-ctx32769", q_scale=q_scale)
    say(f"{wl.name} via decode, every row")
    _full_check(wl, "decode", wl.name)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("q_scale", [1.0, 4.0])
def test_mixed_70b_batch(q_scale):
    """The 4-prefill + 96-decode batch in one lazyattn_prefill call, every row."""
    wl = make("mixed-64q8kv-4p96d", q_scale=q_scale)
    say(f"{wl.name} via prefill (one call), every row")
    _full_check(wl, "prefill", wl.name)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("q_scale", [1.0, 4.0])
def test_kv_split_one_long_request(q_scale):
    """One request, 256 queries over 32,512 keys: 32 query tiles in all (4 per KV head),
    too few for the GPU, so each tile's key range is split and the splits are merged by the
    tile's last one. Every row against the oracle."""
    wl = make("prefill-32q8kv-b1-ctx32512", q_scale=q_scale)
    say(f"{wl.name} via prefill (KV split), every row")
    _full_check(wl, "prefill", wl.name)


def _split_cases():
    """Small layouts long enough (> 512 keys) to be KV-split: uneven split boundaries,
    queries whose causal window ends inside an early split, a mixed batch with decode rows
    and an entry-less request, G from 1 to 16."""
    cases = []
    segs = [Segment("doc", 5 + 40 * i, doc=i % 4) for i in range(25)] + \
        [Segment("private", 5 + 40 * 25 + 3, tokens=300)]
    cases.append(("split-one-request-G1-D64", dict(Hq=2, Hkv=2, D=64, segs=segs, q_len=300,
                                                   n_docs=4, seed=51)))
    cases.append(("split-one-request-G4-peaky", dict(Hq=8, Hkv=2, D=128, segs=segs, q_len=300,
                                                     n_docs=4, seed=52, q_scale=4.0)))
    early = np.concatenate([np.arange(40, 140), 1000 + np.arange(60), [1305]])
    cases.append(("split-early-queries", dict(Hq=8, Hkv=1, D=128, segs=segs, q_len=161,
                                              q_pos=early, n_docs=4, seed=53)))
    cases.append(("split-G16", dict(Hq=16, Hkv=1, D=128, segs=segs, q_len=77, n_docs=4,
                                    seed=54)))
    reqs = [RequestLayout(segs, 130),
            RequestLayout([Segment("doc", 0, doc=2), Segment("private", 32, tokens=5)], 1),
            RequestLayout([], 1, np.array([3])),
            RequestLayout([Segment("doc", 9 + 32 * i, doc=i % 4) for i in range(30)] +
                          [Segment("private", 9 + 32 * 30, tokens=40)], 40)]
    cases.append(("split-mixed-batch", dict(Hq=8, Hkv=2, D=128, requests=reqs, n_docs=4,
                                            seed=55)))
    return cases


@pytest.mark.parametrize("name,kw", _split_cases(), ids=[c[0] for c in _split_cases()])
def test_kv_split_cases(name, kw):
    wl = small(**kw)
    say(f"KV split case {name}: kv_lens {list(wl.kv_lens)}")
    compare(run_hip(wl, "prefill"), oracle_out(wl), f"{name}/prefill")


@pytest.mark.parametrize("bound", [1, 9, 100000])
def test_kv_split_max_entries_hint(bound):
    """A max_entries hint below or far above the real length changes only the KV split."""
    wl = small(**dict(_split_cases())["split-mixed-batch"])
    say(f"KV split, max_entries = {bound}")
    compare(run_hip(wl, "prefill", max_entries=bound), oracle_out(wl), f"split-hint{bound}")


@pytest.mark.timeout(300)
def test_shifted_document_is_detected_full_size():
    """Detection at full size: the long-decode batch with peaky queries, one document of
    every request placed one position later in the words the GPU gets. The GPU output must
    match the oracle on the shifted layout and miss the tolerance against the unshifted one,
    so the full-size comparison sees a one-position placement error."""
    import dataclasses
    wl = make("decode-32q8kv-b8-ctx32769", q_scale=4.0)
    offs = [o.copy() for o in wl.seq_offsets]
    for s in range(wl.num_seqs):
        offs[s][32 * 20: 32 * 21] += 1                # document 20 of each request (32 blocks)
    shifted = dataclasses.replace(wl, seq_offsets=offs)
    say("long decode, peaky, document 20 of every request shifted by one position")
    got = run_hip(shifted, "decode")
    compare(got, oracle_out(shifted), "long-decode-shifted/vs-shifted")
    want = oracle_out(wl)
    d = np.abs(got - want)
    say(f"  vs the unshifted layout: max_abs={d.max():.3e} mean_abs={d.mean():.3e}")
    assert d.max() > MAX_ABS


@pytest.mark.timeout(300)
@pytest.mark.parametrize("variant", ["alibi", "llama31"])
@pytest.mark.parametrize("name,kind", [("decode-32q8kv-b64-ctx4161", "decode"),
                                       ("prefill-32q8kv-b16-ctx5376", "prefill"),
                                       ("decode-32q8kv-b8-ctx32769", "decode")])
def test_full_size_variants(name, kind, variant):
    """The ALiBi and frequency-table entry points on the full-size workloads (positions up
    to ~35k), every row against the oracle."""
    import position_agnostic_kv_paged_amd as L
    from oracle.alibi import alibi_slopes
    wl = make(name)
    say(f"{name} via {kind}, {variant}")
    if variant == "alibi":
        _full_check(wl, kind, f"{name}/{variant}", slopes=alibi_slopes(wl.Hq))
    else:
        _full_check(wl, kind, f"{name}/{variant}", inv_freq=L.llama31_inv_freq(wl.D),
                    oracle_base=oracle.rope.llama31_scale(oracle.rope.inv_freq(wl.D, 500000.0)))


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_gqa16_405b_shape(kind):
    """128 query heads over 8 KV heads (G = 16), head dim 128: 12 requests of 6 Zipf
    documents x 512 tokens at per-request offsets plus a 48-token question; every row."""
    rng = np.random.default_rng(31)
    reqs = []
    for r in range(12):
        start = int(rng.integers(0, 512))
        docs = rng.choice(40, size=6, replace=False)
        segs = [Segment("doc", start + 512 * i, doc=int(d)) for i, d in enumerate(docs)]
        segs.append(Segment("private", start + 512 * 6, tokens=48))
        reqs.append(RequestLayout(segs, 48 if kind == "prefill" else 1))
    wl = build("gqa16", 128, 8, 128, 16, 10000.0, 40, 512, reqs, seed=32)
    say(f"G = 16 (128 q / 8 kv heads) via {kind}")
    _full_check(wl, kind, f"gqa16/{kind}")


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_operand_range_equal_huge_scores(kind):
    """Scores near the stated range: with an all-zero frequency table nothing is rotated,
    and every key and query element is 100, so every visible score is
    128 * 100 * 100 / sqrt(128) (1.6e5 in the log2 domain, past fp16's 65504). All scores
    are equal, so each row is the mean of its visible values (the oracle's float64 result);
    a running maximum kept in fp16 would overflow to inf here."""
    import dataclasses
    wl = small(Hq=8, Hkv=2, D=128, seed=81)
    hundred = np.uint16(0x42C8)                           # bf16 100.0
    fin = wl.k_bits != np.uint16(0x7FC0)                  # keep the NaN padding
    k = np.where(fin, hundred, wl.k_bits).astype(np.uint16)
    q = np.full_like(wl.q_bits, hundred)
    wz = dataclasses.replace(wl, k_bits=k, q_bits=q)
    zero = np.zeros(wl.D // 2)
    say(f"equal huge scores via {kind}")
    got = run_hip(wz, kind, inv_freq=zero)
    want = oracle_out(wz, base=zero)
    compare(got, want, f"equal-huge-scores/{kind}")


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_operand_range_large_keys(kind):
    """Keys scaled to |k| ~ 1e4 (N(0, 1) x 1e4, elements up to ~5e4, below fp16's 65504)
    with queries scaled by 1e-3, so scores stay moderate while the key operands sit near
    the top of the fp16 range."""
    import dataclasses
    from oracle.attention import bf16_bits_to_f64
    from workload import f32_to_bf16_bits
    wl = small(Hq=8, Hkv=2, D=128, seed=82, q_scale=1e-3)
    kf = bf16_bits_to_f64(wl.k_bits)
    fin = np.isfinite(kf)
    k = wl.k_bits.copy()
    k[fin] = f32_to_bf16_bits((kf[fin] * 1e4).astype(np.float32))
    wk = dataclasses.replace(wl, k_bits=k)
    say(f"large keys via {kind}: max |k| = {np.abs(kf[fin]).max() * 1e4:.3g}")
    compare(run_hip(wk, kind), oracle_out(wk), f"large-keys/{kind}")


@pytest.mark.gpu
def test_probes():
    """The ceiling probes run and read what they claim to: the read probe's XOR fold equals
    the buffer's, and the MFMA probe reports positive cycle spans."""
    import torch
    import position_agnostic_kv_paged_amd as L
    g = torch.Generator().manual_seed(31)
    host = torch.randint(-2**31, 2**31 - 1, (3 * 2**20 + 4,), generator=g, dtype=torch.int64)
    host = host.to(torch.int32)
    buf = host.cuda()
    got = L.probe_read(buf).cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert np.bitwise_xor.reduce(got) == want
    cyc, flops = L.probe_mfma(4)
    torch.cuda.synchronize()
    assert flops > 0 and int(cyc.min().item()) > 0
    # gather: the listed 1 KB chunks (one repeated, one id past the buffer, skipped)
    words = host.numpy().view(np.uint32)[: 3 * 2**20]
    chunks = words.reshape(-1, 256)                       # 1 KB each
    ids = np.array([5, 0, chunks.shape[0] - 1, 17, 5, chunks.shape[0], 1200], dtype=np.int32)
    got = L.probe_gather(buf[: 3 * 2**20], torch.from_numpy(ids).cuda(), 1024).cpu().numpy()
    want = np.uint32(0)
    for i in ids:
        if i < chunks.shape[0]:
            want ^= np.bitwise_xor.reduce(chunks[i])
    assert np.bitwise_xor.reduce(got.view(np.uint32)) == want


def _random_batch(seed):
    """A seeded random batch: 1-4 requests of random documents (repeats allowed, gaps, some
    back-to-back), a private tail (partial last block), random query counts including
    single-row and zero-row requests; random G in {1, 2, 4, 8, 16, 32} and D in {64, 128}."""
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    Hkv = int(rng.choice([1, 2])) if G <= 16 else 1
    n_docs, doc_tokens = 4, int(rng.choice([16, 32, 48]))
    reqs = []
    for _ in range(int(rng.integers(1, 5))):
        pos = int(rng.integers(0, 3000))
        segs = []
        for _ in range(int(rng.integers(0, 5))):
            segs.append(Segment("doc", pos, doc=int(rng.integers(0, n_docs))))
            pos += doc_tokens + int(rng.choice([0, 0, rng.integers(1, 40)]))
        tail = int(rng.integers(1, 60))
        segs.append(Segment("private", pos, tokens=tail))
        nq = int(rng.choice([0, 1, int(rng.integers(1, tail + 1)), tail]))
        reqs.append(RequestLayout(segs, nq))
    return build(f"random-{seed}", Hkv * G, Hkv, D, 16, 10000.0, n_docs, doc_tokens, reqs,
                 seed=seed, q_scale=float(rng.choice([1.0, 3.0])))


@pytest.mark.parametrize("seed", range(40))
def test_random_layouts_all_modes(seed):
    """Seeded random layouts through every positional-encoding entry point (RoPE, partial
    rotary, document-rotated pool, ALiBi) via the mixed prefill call and the decode call."""
    from oracle.alibi import alibi_slopes
    from tests.util import doc_stored_offsets
    wl = _random_batch(seed)
    G, D = wl.Hq // wl.Hkv, wl.D
    say(f"random layout {seed}: {wl.num_seqs} requests, G={G}, D={D}, rows={wl.total_q}")
    if wl.total_q == 0:
        return
    want = oracle_out(wl)
    r = 32 if D == 128 else 16
    want_p = oracle_out(wl, rotary_dim=r)
    st = doc_stored_offsets(wl)
    wd, want_d = _docrot_case(wl, st)
    slopes = alibi_slopes(wl.Hq)
    want_a = _alibi_ref(wl, slopes)
    qlen = np.diff(wl.q_indptr)
    kinds = ["prefill"] + (["decode"] if np.all(qlen <= 1) else [])
    for kind in kinds:
        compare(run_hip(wl, kind), want, f"random{seed}/rope/{kind}")
        compare(run_hip(wl, kind, rotary_dim=r), want_p, f"random{seed}/partial/{kind}")
        compare(run_hip(wd, kind, stored=st), want_d, f"random{seed}/doc/{kind}")
        compare(run_hip(wl, kind, slopes=slopes), want_a, f"random{seed}/alibi/{kind}")


@pytest.mark.parametrize("kind", ["prefill", "decode"])
@pytest.mark.parametrize("bound", [1, 3, 1000])
def test_max_entries_hint_is_only_a_hint(kind, bound):
    """max_entries below or far above the real block-table length changes the split-K work
    split and the workspace size, never the result (long rows get longer splits)."""
    segs_long = [Segment("doc", 7 + 32 * i, doc=i % 3) for i in range(40)] + \
        [Segment("private", 7 + 32 * 40, tokens=9)]
    reqs = [RequestLayout(segs_long, 9 if kind == "prefill" else 1),
            RequestLayout([Segment("doc", 0, doc=1), Segment("private", 32, tokens=3)], 1)]
    wl = build("hint", 8, 2, 128, 16, 10000.0, 3, 32, reqs, seed=71)
    say(f"max_entries = {bound} (real {max(len(x) for x in wl.seq_block_ids)}) via {kind}")
    compare(run_hip(wl, kind, max_entries=bound), oracle_out(wl), f"hint{bound}/{kind}")
