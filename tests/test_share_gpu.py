"""Shared-document decode (lazyattn_decode_shared over a lazyattn_decode_share_plan plan)
against the float64 oracle, every output element: full-size Zipf batches, the mini cases,
seeded random layouts, short chunks, rows of one sequence grouped together, and a plan that
does not match the call (zero rows, no fault)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from workload import make, Segment, RequestLayout, build  # noqa: E402
from tests.util import small, oracle_out  # noqa: E402
from tests.gpu_util import compare, say, words_for  # noqa: E402
from tests.test_parity_gpu import _mini_cases, _random_batch  # noqa: E402


def run_shared(wl, max_chunk=64, plan_edit=None, repeat=1, kind="decode"):
    """Plan on the host, copy the plan to the device, call lazyattn_{decode,prefill}_shared
    (a prefill call plans the rows of single-row sequences only)."""
    import torch
    import position_agnostic_kv_paged_amd as L
    t = wl.to_device("cuda")
    words = words_for(wl)
    plan = L.decode_share_plan(wl.q_indptr, wl.block_table, words, wl.Hq, wl.Hkv,
                               single_row_only=kind == "prefill", max_chunk=max_chunk)
    n_items, n_slots = int(plan[4]), int(plan[5])
    if plan_edit is not None:
        plan = plan_edit(plan.copy())
    d_plan = torch.from_numpy(plan).cuda()
    meta = torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).cuda()
    max_entries = max(len(x) for x in wl.seq_block_ids)
    outs = []
    for _ in range(repeat):
        fn = L.prefill_shared if kind == "prefill" else L.decode_shared
        out = fn(t["q"], t["k_pool"], t["v_pool"], t["block_table"], meta,
                              t["kv_lens"], t["q_indptr"], t["q_pos"], wl.rope_base,
                              max_entries, d_plan, n_items, n_slots)
        torch.cuda.synchronize()
        outs.append(out.float().cpu().numpy().astype(np.float64))
    grouped = int(np.sum(plan[8 + wl.total_q + 1:].reshape(n_items, -1)[:, 1] > 1)) \
        if plan_edit is None and n_items else 0
    return (outs[0] if repeat == 1 else outs), grouped


@pytest.mark.timeout(300)
@pytest.mark.parametrize("q_scale", [1.0, 4.0])
@pytest.mark.parametrize("name", ["decode-32q8kv-b64-ctx4161", "decode-32q8kv-b8-ctx32769"])
def test_shared_full_size(name, q_scale):
    wl = make(name, q_scale=q_scale)
    got, grouped = run_shared(wl)
    say(f"{wl.name} shared decode: {grouped} grouped items, every row")
    compare(got, oracle_out(wl), f"{wl.name}/shared")


@pytest.mark.timeout(300)
def test_shared_mixed_batch_decode_rows():
    """The 96 decode requests of the mixed batch (64 query heads, G = 8: two rows per item)."""
    wl = make("mixed-64q8kv-4p96d")
    qlen = np.diff(wl.q_indptr)
    keep = [s for s in range(wl.num_seqs) if qlen[s] == 1]
    wd = build("mixed-decode-half", wl.Hq, wl.Hkv, wl.D, wl.B, wl.rope_base,
               wl.info.get("n_docs", 2000), wl.info.get("doc_tokens", 1024),
               [wl.layouts[s] for s in keep], seed=1004) if wl.layouts else None
    if wd is None:
        pytest.skip("workload has no layouts")
    got, grouped = run_shared(wd, max_chunk=96)
    say(f"mixed decode half shared decode: {grouped} grouped items, every row")
    assert grouped > 0
    compare(got, oracle_out(wd), "mixed-decode/shared")


@pytest.mark.parametrize("name,kw", _mini_cases(), ids=[c[0] for c in _mini_cases()])
def test_shared_mini_cases(name, kw):
    wl = small(**kw)
    got, _ = run_shared(wl, max_chunk=4)
    compare(got, oracle_out(wl), f"{name}/shared")


@pytest.mark.parametrize("seed", range(40))
def test_shared_random_layouts(seed):
    wl = _random_batch(seed)
    if wl.total_q == 0:
        return
    got, grouped = run_shared(wl, max_chunk=int(np.random.default_rng(seed).choice([4, 8, 64])))
    say(f"random {seed}: G={wl.Hq // wl.Hkv}, {grouped} grouped items")
    compare(got, oracle_out(wl), f"random{seed}/shared")


def test_shared_rows_of_one_sequence_and_repeats():
    """Six query rows of one sequence (every block shared, G = 4: four rows per item), a
    document repeated inside a request, a request without entries."""
    segs = [Segment("doc", 3, doc=1), Segment("doc", 20, doc=0), Segment("doc", 100, doc=1),
            Segment("private", 140, tokens=21)]
    reqs = [RequestLayout(segs, 6), RequestLayout([], 1, np.array([9])),
            RequestLayout([Segment("doc", 500, doc=1), Segment("private", 600, tokens=3)], 1)]
    wl = build("rows-repeats", 8, 2, 128, 16, 10000.0, 2, 64, reqs, seed=7, q_scale=4.0)
    got, grouped = run_shared(wl, max_chunk=4)
    assert grouped > 0
    compare(got, oracle_out(wl), "rows-repeats/shared")
    r0, r1 = int(wl.q_indptr[1]), int(wl.q_indptr[2])
    assert np.array_equal(got[r0:r1], np.zeros_like(got[r0:r1]))


def test_shared_run_to_run_bitwise():
    wl = make("decode-32q8kv-b64-ctx4161")
    a, b = run_shared(wl, repeat=2)[0]
    assert np.array_equal(a, b)


@pytest.mark.parametrize("edit", ["magic", "version", "members"])
def test_shared_mismatched_plan_gives_zero_rows(edit):
    """A plan whose header does not match the call is not followed: every row is zero. A plan
    of the earlier layout (version 1, items not cut where a member's offset delta changes)
    is refused the same way."""
    wl = small(Hq=8, Hkv=2, D=128, seed=9)

    def spoil(p):
        if edit == "magic":
            p[0] ^= 1
        elif edit == "version":
            p[1] = 1
        else:
            p[2] += 1
        return p
    got, _ = run_shared(wl, plan_edit=spoil)
    assert np.all(got == 0.0)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("q_scale", [1.0, 4.0])
def test_shared_prefill_call_mixed_batch(q_scale):
    """The whole mixed batch in one lazyattn_prefill_shared call (prefill tiles plus the
    decode rows over the plan), every row."""
    wl = make("mixed-64q8kv-4p96d", q_scale=q_scale)
    got, grouped = run_shared(wl, max_chunk=64, kind="prefill")
    say(f"{wl.name} prefill_shared: {grouped} grouped decode items, every row")
    assert grouped > 0
    compare(got, oracle_out(wl), f"{wl.name}/prefill-shared")


@pytest.mark.parametrize("seed", range(40))
def test_shared_prefill_call_random_layouts(seed):
    wl = _random_batch(seed)
    if wl.total_q == 0:
        return
    got, _ = run_shared(wl, max_chunk=int(np.random.default_rng(seed).choice([4, 8, 64])),
                        kind="prefill")
    compare(got, oracle_out(wl), f"random{seed}/prefill-shared")


def test_shared_prefill_call_small_mixed_and_empty():
    """Prefill, decode and empty requests in one call; two decode rows share a document."""
    d = [Segment("doc", 11, doc=0), Segment("doc", 60, doc=1), Segment("private", 120, tokens=9)]
    reqs = [RequestLayout(d, 9), RequestLayout(d, 1), RequestLayout([], 0),
            RequestLayout([Segment("doc", 300, doc=1), Segment("doc", 364, doc=0),
                           Segment("private", 430, tokens=2)], 1),
            RequestLayout([], 1, np.array([5]))]
    wl = build("small-mixed-shared", 16, 2, 128, 16, 10000.0, 2, 64, reqs, seed=13,
               q_scale=3.0)
    got, grouped = run_shared(wl, max_chunk=4, kind="prefill")
    assert grouped > 0
    compare(got, oracle_out(wl), "small-mixed/prefill-shared")


def test_shared_prefill_call_mismatched_plan():
    """lazyattn_prefill_shared with a plan of another version: the decode rows (single-row
    sequences) are zero, the prefill rows are still computed as by lazyattn_prefill."""
    d = [Segment("doc", 11, doc=0), Segment("doc", 60, doc=1), Segment("private", 120, tokens=9)]
    reqs = [RequestLayout(d, 9), RequestLayout(d, 1),
            RequestLayout([Segment("doc", 300, doc=1), Segment("private", 364, tokens=20)], 20),
            RequestLayout([Segment("doc", 300, doc=1), Segment("doc", 364, doc=0),
                           Segment("private", 430, tokens=2)], 1)]
    wl = build("small-mixed-spoiled", 16, 2, 128, 16, 10000.0, 2, 64, reqs, seed=17)

    def spoil(p):
        p[1] = 1
        return p
    got, _ = run_shared(wl, max_chunk=4, kind="prefill", plan_edit=spoil)
    qlen = np.diff(wl.q_indptr)
    dec = [int(wl.q_indptr[s]) for s in range(wl.num_seqs) if qlen[s] == 1]
    pre = [r for s in range(wl.num_seqs) if qlen[s] > 1
           for r in range(int(wl.q_indptr[s]), int(wl.q_indptr[s + 1]))]
    assert len(dec) == 2 and len(pre) == 29
    assert np.all(got[dec] == 0.0)
    compare(got[pre], oracle_out(wl)[pre], "small-mixed/prefill-shared, spoiled plan")
