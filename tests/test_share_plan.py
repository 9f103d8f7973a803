"""Host planner of shared-document decode (lazyattn_decode_share_plan), on the CPU: the plan
covers every (row, entry) of the planned rows exactly once, grouped members read the same
block ids, every member's logical offsets advance by one block per entry inside an item,
slots are consecutive per row, and the header describes the plan."""
import numpy as np
import pytest

from workload import make, Segment, RequestLayout, build
from tests.gpu_util import words_for


def _lib():
    import position_agnostic_kv_paged_amd as L
    L.lib()
    return L


def _parse(plan, total_q):
    M, rec = int(plan[2]), int(plan[3])
    n_items, n_slots = int(plan[4]), int(plan[5])
    prefix = plan[8: 8 + total_q + 1]
    recs = plan[8 + total_q + 1:].reshape(n_items, rec)
    return M, n_items, n_slots, prefix, recs


def _check(wl, single_row_only, max_chunk, waves=2048):
    L = _lib()
    words = words_for(wl)
    G = wl.Hq // wl.Hkv
    plan = L.decode_share_plan(wl.q_indptr, wl.block_table, words, wl.Hq, wl.Hkv,
                               single_row_only=single_row_only, max_chunk=max_chunk,
                               waves=waves)
    assert plan[0] == 0x5053414C and plan[1] == 2
    assert plan[6] == wl.total_q and plan[7] == wl.num_seqs
    M, n_items, n_slots, prefix, recs = _parse(plan, wl.total_q)
    assert M == (16 // G if G <= 16 else 1) and plan[3] == 2 + 4 * M
    assert len(plan) == 8 + wl.total_q + 1 + n_items * (2 + 4 * M)
    assert prefix[0] == 0 and prefix[-1] == n_slots and np.all(np.diff(prefix) >= 0)
    qlen = np.diff(wl.q_indptr)
    planned = [r for s in range(wl.num_seqs)
               for r in range(wl.q_indptr[s], wl.q_indptr[s + 1])
               if not single_row_only or qlen[s] == 1]
    seq_of = np.repeat(np.arange(wl.num_seqs), qlen)
    covered = {r: np.zeros(len(wl.seq_block_ids[seq_of[r]]), dtype=np.int64) for r in planned}
    slots_seen = {r: [] for r in planned}
    grouped = 0
    for it in recs:
        ln, nm = int(it[0]), int(it[1])
        if nm == 0:                              # balancing filler
            assert ln == 0
            continue
        assert 1 <= nm <= M and ln >= 1 and ln <= min(max_chunk, 128 // M)
        lead = None
        for k in range(nm):
            row, seq, eb, slot = (int(x) for x in it[2 + 4 * k: 6 + 4 * k])
            assert row in covered and seq_of[row] == seq
            ids = wl.seq_block_ids[seq][eb: eb + ln]
            assert len(ids) == ln
            lead = ids if lead is None else lead
            assert np.array_equal(ids, lead), "members read the same blocks"
            offs = np.asarray(wl.seq_offsets[seq][eb: eb + ln], dtype=np.int64)
            assert np.all(np.diff(offs) == wl.B), "offsets contiguous inside an item"
            covered[row][eb: eb + ln] += 1
            slots_seen[row].append(slot)
        assert len({int(x) for x in it[2: 2 + 4 * nm: 4]}) == nm, "distinct member rows"
        grouped += nm > 1
    for r in planned:
        assert np.all(covered[r] == 1), f"row {r}: every entry exactly once"
        assert sorted(slots_seen[r]) == list(range(prefix[r], prefix[r + 1]))
    for r in range(wl.total_q):
        if r not in covered:
            assert prefix[r + 1] == prefix[r]
    return grouped, n_items


@pytest.mark.parametrize("name", ["decode-32q8kv-b64-ctx4161", "decode-32q8kv-b8-ctx32769",
                                  "tiny-prefill-4q1kv-d64"])
@pytest.mark.parametrize("max_chunk,waves", [(4, 2048), (64, 0), (16, 64)])
def test_plan_covers_every_entry_once(name, max_chunk, waves):
    wl = make(name)
    grouped, _ = _check(wl, False, max_chunk, waves)
    if name == "decode-32q8kv-b64-ctx4161":
        assert grouped > 0                       # Zipf-shared documents are grouped


def test_plan_mixed_batch_single_row_only():
    """The decode rows of the mixed batch only (prefill rows get no slots)."""
    wl = make("mixed-64q8kv-4p96d")
    grouped, _ = _check(wl, True, 96)
    assert grouped > 0


def test_plan_rows_of_one_sequence_group_together():
    """Several query rows of one sequence read the same table: they share every block."""
    segs = [Segment("doc", 0, doc=0), Segment("doc", 64, doc=1),
            Segment("private", 128, tokens=20)]
    wl = build("multirow", 8, 2, 64, 16, 10000.0, 2, 64, [RequestLayout(segs, 6)], seed=5)
    grouped, n_items = _check(wl, False, 64, waves=0)
    assert grouped == n_items                    # 6 rows, G = 4: groups of up to 4 rows


def test_plan_repeats_and_empty_sequences():
    segs = [Segment("doc", 3, doc=1), Segment("doc", 20, doc=0), Segment("doc", 100, doc=1),
            Segment("private", 140, tokens=21)]
    reqs = [RequestLayout(segs, 1), RequestLayout([], 1, np.array([9])),
            RequestLayout([Segment("doc", 500, doc=1), Segment("private", 600, tokens=3)], 1),
            RequestLayout(segs, 0)]
    wl = build("repeats", 16, 2, 128, 16, 10000.0, 2, 64, reqs, seed=6)
    _check(wl, False, 4)
    _check(wl, True, 8)


def test_plan_errors():
    L = _lib()
    from position_agnostic_kv_paged_amd._lib import LazyAttnError
    wl = make("tiny-prefill-4q1kv-d64")
    words = words_for(wl)
    with pytest.raises(LazyAttnError):
        L.decode_share_plan(wl.q_indptr, wl.block_table, words, wl.Hq, wl.Hkv, max_chunk=3)
    bad = np.array(wl.q_indptr).copy()
    bad[0] = 1                                   # CSR must start at 0
    with pytest.raises(LazyAttnError):
        L.decode_share_plan(bad, wl.block_table, words, wl.Hq, wl.Hkv)


def test_plan_keeps_runs_of_one_document_on_one_xcd_class():
    """Items that read the same run of blocks go to lanes of one class (lane mod 8, the XCD
    both decode launches run that lane's items on), and the plan still covers every entry."""
    L = _lib()
    doc = [Segment("doc", 0, doc=0), Segment("private", 4096, tokens=40)]
    reqs = [RequestLayout(doc, 1) for _ in range(20)]
    wl = build("same-doc", 16, 2, 64, 16, 10000.0, 1, 4096, reqs, seed=3)
    _check(wl, False, 12, waves=2048)
    words = words_for(wl)
    # 12-block runs: a row pair's 22 items would put the next pair's copies 22 lanes on
    plan = L.decode_share_plan(wl.q_indptr, wl.block_table, words, wl.Hq, wl.Hkv,
                               max_chunk=12, waves=2048)
    M, n_items, _, _, recs = _parse(plan, wl.total_q)
    lanes = 2048 // wl.Hkv
    ids = (np.asarray(words).view(np.uint32) & ((1 << 17) - 1)).astype(np.int64)
    bt = np.asarray(wl.block_table)
    by_run = {}
    for pos, it in enumerate(recs):
        ln, nm = int(it[0]), int(it[1])
        if nm == 0:
            continue
        seq, eb = int(it[3]), int(it[4])
        run = tuple(ids[bt[seq] + eb: bt[seq] + eb + ln])
        by_run.setdefault(run, []).append((pos % lanes) % 8)
    shared = {r: c for r, c in by_run.items() if len(c) > 1}
    assert shared, "the 20 rows of one document give repeated runs"
    for run, classes in shared.items():
        assert len(set(classes)) == 1, f"run of {len(run)} blocks spread over classes {classes}"
