"""bench.py on the CPU: the algorithmic counts behind `value` and `roofline.achieved`,
checked by brute force on small layouts, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from tests.util import small
from workload import Segment, make

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _brute_visible_pairs(wl, seqs):
    """Count (query row, key) pairs with key position <= row position, one pair at a time."""
    n = 0
    for s in seqs:
        T = len(wl.seq_offsets[s])
        kv = int(wl.kv_lens[s])
        keys = []
        for t in range(T):
            n_t = wl.B if t < T - 1 else kv - wl.B * (T - 1)
            keys += [int(wl.seq_offsets[s][t]) + j for j in range(n_t)]
        for r in range(int(wl.q_indptr[s]), int(wl.q_indptr[s + 1])):
            n += sum(1 for L in keys if L <= int(wl.q_pos[r]))
    return n


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_visible_pairs_equals_brute_force(seed):
    # overlapping documents, a gap, a repeated document and a partial tail
    segs = [Segment("doc", 3, doc=1), Segment("doc", 20, doc=0), Segment("doc", 100, doc=1),
            Segment("private", 140, tokens=21)]
    wl = small(segs=segs, q_len=21, seed=seed)
    seqs = list(range(wl.num_seqs))
    assert bench.visible_pairs(wl, seqs) == _brute_visible_pairs(wl, seqs)
    assert bench.prefill_flops(wl, seqs) == 4.0 * wl.D * wl.Hq * _brute_visible_pairs(wl, seqs)


def test_counts_of_the_mixed_batch():
    """The figures the bench line quotes for the mixed batch: 1.1167 TFLOP over the prefill
    rows and 4.8357 GB of logical decode bytes (K + V of every key of every decode row,
    plus q, out and one word per entry)."""
    wl = make("mixed-64q8kv-4p96d")
    qlen = np.diff(wl.q_indptr)
    pre = [s for s in range(wl.num_seqs) if qlen[s] > 1]
    dec = [s for s in range(wl.num_seqs) if qlen[s] == 1]
    assert (len(pre), len(dec)) == (4, 96)
    assert abs(bench.prefill_flops(wl, pre) / 1e12 - 1.1167) < 1e-4
    kv = sum(int(wl.kv_lens[s]) for s in dec) * wl.Hkv * wl.D * 2 * 2
    extra = len(dec) * wl.Hq * wl.D * 2 * 2 + 4 * sum(len(wl.seq_offsets[s]) for s in dec)
    assert bench.decode_bytes(wl, dec) == kv + extra
    assert abs(bench.decode_bytes(wl, dec) / 1e9 - 4.8357) < 1e-4
    # distinct blocks: never more than the logical bytes; Zipf reuse makes them fewer
    assert bench.unique_decode_bytes(wl, dec) < 0.5 * bench.decode_bytes(wl, dec)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "single MI355X" in r.stderr and r.stdout.strip() == ""
