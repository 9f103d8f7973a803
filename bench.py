#!/usr/bin/env python3
"""Benchmark of the LazyAttention hot path on one MI355X.

Workload: the mixed continuous batch "mixed-64q8kv-4p96d" (64 q / 8 KV heads, head dim
128, bf16, block size 16, one 2000-document position-free pool): 4 prefill requests
(16 Zipf(1.1) documents x 1024 tokens + 512-token suffix prefilled causally) and 96 decode
requests (12 documents x 1024 tokens + 1 token). One step = ONE lazyattn_prefill call over
the whole batch (prefill tiles and decode items in one launch), on the current HIP stream,
bracketed by HIP events. Inputs are resident in HBM before timing.

Reported (one JSON line):
  value        attention TFLOP/s of the whole step (algorithmic: 4*D FLOP per visible
               (query, key, q-head) pair of every row, prefill and decode);
  mixed_step   the step against the sum of its halves run as separate calls, and against
               the overlapped roofline max(MFMA time, HBM time) of the whole batch;
  prefill      the prefill half alone (same kernel): TFLOP/s, fraction of the MFMA peak --
               the `roofline` object describes this launch;
  decode       the decode half alone (lazyattn_decode): GB/s of logical K+V bytes, of
               distinct blocks, counter-measured HBM bytes; cold-cache and no-reuse rates;
  decode_controls  the two decode configurations (C2, C4): warm, cold (1 GiB written
               before every repetition) and the no-reuse control of the same shape;
plus p10/median/p90 of every timing, the rotation ablation, the measured ceilings and the
float64 oracle timed on a bounded sample on the host cores.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (% MFMA peak) + decode attn HBM GB/s, Zipf RAG batch"
COPY_CALIBRATION_BYTES = 256 << 20   # plain device copy run once (counter calibration)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
WORKLOAD = "mixed-64q8kv-4p96d"
PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def visible_pairs(wl, seqs):
    """Sum over query rows of the number of keys at logical position <= the row's."""
    total = 0
    for s in seqs:
        T = len(wl.seq_offsets[s])
        kv = int(wl.kv_lens[s])
        pos = np.concatenate([wl.seq_offsets[s][t] + np.arange(16 if t < T - 1 else kv - 16 * t)
                              for t in range(T)])
        pos.sort()
        qp = wl.q_pos[wl.q_indptr[s]: wl.q_indptr[s + 1]]
        total += int(np.searchsorted(pos, qp, side="right").sum())
    return total


def prefill_flops(wl, seqs):
    return 4.0 * wl.D * wl.Hq * visible_pairs(wl, seqs)


def decode_bytes(wl, seqs):
    kv = sum(int(wl.kv_lens[s]) for s in seqs) * 2 * wl.Hkv * wl.D * 2
    rows = sum(int(wl.q_indptr[s + 1] - wl.q_indptr[s]) for s in seqs)
    entries = sum(len(wl.seq_offsets[s]) for s in seqs)
    return float(kv + 2 * rows * wl.Hq * wl.D * 2 + 4 * entries)


def kernel_source_hash(kernel):
    """Hash of the sources a kernel is built from (ties recorded counters to a kernel version)."""
    import hashlib
    csrc = os.path.join(ROOT, "position_agnostic_kv_paged_amd", "csrc")
    files = {"prefill": ["prefill_body.h", "mixed.hip", "decode_body.h", "decode_plan.h"],
             "decode": ["decode.hip", "decode_body.h"],
             "decode_shared": ["decode.hip", "decode_body.h", "decode_plan.h"]}[kernel]
    h = hashlib.sha256()
    for f in files + ["lazyattn_common.h", "lazyattn_kernels.h"]:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            # code only: comment-only lines and trailing // comments do not change a kernel
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def recorded_traffic(kernel):
    """HBM bytes per launch from the committed counter record, or None if the kernel changed."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def half_inputs(wl, seqs, dev, pool):
    """CSR arrays, queries and packed words of a subset of sequences (shares the pool)."""
    import torch
    import position_agnostic_kv_paged_amd as L
    ids = [wl.seq_block_ids[s] for s in seqs]
    offs = [wl.seq_offsets[s] for s in seqs]
    bt = np.concatenate([[0], np.cumsum([len(x) for x in ids])]).astype(np.int32)
    words = L.encode_meta(np.concatenate(ids), np.concatenate(offs), bt)
    rows = [np.arange(wl.q_indptr[s], wl.q_indptr[s + 1]) for s in seqs]
    qcnt = [len(r) for r in rows]
    rows = np.concatenate(rows)
    q = torch.from_numpy(wl.q_bits[rows].view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    return dict(q=q, k_pool=pool["k_pool"], v_pool=pool["v_pool"], block_table=i32(bt),
                block_meta=torch.from_numpy(words.view(np.int32)).to(dev),
                kv_lens=i32(wl.kv_lens[seqs]),
                q_indptr=i32(np.concatenate([[0], np.cumsum(qcnt)])),
                q_pos=i32(wl.q_pos[rows]), max_entries=max(len(x) for x in ids),
                out=torch.empty_like(q),
                host=dict(q_indptr=np.concatenate([[0], np.cumsum(qcnt)]).astype(np.int32),
                          block_table=bt, words=words))


def _counter_rows(run_dir):
    """Rows of the rocprofv3 --pmc csv output under run_dir."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"),
                              recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {run_dir}")
    return rows


def record_traffic(fetch_dir, write_dir):
    """Write profiles/traffic.json from one FETCH_SIZE and one WRITE_SIZE rocprofv3 run of
    this script: per-launch KiB of each attention kernel, scaled by what the same counter
    reads on the calibration copy of COPY_CALIBRATION_BYTES (the runtime copy kernel that
    writes exactly that size; both runs dispatch in the same order)."""
    fetch, write = _counter_rows(fetch_dir), _counter_rows(write_dir)

    def per_dispatch(rows, counter):
        out = {}
        for r in rows:
            if r["Counter_Name"] == counter:
                key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                out[key] = out.get(key, 0.0) + float(r["Counter_Value"])
        return out
    f, w = per_dispatch(fetch, "FETCH_SIZE"), per_dispatch(write, "WRITE_SIZE")
    target_kib = COPY_CALIBRATION_BYTES / 1024
    # the calibration copy is the runtime's device-to-device copy kernel writing exactly the
    # calibration size (other kernels of the run may write as much: fills, conversions)
    near = [k for k in w if "copyBuffer" in k[1] and abs(w[k] - target_kib) < 0.01 * target_kib
            and k in f]
    if len(near) != 1:
        raise SystemExit(f"calibration copy not found uniquely in the counter runs ({near})")
    cal = near[0]
    rec = {"_about": "HBM-side bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE "
                     "(KiB per dispatch), each scaled by the factor that maps the same counter "
                     "on a plain device copy of known size (run once inside bench.py) to that "
                     "size. Valid while the kernel sources hash to source_hash.",
           "workload": WORKLOAD,
           "calibration": {"copy_bytes": COPY_CALIBRATION_BYTES, "fetch_kib_on_copy": f[cal],
                           "write_kib_on_copy": w[cal],
                           "fetch_factor": target_kib / f[cal],
                           "write_factor": target_kib / w[cal]}}
    for kernel, tag, mode in (("prefill", "lazyattn::mixed_kernel<", ", 0>("),
                              ("decode", "lazyattn::decode_kernel<", ", 0>("),
                              ("decode_shared", "lazyattn::decode_plan_kernel<", ">(")):
        # the counter runs use --counters: prefill-half calls (mixed_kernel with prefill items
        # only), decode-half calls (decode_kernel) and the decode half over its plan
        # (decode_plan_kernel, RoPE only); the lazy (RoPE, mode 0) instantiation only, the
        # materialised baseline's is mode 1
        keys = [k for k in f if tag in k[1] and mode in k[1] and k in w]
        if not keys:
            continue
        top = max(f[k] for k in keys)
        keys = [k for k in keys if f[k] > 0.01 * top]
        fk, wk = [f[k] for k in keys], [w[k] for k in keys]
        fkib, wkib = float(np.mean(fk)), float(np.mean(wk))
        rec[kernel] = {"source_hash": kernel_source_hash(kernel), "dispatches": len(fk),
                       "fetch_kib": fkib, "write_kib": wkib,
                       "hbm_bytes_per_launch": 1024 * (fkib * rec["calibration"]["fetch_factor"]
                                                       + wkib * rec["calibration"]["write_factor"])}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def cpu_baseline(wl, pre_seqs, dec_seqs, budget_s=15.0):
    """The float64 oracle (as it stands) on a bounded sample of the same batch."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    cores = len(os.sched_getaffinity(0))
    k_bits, v_bits = wl.k_bits, wl.v_bits
    # prefill sample: the whole first prefill request (all its query rows, all 64 heads)
    s = pre_seqs[0]
    rows = np.arange(int(wl.q_indptr[s]), int(wl.q_indptr[s + 1]), dtype=np.int64)
    t0 = time.perf_counter()
    ids = [None] * wl.num_seqs
    ids[s] = wl.compact_ids(s)
    oracle.attention_rows(wl.q_bits, k_bits, v_bits, ids, wl.seq_offsets, wl.kv_lens,
                          wl.q_indptr, wl.q_pos, wl.rope_base, wl.B, s, rows)
    t_pre = time.perf_counter() - t0
    qp = wl.q_pos[rows]
    T = len(wl.seq_offsets[s])
    kv = int(wl.kv_lens[s])
    pos = np.sort(np.concatenate([wl.seq_offsets[s][t] + np.arange(16 if t < T - 1 else kv - 16 * t)
                                  for t in range(T)]))
    pre_flops = 4.0 * wl.D * wl.Hq * float(np.searchsorted(pos, qp, side="right").sum())
    # decode sample: whole decode requests until the time budget is used
    t0 = time.perf_counter()
    done, dbytes = 0, 0.0
    for s in dec_seqs:
        ids = [None] * wl.num_seqs
        ids[s] = wl.compact_ids(s)
        oracle.attention_rows(wl.q_bits, k_bits, v_bits, ids, wl.seq_offsets, wl.kv_lens,
                              wl.q_indptr, wl.q_pos, wl.rope_base, wl.B, s,
                              np.array([wl.q_indptr[s]]))
        done += 1
        dbytes += decode_bytes(wl, [s])
        if time.perf_counter() - t0 > budget_s:
            break
    t_dec = time.perf_counter() - t0
    return {"value": pre_flops / t_pre / 1e12, "unit": "TFLOP/s", "cores": cores,
            "blas_threads": blas, "kind": "oracle",
            "decode": {"value": dbytes / t_dec / 1e9, "unit": "GB/s"},
            "sample": f"prefill: one whole request ({len(rows)} query rows x {wl.Hq} heads "
                      f"against {kv} keys, {t_pre:.1f} s); decode: {done} whole decode requests "
                      f"({t_dec:.1f} s); float64 numpy, one sequence at a time"}


def unique_decode_bytes(wl, seqs):
    """K+V bytes of the distinct pool blocks the sequences reference (each read once) plus
    q, out and the words: what an ideal cache would fetch."""
    ids = np.unique(np.concatenate([wl.seq_block_ids[s] for s in seqs]))
    kv = len(ids) * wl.B * 2 * wl.Hkv * wl.D * 2
    rows = sum(int(wl.q_indptr[s + 1] - wl.q_indptr[s]) for s in seqs)
    entries = sum(len(wl.seq_offsets[s]) for s in seqs)
    return float(kv + 2 * rows * wl.Hq * wl.D * 2 + 4 * entries)


def pct(xs):
    xs = np.sort(np.asarray(xs))
    return {"p10": float(np.percentile(xs, 10)), "median": float(np.median(xs)),
            "p90": float(np.percentile(xs, 90))}


def measure_ingest(torch, L, wl, stream, reps, n_tokens=1 << 17):
    """lazyattn_ingest_kv writing n_tokens new (K, V) rows of this workload's head shape into
    distinct slots of a scratch pool, in a seeded random block order: bytes moved = read +
    write of K and V."""
    nb = n_tokens // wl.B
    pool_k = torch.empty((nb, wl.Hkv, wl.B, wl.D), dtype=torch.bfloat16, device="cuda")
    pool_v = torch.empty_like(pool_k)
    kn = torch.randn((n_tokens, wl.Hkv, wl.D), device="cuda").to(torch.bfloat16)
    vn = torch.randn_like(kn)
    g = torch.Generator(device="cpu").manual_seed(5)
    blocks = torch.randperm(nb, generator=g).to(torch.int32)
    slots = (blocks[:, None] * wl.B + torch.arange(wl.B, dtype=torch.int32)[None, :]).reshape(-1)
    slots = slots.cuda()
    for _ in range(3):
        L.ingest_kv(kn, vn, slots, pool_k, pool_v, stream=stream)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
    for k in range(reps):
        e[2 * k].record(stream)
        L.ingest_kv(kn, vn, slots, pool_k, pool_v, stream=stream)
        e[2 * k + 1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([e[2 * k].elapsed_time(e[2 * k + 1]) for k in range(reps)]))
    moved = 4.0 * n_tokens * wl.Hkv * wl.D * 2 + 4.0 * n_tokens
    del pool_k, pool_v, kn, vn
    return {"tokens": n_tokens, "ms": ms, "gbs": moved / (ms / 1e3) / 1e9,
            "frac_hbm_peak": moved / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
            "bytes": "read + write of K and V rows, plus the 4-byte slot of each token"}


def measured_ceilings(torch, L, stream, reps=5):
    """What the chip sustains here: the MFMA loop's TFLOP/s and shader clock (s_memtime
    cycles over event time), and a plain 2 GiB stream read's GB/s (medians over reps)."""
    iters = 2000
    cyc = torch.empty(L.probe_cus() * 8, dtype=torch.int64, device="cuda")
    buf = torch.empty(1 << 29, dtype=torch.int32, device="cuda").fill_(7)
    half = buf.numel() // 2
    chunk = 4096                                           # one (block, KV head) of K at D = 128
    n_chunks = buf.numel() * 4 // chunk
    order = torch.randperm(n_chunks, generator=torch.Generator().manual_seed(11))
    ids = order.to(torch.int32).to("cuda")
    mf, ghz, rd, cp, ga = [], [], [], [], []
    for r in range(reps + 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
        e[0].record(stream)
        _, flops = L.probe_mfma(iters, cycles=cyc, stream=stream)
        e[1].record(stream)
        e[2].record(stream)
        L.probe_read(buf, stream=stream)
        e[3].record(stream)
        e[6].record(stream)
        L.probe_gather(buf, ids, chunk, stream=stream)     # the same 2 GiB in random 4 KB chunks
        e[7].record(stream)
        e[4].record(stream)                                # (last: it leaves dirty lines behind)
        buf[half:].copy_(buf[:half])                       # plain device copy, 1 GiB each way
        e[5].record(stream)
        torch.cuda.synchronize()
        if r == 0:
            continue                                       # first launch: code load
        t = e[0].elapsed_time(e[1]) / 1e3
        mf.append(flops / t / 1e12)
        ghz.append(float(cyc.max().item()) / t / 1e9)
        rd.append(buf.numel() * 4 / (e[2].elapsed_time(e[3]) / 1e3) / 1e9)
        cp.append(2 * half * 4 / (e[4].elapsed_time(e[5]) / 1e3) / 1e9)
        ga.append(buf.numel() * 4 / (e[6].elapsed_time(e[7]) / 1e3) / 1e9)
    del buf, ids
    return {"mfma_f16_tflops": float(np.median(mf)), "shader_ghz": float(np.median(ghz)),
            "hbm_read_gbs": float(np.median(rd)), "hbm_copy_gbs": float(np.median(cp)),
            "hbm_gather_gbs": float(np.median(ga)),
            "note": "MFMA: 8 waves/CU of independent 32x32x16 fp16 products; read: 2 GiB, "
                    "16-byte non-temporal loads, 8 workgroups of 256 per CU; copy: torch "
                    "device-to-device copy of 1 GiB, read + write bytes; gather: the same "
                    "2 GiB as 4 KB chunks in a seeded random order, one wave per chunk, "
                    "ordinary 16-byte loads"}


SETTLE_S = 0.05


def settle(torch, fn, seconds=SETTLE_S):
    """Run fn back to back for `seconds` of wall time, untimed: the shader clock ramps up
    over the first milliseconds of sustained load (a short call after an idle gap runs
    slower than the same call under continuous load), so every timing starts from the
    clock that steady work sees."""
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def timed(torch, stream, fn, reps, warmup, flush=None):
    """Median-style timing of fn on `stream`: the clock settled (settle), warmup calls,
    then reps calls each bracketed by HIP events (a flush fill before each one, outside the
    events, when given)."""
    settle(torch, fn)
    for _ in range(warmup):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
    for k in range(reps):
        if flush is not None:
            flush.fill_(1.0)
        ev[2 * k].record(stream)
        fn()
        ev[2 * k + 1].record(stream)
    torch.cuda.synchronize()
    ts = [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(reps)]
    st = pct(ts)
    st["mean"] = float(np.mean(ts))
    return st


def attention_call(L, fn, wl, a, ws, stream):
    return lambda: fn(a["q"], a["k_pool"], a["v_pool"], a["block_table"], a["block_meta"],
                      a["kv_lens"], a["q_indptr"], a["q_pos"], wl.rope_base, a["max_entries"],
                      out=a["out"], workspace=ws, stream=stream)


def shared_call(torch, L, kind, wl, a, dev, stream, max_chunk=64):
    """The same call over a shared-document plan (lazyattn_{prefill,decode}_shared): the
    plan is built on the host from the batch's tables before any timing (its build time is
    reported, not part of the timed calls). Returns (call, plan facts)."""
    h = a["host"]
    t0 = time.perf_counter()
    plan = L.decode_share_plan(h["q_indptr"], h["block_table"], h["words"], wl.Hq, wl.Hkv,
                               single_row_only=kind == "prefill", max_chunk=max_chunk)
    plan_ms = (time.perf_counter() - t0) * 1e3
    n_items, n_slots = int(plan[4]), int(plan[5])
    total_q = int(h["q_indptr"][-1])
    recs = plan[8 + total_q + 1:].reshape(n_items, -1) if n_items else np.zeros((0, 2), np.int32)
    n_entries = int(h["block_table"][-1]) if kind == "decode" else sum(
        int(h["block_table"][s + 1] - h["block_table"][s])
        for s in range(len(h["q_indptr"]) - 1) if h["q_indptr"][s + 1] - h["q_indptr"][s] == 1)
    d_plan = torch.from_numpy(plan).to(dev)
    ws = torch.empty(max(16, L.shared_workspace_bytes(kind, a["kv_lens"].numel(), total_q,
                                                      a["max_entries"], n_slots, wl.Hq,
                                                      wl.Hkv, wl.D)),
                     dtype=torch.uint8, device=dev)
    fn = L.prefill_shared if kind == "prefill" else L.decode_shared
    call = lambda: fn(a["q"], a["k_pool"], a["v_pool"], a["block_table"], a["block_meta"],  # noqa
                      a["kv_lens"], a["q_indptr"], a["q_pos"], wl.rope_base, a["max_entries"],
                      d_plan, n_items, n_slots, out=a["out"], workspace=ws, stream=stream)
    facts = {"plan_host_ms": plan_ms, "items": n_items,
             "grouped_items": int((recs[:, 1] > 1).sum()) if n_items else 0,
             "decode_blocks_read_frac": float(recs[:, 0].sum() / max(n_entries, 1))
             if n_items else 0.0}
    return call, facts


def workspace_for(torch, L, kind, wl, a, dev):
    return torch.empty(L.workspace_bytes(kind, a["kv_lens"].numel(), a["q"].shape[0],
                                         a["max_entries"], wl.Hq, wl.Hkv, wl.D),
                       dtype=torch.uint8, device=dev)


def decode_control(torch, L, name, dev, stream, reps, warmup, flush):
    """Warm, cold and no-reuse rates of a decode configuration (lazyattn_decode)."""
    from workload import make
    out = {}
    for label, no_reuse in (("zipf", False), ("no_reuse", True)):
        wl = make(name, no_reuse=no_reuse)
        pool = wl.to_device(dev)
        seqs = list(range(wl.num_seqs))
        a = half_inputs(wl, seqs, dev, pool)
        ws = workspace_for(torch, L, "decode", wl, a, dev)
        f = attention_call(L, L.decode, wl, a, ws, stream)
        nbytes = decode_bytes(wl, seqs)
        runs = (("warm", None), ("cold", flush)) if not no_reuse else (("warm", None),)
        for mode, fl in runs:
            st = timed(torch, stream, f, reps, warmup, fl)
            key = label if label == "no_reuse" else mode
            out[key] = {"ms": st, "gbs": nbytes / (st["median"] / 1e3) / 1e9,
                        "frac_hbm_peak": nbytes / (st["median"] / 1e3) / 1e9 / PEAK_HBM_GBS}
        if not no_reuse:                                  # over a shared-document plan
            fs, facts = shared_call(torch, L, "decode", wl, a, dev, stream)
            st = timed(torch, stream, fs, reps, warmup)
            out["shared_plan"] = dict(facts, ms=st, gbs=nbytes / (st["median"] / 1e3) / 1e9,
                                      speedup=out["warm"]["ms"]["median"] / st["median"])
        del pool, a, ws
        torch.cuda.empty_cache()
    out["algorithmic_gb"] = nbytes / 1e9
    out["note"] = ("logical K+V bytes of every (sequence, key) plus q, out and words over the "
                   "median call time; cold: 1 GiB written before each repetition (L2 and MALL "
                   "flushed); no_reuse: every document appears once (no block read twice)")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first ~10 launches after the inputs are uploaded run up to 15% slower (the clock
    # ramps under load); the timed steps measure the steady state
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=50,
                    help="repetitions of every reference timing (halves, controls, ablation)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="configuration of the step (default: the mixed batch); the others are "
                         "the parity configurations, timed for reference")
    ap.add_argument("--no-reuse", action="store_true",
                    help="control of the same shape in which every document appears once")
    ap.add_argument("--cold", action="store_true",
                    help="overwrite a 1 GiB buffer before every step (flushes L2 and MALL; "
                         "outside the timed calls)")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the rotation ablation and the variants")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the shared-document plan timings")
    ap.add_argument("--no-controls", action="store_true",
                    help="skip the decode configurations' cold and no-reuse controls")
    ap.add_argument("--counters", action="store_true",
                    help="profiling pass for rocprofv3 --pmc: only prefill-half and decode-half "
                         "calls, a few of each, then exit")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs of this "
                         "script with --counters (FETCH_SIZE, then WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library runs the attention path on a "
              "single MI355X (no multi-GPU sharding); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import position_agnostic_kv_paged_amd as L
    from workload import make
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    L.lib()
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    wl = make(args.workload, no_reuse=args.no_reuse)
    qlen = np.diff(wl.q_indptr)
    all_seqs = list(range(wl.num_seqs))
    pre_seqs = [s for s in all_seqs if qlen[s] > 1]
    dec_seqs = [s for s in all_seqs if qlen[s] == 1]
    pool = wl.to_device(dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    # the step: one lazyattn_prefill call over the whole batch (any mix of query lengths);
    # a pure decode configuration runs lazyattn_decode
    step_fn = L.prefill if pre_seqs else L.decode
    step_kind = "prefill" if pre_seqs else "decode"
    a_all = half_inputs(wl, all_seqs, dev, pool)
    ws_all = workspace_for(torch, L, step_kind, wl, a_all, dev)
    step = attention_call(L, step_fn, wl, a_all, ws_all, stream)
    halves = {}
    for kind, seqs, fn in (("prefill", pre_seqs, L.prefill), ("decode", dec_seqs, L.decode)):
        if seqs:
            a = half_inputs(wl, seqs, dev, pool)
            ws = workspace_for(torch, L, kind, wl, a, dev)
            halves[kind] = (seqs, fn, a, ws, attention_call(L, fn, wl, a, ws, stream))

    # a plain copy of known size, once, so that FETCH_SIZE / WRITE_SIZE counter runs over
    # this program can be scaled to bytes (the factor is recorded with the counters)
    src = torch.empty(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    del src, dst
    torch.cuda.synchronize()
    if args.counters:
        for kind in ("prefill", "decode"):
            if kind in halves:
                for _ in range(5):
                    halves[kind][4]()
        done = sorted(halves)
        if "decode" in halves and not args.no_shared:
            # the decode half over its shared-document plan (decode_plan_kernel)
            sh, _ = shared_call(torch, L, "decode", wl, halves["decode"][2], dev, stream)
            for _ in range(5):
                sh()
            done.append("decode_shared")
        torch.cuda.synchronize()
        print(json.dumps({"counters_pass": done}), flush=True)
        return

    # ---- the timed step -------------------------------------------------------------------
    settle(torch, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    cold = flush if args.cold else None
    t0 = time.perf_counter()
    for k in range(args.steps):
        if cold is not None:
            cold.fill_(1.0)
        ev[2 * k].record(stream)
        step()
        ev[2 * k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ts = [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(args.steps)]
    step_ms = float(np.mean(ts))
    pre_flops = prefill_flops(wl, pre_seqs) if pre_seqs else 0.0
    dec_flops = 4.0 * wl.D * wl.Hq * sum(int(wl.kv_lens[s]) for s in dec_seqs)
    dbytes = decode_bytes(wl, dec_seqs) if dec_seqs else 0.0
    value = (pre_flops + dec_flops) / (step_ms / 1e3) / 1e12

    line = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": step_ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16, Zipf document reuse)"
                    + (", no-reuse control" if args.no_reuse else "")
                    + (", cold L2/MALL before every step" if args.cold else ""),
            "config": {"workload": wl.name, "Hq": wl.Hq, "Hkv": wl.Hkv, "head_dim": wl.D,
                       "operands": "bf16 in/out, fp16 rotated q/k and bf16 p/v on MFMA, fp32 "
                                   "accumulation",
                       "block": wl.B, "prefill_requests": len(pre_seqs),
                       "decode_requests": len(dec_seqs), "pool_blocks": wl.num_blocks,
                       "step": f"one {'lazyattn_prefill' if pre_seqs else 'lazyattn_decode'} "
                               f"call over the whole batch"},
            "step_ms_pct": pct(ts),
            "clock_settle_s": SETTLE_S,
            "value_definition": "algorithmic attention FLOPs of the whole step (prefill and "
                                "decode rows, 4*D per visible (query, key, q-head) pair) over "
                                "the mean step time"}

    # ---- the halves alone: per-kernel rooflines ----------------------------------------------
    roofs = []
    if "prefill" in halves:
        seqs, fn, a, ws, f = halves["prefill"]
        st = timed(torch, stream, f, args.reps, args.warmup)
        t = st["mean"] / 1e3
        val = pre_flops / t / 1e12
        line["prefill"] = {"value": val, "unit": "TFLOP/s", "ms": st["mean"], "ms_pct": st,
                           "frac_mfma_peak": val / PEAK_MFMA_TFLOPS,
                           "algorithmic_tflop": pre_flops / 1e12,
                           "call": "lazyattn_prefill over the prefill requests alone"}
        roofs.append((t, {"kernel": "mixed_kernel (prefill items)", "bound": "mfma",
                          "achieved": val, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                          "traffic_key": "prefill"}))
    if "decode" in halves:
        seqs, fn, a, ws, f = halves["decode"]
        st = timed(torch, stream, f, args.reps, args.warmup)
        stc = timed(torch, stream, f, args.reps, 3, flush)
        t = st["mean"] / 1e3
        ubytes = unique_decode_bytes(wl, seqs)
        val = dbytes / t / 1e9
        line["decode"] = {"value": val, "unit": "GB/s", "ms": st["mean"], "ms_pct": st,
                          "frac_hbm_peak": val / PEAK_HBM_GBS,
                          "algorithmic_gb": dbytes / 1e9,
                          "unique_gb": ubytes / 1e9, "unique_gbs": ubytes / t / 1e9,
                          "cold_ms_pct": stc,
                          "cold_gbs": dbytes / (stc["median"] / 1e3) / 1e9,
                          "call": "lazyattn_decode over the decode requests alone"}
        roofs.append((t, {"kernel": "decode_kernel", "bound": "hbm", "achieved": val,
                          "peak": PEAK_HBM_GBS, "unit": "GB/s", "traffic_key": "decode"}))
    if pre_seqs and dec_seqs:
        halves_ms = line["prefill"]["ms"] + line["decode"]["ms"]
        roof_us = max(pre_flops / (PEAK_MFMA_TFLOPS * 1e12), dbytes / (PEAK_HBM_GBS * 1e9)) * 1e6
        line["mixed_step"] = {"ms": step_ms, "sum_of_halves_ms": halves_ms,
                              "speedup_vs_halves": halves_ms / step_ms,
                              "overlapped_roofline_us": roof_us,
                              "frac_overlapped_roofline": roof_us / 1e3 / step_ms,
                              "serial_roofline_us": (pre_flops / (PEAK_MFMA_TFLOPS * 1e12)
                                                     + dbytes / (PEAK_HBM_GBS * 1e9)) * 1e6}
    # ---- the same step and decode half over a shared-document plan: the decode rows that
    # read the same runs of blocks share their loads (lazyattn_*_shared). The plan is built
    # on the host from the batch's tables before timing; its build time is reported ----
    if dec_seqs and not args.no_shared:
        fs, facts = shared_call(torch, L, step_kind, wl, a_all, dev, stream)
        st = timed(torch, stream, fs, args.reps, args.warmup)
        sh = dict(facts, call=f"{'lazyattn_prefill_shared' if pre_seqs else 'lazyattn_decode_shared'}"
                              " over the whole batch", ms=st["mean"], ms_pct=st,
                  value=(pre_flops + dec_flops) / (st["mean"] / 1e3) / 1e12,
                  speedup_vs_step=step_ms / st["mean"])
        if pre_seqs and "decode" in halves:
            seqs, fn, a, ws, f = halves["decode"]
            fd, fdf = shared_call(torch, L, "decode", wl, a, dev, stream)
            std = timed(torch, stream, fd, args.reps, args.warmup)
            sh["decode_half"] = dict(fdf, ms=std["mean"], ms_pct=std,
                                     gbs=dbytes / (std["mean"] / 1e3) / 1e9,
                                     speedup=line["decode"]["ms"] / std["mean"])
            # bytes beyond L2 per launch from the committed counter record (while valid)
            rec = (recorded_traffic("decode_shared")
                   if wl.name == WORKLOAD and not args.no_reuse else None)
            sh["decode_half"]["hbm_counter_gb"] = rec / 1e9 if rec else None
            sh["decode_half"]["hbm_counter_gbs"] = (rec / (std["mean"] / 1e3) / 1e9
                                                    if rec else None)
        sh["note"] = ("the plan groups up to 16/G decode rows that read the same run of "
                      "blocks into one item, so each block is loaded once for all of them; "
                      "value and gbs count the same algorithmic work as the plain call")
        line["shared_plan"] = sh
    if roofs:
        t_dom, roof = max(roofs, key=lambda r: r[0])
        roof["frac"] = roof["achieved"] / roof["peak"]
        key = roof.pop("traffic_key")
        rec = recorded_traffic(key) if wl.name == WORKLOAD and not args.no_reuse else None
        roof["traffic"] = rec
        roof["launch_ms"] = t_dom * 1e3
        line["roofline"] = roof
    if "decode" in line and wl.name == WORKLOAD and not args.no_reuse:
        rec = recorded_traffic("decode")
        line["decode"]["hbm_counter_gbs"] = (rec / (line["decode"]["ms"] / 1e3) / 1e9
                                             if rec else None)

    # ---- rotation ablation: the same calls with the key rotation compiled out (the
    # materialised baseline's kernels), timed on the same inputs -- only the time is used ----
    if not args.no_ablation:
        baseline = {"prefill": L.prefill_rotated_pool, "decode": L.decode_rotated_pool}
        abl, var_a, var_d = {}, {}, {}
        slopes = torch.tensor([2.0 ** (-8.0 * i / wl.Hq) for i in range(1, wl.Hq + 1)],
                              dtype=torch.float32, device=dev)
        st_all = wl.doc_stored_offsets()
        for kind, (seqs, fn, a, ws, f) in halves.items():
            t_lazy = line[kind]["ms_pct"]["median"]
            t_base = timed(torch, stream, attention_call(L, baseline[kind], wl, a, ws, stream),
                           args.reps, args.warmup)["median"]
            n_ent = int(a["block_table"][-1].item())
            dk = torch.empty((n_ent, wl.Hkv, wl.B, wl.D), dtype=torch.bfloat16, device=dev)
            dv = torch.empty_like(dk)
            dm = torch.empty(n_ent, dtype=torch.int32, device=dev)

            def mat():
                L.materialize_rotated(pool["k_pool"], pool["v_pool"], a["block_table"],
                                      a["block_meta"], a["kv_lens"], wl.rope_base, n_ent,
                                      dk, dv, dm, stream=stream)
            t_mat = timed(torch, stream, mat, args.reps, args.warmup)["median"]
            del dk, dv, dm
            abl[kind] = {"baseline_ms": t_base, "lazy_ms": t_lazy,
                         "rotation_overhead": t_lazy / t_base - 1.0,
                         "materialize_ms": t_mat,
                         "materialize_then_attend_ms": t_mat + t_base,
                         "lazy_speedup_vs_materialize": (t_mat + t_base) / t_lazy}

            def alibi():
                fn(a["q"], a["k_pool"], a["v_pool"], a["block_table"], a["block_meta"],
                   a["kv_lens"], a["q_indptr"], a["q_pos"], wl.rope_base, a["max_entries"],
                   out=a["out"], workspace=ws, stream=stream, slopes=slopes)
            var_a[kind] = {"ms": timed(torch, stream, alibi, args.reps, args.warmup)["median"],
                           "rope_ms": t_lazy}
            stv = torch.from_numpy(np.concatenate([st_all[x] for x in seqs]).astype(np.int32)).to(dev)

            def doc():
                fn(a["q"], a["k_pool"], a["v_pool"], a["block_table"], a["block_meta"],
                   a["kv_lens"], a["q_indptr"], a["q_pos"], wl.rope_base, a["max_entries"],
                   out=a["out"], workspace=ws, stream=stream, stored_offsets=stv)
            var_d[kind] = {"ms": timed(torch, stream, doc, args.reps, args.warmup)["median"],
                           "rope_ms": t_lazy}
        line["rotation_ablation"] = abl
        line["alibi"] = var_a
        # the document-rotated pool variant (only the time is used: the pool's keys are not
        # stored rotated here, the work is the same)
        line["doc_rotated_pool"] = var_d
    # ingest of new tokens' K/V into pool slots (separate scratch pool; not part of a step)
    line["ingest"] = measure_ingest(torch, L, wl, stream, args.steps)
    # the same kernels' rates against what the chip sustains on plain probes
    ceil = measured_ceilings(torch, L, stream)
    line["measured_ceilings"] = ceil
    if "prefill" in line:
        line["prefill"]["frac_measured_mfma"] = line["prefill"]["value"] / ceil["mfma_f16_tflops"]
    if "decode" in line:
        line["decode"]["frac_measured_read"] = line["decode"]["value"] / ceil["hbm_read_gbs"]
    line["ingest"]["frac_measured_copy"] = line["ingest"]["gbs"] / ceil["hbm_copy_gbs"]
    if not args.no_cpu_baseline and wl.name == WORKLOAD and pre_seqs and dec_seqs:
        line["cpu_baseline"] = cpu_baseline(wl, pre_seqs, dec_seqs)
    # the C5 decode half without reuse, and the decode configurations' controls
    if not args.no_controls and wl.name == WORKLOAD and not args.no_reuse:
        del pool, a_all, ws_all, halves
        torch.cuda.empty_cache()
        wn = make(WORKLOAD, no_reuse=True)
        pn = wn.to_device(dev)
        dn = [x for x in range(wn.num_seqs) if wn.q_indptr[x + 1] - wn.q_indptr[x] == 1]
        an = half_inputs(wn, dn, dev, pn)
        wsn = workspace_for(torch, L, "decode", wn, an, dev)
        stn = timed(torch, stream, attention_call(L, L.decode, wn, an, wsn, stream), args.reps,
                    args.warmup)
        line["decode"]["no_reuse_ms_pct"] = stn
        line["decode"]["no_reuse_gbs"] = decode_bytes(wn, dn) / (stn["median"] / 1e3) / 1e9
        line["decode"]["no_reuse_frac_measured_gather"] = (line["decode"]["no_reuse_gbs"]
                                                           / ceil["hbm_gather_gbs"])
        del pn, an, wsn
        torch.cuda.empty_cache()
        line["decode_controls"] = {
            name: decode_control(torch, L, name, dev, stream, args.reps, args.warmup, flush)
            for name in ("decode-32q8kv-b64-ctx4161", "decode-32q8kv-b8-ctx32769")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
