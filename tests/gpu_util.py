"""Helpers for GPU parity tests: run the HIP path on a workload (no attention arithmetic)."""
import sys

import numpy as np

MAX_ABS = 2e-2    # bf16 outputs vs float64 oracle: max |diff|
MEAN_ABS = 2e-3   # mean |diff|


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def words_for(wl):
    import position_agnostic_kv_paged_amd as L
    return L.encode_meta(wl.flat_block_ids, wl.flat_offsets, wl.block_table)


def run_hip(wl, kind, dev="cuda", tensors=None, words=None, repeat=1, inv_freq=None,
            slopes=None, rotary_dim=None, stored=None, max_entries=None):
    """Call lazyattn_prefill / lazyattn_decode on the workload; returns float64 [total_q,Hq,D]."""
    import torch
    import position_agnostic_kv_paged_amd as L
    t = tensors if tensors is not None else wl.to_device(dev)
    if words is None:
        words = words_for(wl)
    meta = torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(dev)
    if max_entries is None:
        max_entries = max(len(x) for x in wl.seq_block_ids)
    fn = L.prefill if kind == "prefill" else L.decode
    st = None if stored is None else \
        torch.from_numpy(np.concatenate(stored).astype(np.int32)).to(dev)
    outs = []
    for _ in range(repeat):
        out = fn(t["q"], t["k_pool"], t["v_pool"], t["block_table"], meta, t["kv_lens"],
                 t["q_indptr"], t["q_pos"], wl.rope_base, max_entries, inv_freq=inv_freq,
                 slopes=None if slopes is None else
                 torch.as_tensor(np.asarray(slopes, np.float32), device=dev),
                 rotary_dim=rotary_dim, stored_offsets=st)
        torch.cuda.synchronize()
        outs.append(out.float().cpu().numpy().astype(np.float64))
    return outs[0] if repeat == 1 else outs


def compare(got, want, label):
    d = np.abs(got - want)
    mx, mean = float(d.max()), float(d.mean())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    say(f"  {label}: max_abs={mx:.3e} mean_abs={mean:.3e} rel={rel:.3e}")
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{label}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean, rel
