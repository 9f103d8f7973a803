"""Thin torch-facing wrappers over the C ABI (include/lazyattn.h).

Only argument marshalling happens here: device pointers from torch tensors, the current
HIP stream, workspace allocation through torch. Every step of the attention path runs in
the HIP kernels of liblazyattn.so.
"""
import ctypes

import numpy as np

from ._lib import lib, check, PoolStats, ERR_NOSPACE

BLOCK = 16


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dims(q, k_pool):
    total_q, Hq, D = q.shape
    num_blocks, Hkv, B, D2 = k_pool.shape
    if D2 != D:
        raise ValueError("q and k_pool head dims differ")
    return total_q, Hq, D, num_blocks, Hkv, B


def workspace_bytes(kind, num_seqs, total_q, max_entries, Hq, Hkv, D):
    f = lib().lazyattn_prefill_workspace_bytes if kind == "prefill" else \
        lib().lazyattn_decode_workspace_bytes
    return int(f(num_seqs, total_q, max_entries, Hq, Hkv, D))


def _attention(kind, q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_pos,
               rope_base, max_entries, out=None, workspace=None, stream=None,
               rotated_pool=False, inv_freq=None, slopes=None, rotary_dim=None,
               stored_offsets=None):
    import torch
    total_q, Hq, D, num_blocks, Hkv, B = _dims(q, k_pool)
    num_seqs = kv_lens.numel()
    if out is None:
        out = torch.empty_like(q)
    need = workspace_bytes(kind, num_seqs, total_q, max_entries, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    extra, pre = [], []
    if stored_offsets is not None:
        if rotated_pool or inv_freq is not None or slopes is not None or rotary_dim is not None:
            raise ValueError("stored_offsets combines with rope_base only")
        if stored_offsets.dtype != torch.int32 or not stored_offsets.is_contiguous() or \
                stored_offsets.numel() != block_meta.numel():
            raise ValueError("stored_offsets must be a contiguous int32 device tensor with one "
                             "entry per block-table entry")
        name, pe, pre = "lazyattn_" + kind + "_doc_rotated", float(rope_base), [_ptr(stored_offsets)]
    elif rotary_dim is not None and rotary_dim != D:
        if rotated_pool or inv_freq is not None or slopes is not None:
            raise ValueError("rotary_dim combines with rope_base only")
        name, pe = "lazyattn_" + kind + "_partial", float(rope_base)
        extra = [int(rotary_dim)]
    elif slopes is not None:
        if rotated_pool or inv_freq is not None:
            raise ValueError("ALiBi slopes exclude RoPE options")
        if slopes.dtype != torch.float32 or slopes.numel() != Hq or not slopes.is_contiguous():
            raise ValueError(f"slopes must be a contiguous float32 device tensor of Hq = {Hq}")
        name, pe = "lazyattn_" + kind + "_alibi", _ptr(slopes)
    elif inv_freq is not None:
        if rotated_pool:
            raise ValueError("a frequency table applies to the position-free pool only")
        fr = np.ascontiguousarray(inv_freq, dtype=np.float64)
        if fr.shape != (D // 2,):
            raise ValueError(f"inv_freq must hold D/2 = {D // 2} frequencies")
        name, pe = "lazyattn_" + kind + "_freqs", ctypes.c_void_p(fr.ctypes.data)
    else:
        name = "lazyattn_" + kind + ("_rotated_pool" if rotated_pool else "")
        pe = float(rope_base)
    fn = getattr(lib(), name)
    rc = fn(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(block_meta),
            _ptr(kv_lens), _ptr(q_indptr), _ptr(q_pos), *pre, pe, *extra, num_seqs, total_q,
            Hq, Hkv, D, B, num_blocks, int(max_entries), _ptr(out), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    check(rc, name)
    return out


def prefill(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_pos, rope_base,
            max_entries, out=None, workspace=None, stream=None, inv_freq=None, slopes=None,
            rotary_dim=None, stored_offsets=None):
    """lazyattn_prefill on torch tensors (all on one HIP device); returns out. With inv_freq
    (D/2 radians per position), lazyattn_prefill_freqs; with slopes (float32 device [Hq]),
    lazyattn_prefill_alibi; rope_base is then not used. With rotary_dim below D (a multiple
    of 16), lazyattn_prefill_partial (partial rotary). With stored_offsets (int32 device,
    one per block-table entry), lazyattn_prefill_doc_rotated (keys stored with RoPE at
    those offsets)."""
    return _attention("prefill", q, k_pool, v_pool, block_table, block_meta, kv_lens,
                      q_indptr, q_pos, rope_base, max_entries, out, workspace, stream,
                      inv_freq=inv_freq, slopes=slopes, rotary_dim=rotary_dim,
                      stored_offsets=stored_offsets)


def decode(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_pos, rope_base,
           max_entries, out=None, workspace=None, stream=None, inv_freq=None, slopes=None,
           rotary_dim=None, stored_offsets=None):
    """lazyattn_decode on torch tensors; returns out (inv_freq, slopes, rotary_dim,
    stored_offsets as for prefill)."""
    return _attention("decode", q, k_pool, v_pool, block_table, block_meta, kv_lens,
                      q_indptr, q_pos, rope_base, max_entries, out, workspace, stream,
                      inv_freq=inv_freq, slopes=slopes, rotary_dim=rotary_dim,
                      stored_offsets=stored_offsets)


def decode_noalloc(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_pos,
                   rope_base, max_entries, out, stream=None):
    """lazyattn_decode_noalloc: lazyattn_decode with the library's fixed per-device buffer in
    place of a workspace (nothing is allocated; `out` must be given). Calls that overlap on
    one device race."""
    total_q, Hq, D, num_blocks, Hkv, B = _dims(q, k_pool)
    rc = lib().lazyattn_decode_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(block_meta),
        _ptr(kv_lens), _ptr(q_indptr), _ptr(q_pos), float(rope_base), kv_lens.numel(), total_q,
        Hq, Hkv, D, B, num_blocks, int(max_entries), _ptr(out), _stream(stream))
    check(rc, "lazyattn_decode_noalloc")
    return out


def decode_share_plan(q_indptr, block_table, block_meta, Hq, Hkv, single_row_only=False,
                      max_chunk=16, waves=None):
    """lazyattn_decode_share_plan on host (numpy) tables: returns the int32 plan (numpy); its
    header holds the item count [4] and slot count [5]. waves defaults to the resident
    decode waves of the device (8 per compute unit)."""
    if waves is None:
        waves = 8 * probe_cus()
    qi = np.ascontiguousarray(q_indptr, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    bm = np.ascontiguousarray(block_meta, dtype=np.uint32)
    n = ctypes.c_int64(0)
    args = (qi.ctypes.data, bt.ctypes.data, bm.ctypes.data if bm.size else None, len(qi) - 1,
            int(qi[-1]), int(Hq), int(Hkv), int(bool(single_row_only)), int(max_chunk),
            int(waves))
    # one planner call with a generous guess of the length; a second only if it was short
    G = Hq // Hkv
    rec = 2 + 4 * (16 // G if G <= 16 else 1)
    lanes = max(1, int(waves) // max(1, Hkv if G <= 16 else Hq // 16))
    guess = 8 + len(qi) + rec * (int(bt[-1]) // 4 + int(qi[-1]) + 2 * lanes + 64)
    plan = np.zeros(guess, dtype=np.int32)
    rc = lib().lazyattn_decode_share_plan(*args, plan.ctypes.data, guess, ctypes.byref(n))
    if rc == ERR_NOSPACE:
        plan = np.zeros(n.value, dtype=np.int32)
        rc = lib().lazyattn_decode_share_plan(*args, plan.ctypes.data, n.value,
                                              ctypes.byref(n))
    check(rc, "lazyattn_decode_share_plan")
    return plan[: n.value]


def shared_workspace_bytes(kind, num_seqs, total_q, max_entries, plan_slots, Hq, Hkv, D):
    """lazyattn_{prefill,decode}_shared_workspace_bytes."""
    if kind == "prefill":
        return int(lib().lazyattn_prefill_shared_workspace_bytes(
            num_seqs, total_q, int(max_entries), int(plan_slots), Hq, Hkv, D))
    return int(lib().lazyattn_decode_shared_workspace_bytes(num_seqs, total_q, int(plan_slots),
                                                            Hq, Hkv, D))


def _shared(kind, q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_pos,
            rope_base, max_entries, plan, plan_items, plan_slots, out, workspace, stream):
    import torch
    total_q, Hq, D, num_blocks, Hkv, B = _dims(q, k_pool)
    num_seqs = kv_lens.numel()
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        need = shared_workspace_bytes(kind, num_seqs, total_q, max_entries, plan_slots, Hq,
                                      Hkv, D)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    name = f"lazyattn_{kind}_shared"
    rc = getattr(lib(), name)(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(block_meta),
        _ptr(kv_lens), _ptr(q_indptr), _ptr(q_pos), float(rope_base), num_seqs, total_q, Hq,
        Hkv, D, B, num_blocks, int(max_entries), _ptr(plan), int(plan_items), int(plan_slots),
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    check(rc, name)
    return out


def decode_shared(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_pos,
                  rope_base, max_entries, plan, plan_items, plan_slots, out=None,
                  workspace=None, stream=None):
    """lazyattn_decode_shared: decode over a shared-document plan (`plan` a device int32
    copy of decode_share_plan's result, plan_items / plan_slots its header [4] / [5])."""
    return _shared("decode", q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr,
                   q_pos, rope_base, max_entries, plan, plan_items, plan_slots, out, workspace,
                   stream)


def prefill_shared(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_pos,
                   rope_base, max_entries, plan, plan_items, plan_slots, out=None,
                   workspace=None, stream=None):
    """lazyattn_prefill_shared: a batch of any query lengths, its decode rows over a plan
    built with single_row_only=True."""
    return _shared("prefill", q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr,
                   q_pos, rope_base, max_entries, plan, plan_items, plan_slots, out, workspace,
                   stream)


def llama31_inv_freq(D, base=500000.0, factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
                     original_context=8192):
    """lazyattn_llama31_inv_freq: the Llama 3.1 frequency-scaled RoPE table (host, float64,
    D/2 radians per position) for the *_freqs entry points."""
    out = np.zeros(D // 2 if D > 0 else 1, dtype=np.float64)
    rc = lib().lazyattn_llama31_inv_freq(int(D), float(base), float(factor),
                                         float(low_freq_factor), float(high_freq_factor),
                                         float(original_context), out.ctypes.data)
    check(rc, "lazyattn_llama31_inv_freq")
    return out


def prefill_rotated_pool(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_pos,
                         rope_base, max_entries, out=None, workspace=None, stream=None):
    """lazyattn_prefill_rotated_pool: the materialised baseline (k_pool holds keys already
    rotated to the positions they are referenced at); returns out."""
    return _attention("prefill", q, k_pool, v_pool, block_table, block_meta, kv_lens,
                      q_indptr, q_pos, rope_base, max_entries, out, workspace, stream, True)


def decode_rotated_pool(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_pos,
                        rope_base, max_entries, out=None, workspace=None, stream=None):
    """lazyattn_decode_rotated_pool (materialised baseline); returns out."""
    return _attention("decode", q, k_pool, v_pool, block_table, block_meta, kv_lens,
                      q_indptr, q_pos, rope_base, max_entries, out, workspace, stream, True)


def materialize_rotated(k_pool, v_pool, block_table, block_meta, kv_lens, rope_base, n_entries,
                        dst_k=None, dst_v=None, dst_meta=None, stream=None):
    """lazyattn_materialize_rotated: private rotated copies of every entry's block; returns
    (dst_k, dst_v, dst_meta) (allocated with torch when not given)."""
    import torch
    num_blocks, Hkv, B, D = k_pool.shape
    if dst_k is None:
        dst_k = torch.empty((max(n_entries, 1), Hkv, B, D), dtype=k_pool.dtype,
                            device=k_pool.device)
    if dst_v is None:
        dst_v = torch.empty_like(dst_k)
    if dst_meta is None:
        dst_meta = torch.empty(max(n_entries, 1), dtype=torch.int32, device=k_pool.device)
    rc = lib().lazyattn_materialize_rotated(
        _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(block_meta), _ptr(kv_lens),
        float(rope_base), kv_lens.numel(), int(n_entries), Hkv, D, B, num_blocks, _ptr(dst_k),
        _ptr(dst_v), _ptr(dst_meta), _stream(stream))
    check(rc, "lazyattn_materialize_rotated")
    return dst_k, dst_v, dst_meta


def encode_meta(block_ids, offsets, block_table, B=BLOCK):
    """Host encoder: (int32 ids, int64 offsets, int32 CSR) -> uint32 words (numpy)."""
    ids = np.ascontiguousarray(block_ids, dtype=np.int32)
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    words = np.zeros(len(ids), dtype=np.uint32)
    bad = ctypes.c_int64(-1)
    rc = lib().lazyattn_encode_meta(ids.ctypes.data, offs.ctypes.data, bt.ctypes.data,
                                    len(bt) - 1, B, words.ctypes.data, ctypes.byref(bad))
    check(rc, f"lazyattn_encode_meta (first bad entry {bad.value})")
    return words


def debug_decode_meta(words, block_table, stream=None):
    """Device decoder of packed words (tests): returns (ids, offsets) int32 tensors."""
    import torch
    n = words.numel()
    ids = torch.empty(n, dtype=torch.int32, device=words.device)
    offs = torch.empty(n, dtype=torch.int32, device=words.device)
    rc = lib().lazyattn_debug_decode_meta(_ptr(words), _ptr(block_table),
                                          block_table.numel() - 1, n, BLOCK, _ptr(ids),
                                          _ptr(offs), _stream(stream))
    check(rc, "lazyattn_debug_decode_meta")
    return ids, offs


def probe_cus():
    """Compute units the probes (and the decode grid) are sized for."""
    return int(lib().lazyattn_probe_cus())


def probe_mfma(iters, cycles=None, scratch=None, stream=None):
    """lazyattn_probe_mfma: launches the MFMA loop; returns (cycles uint64-as-int64 tensor,
    flops of the launch). Time it with events on `stream`."""
    import torch
    n = probe_cus()
    if cycles is None:
        cycles = torch.empty(n * 8, dtype=torch.int64, device="cuda")
    if scratch is None:
        scratch = torch.empty(n * 512, dtype=torch.float32, device=cycles.device)
    rc = lib().lazyattn_probe_mfma(int(iters), _ptr(cycles), _ptr(scratch), _stream(stream))
    check(rc, "lazyattn_probe_mfma")
    return cycles, float(n) * 8 * iters * 16 * 2 * 32 * 32 * 16


def probe_read(buf, scratch=None, stream=None):
    """lazyattn_probe_read: reads every byte of the device tensor `buf` once; returns the
    uint32 scratch whose XOR is the XOR of buf's 32-bit words."""
    import torch
    if scratch is None:
        scratch = torch.empty(8 * probe_cus() * 256, dtype=torch.int32, device=buf.device)
    rc = lib().lazyattn_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(scratch),
                                   _stream(stream))
    check(rc, "lazyattn_probe_read")
    return scratch


def probe_gather(buf, chunk_ids, chunk_bytes, scratch=None, stream=None):
    """lazyattn_probe_gather: reads the chunk_bytes-sized chunks of the device tensor `buf`
    listed in chunk_ids (device int32), one wave per chunk; returns the uint32 scratch
    whose XOR is the XOR of the 32-bit words of the chunks read."""
    import torch
    if scratch is None:
        scratch = torch.empty(8 * probe_cus() * 256, dtype=torch.int32, device=buf.device)
    rc = lib().lazyattn_probe_gather(_ptr(buf), buf.numel() * buf.element_size(),
                                     _ptr(chunk_ids), chunk_ids.numel(), int(chunk_bytes),
                                     _ptr(scratch), _stream(stream))
    check(rc, "lazyattn_probe_gather")
    return scratch


def ingest_kv(k_new, v_new, slot_mapping, k_pool, v_pool, stream=None):
    """lazyattn_ingest_kv: scatter new tokens' K/V (bf16 [n, Hkv, D], unrotated) into the pool
    slots slot_mapping (int32 [n], block_id * B + slot; negative = skip)."""
    n, Hkv, D = k_new.shape
    num_blocks, _, B, _ = k_pool.shape
    rc = lib().lazyattn_ingest_kv(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), n, Hkv, D, B,
                                  num_blocks, _ptr(k_pool), _ptr(v_pool), _stream(stream))
    check(rc, "lazyattn_ingest_kv")


class PoolIndex:
    """Host index of the position-free pool (lazyattn_pool_*): document key -> block ids,
    references, LRU eviction of unreferenced documents, private blocks."""

    def __init__(self, num_blocks, block_size=BLOCK):
        self._h = ctypes.c_void_p()
        check(lib().lazyattn_pool_create(int(num_blocks), int(block_size), ctypes.byref(self._h)),
              "lazyattn_pool_create")
        self.block_size = int(block_size)

    def close(self):
        if self._h:
            lib().lazyattn_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def acquire(self, key, n_tokens):
        """-> (block ids int32 array, hit)."""
        cap = (int(n_tokens) + self.block_size - 1) // self.block_size
        buf = (ctypes.c_int32 * max(cap, 1))()
        n, hit = ctypes.c_int32(), ctypes.c_int32()
        check(lib().lazyattn_pool_acquire(self._h, ctypes.c_uint64(int(key)), int(n_tokens), buf,
                                          cap, ctypes.byref(n), ctypes.byref(hit)),
              "lazyattn_pool_acquire")
        return np.frombuffer(buf, dtype=np.int32, count=n.value).copy(), bool(hit.value)

    def release(self, key):
        check(lib().lazyattn_pool_release(self._h, ctypes.c_uint64(int(key))),
              "lazyattn_pool_release")

    def alloc_private(self, n_blocks):
        buf = (ctypes.c_int32 * max(int(n_blocks), 1))()
        check(lib().lazyattn_pool_alloc_private(self._h, int(n_blocks), buf),
              "lazyattn_pool_alloc_private")
        return np.frombuffer(buf, dtype=np.int32, count=int(n_blocks)).copy()

    def free_private(self, blocks):
        b = np.ascontiguousarray(blocks, dtype=np.int32)
        check(lib().lazyattn_pool_free_private(
            self._h, b.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(b)),
              "lazyattn_pool_free_private")

    def stats(self):
        st = PoolStats()
        check(lib().lazyattn_pool_stats(self._h, ctypes.byref(st)), "lazyattn_pool_stats")
        return {name: getattr(st, name) for name, _ in PoolStats._fields_}
