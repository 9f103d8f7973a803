"""Materialise-then-attend reference for LazyAttention (test infrastructure only).

What the deferred method must equal (LazyAttention summary, "Mathematical
Equivalence"): attention over a KV copy whose keys carry RoPE at their absolute
logical positions. The steps below follow that definition directly:

  1. materialise: for every block-table entry t (physical block id_t, logical
     offset off_t) and slot j < n_t, the key at logical position L = off_t + j
     is R(L) k (float64) and the value is v unchanged; only the sequence's last
     entry may be partial, n_t = kv_len - (T-1) B;
  2. rotate each query row by R(p) at its logical position p;
  3. score s = <R(p) q, R(L) k> / sqrt(D) for the key/value head
     floor(h / G) of query head h (grouped-query attention, G = Hq / Hkv);
  4. causal mask on logical positions: a key is visible iff L <= p;
  5. max-subtracted softmax over visible keys in float64, output sum p_j v_j;
     a row with no visible key outputs 0.

Inputs are the same seeded tensors the GPU receives, as raw bf16 bit patterns
(uint16) that are widened exactly to float64.
"""
import numpy as np

from .rope import rotate


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def materialise(k_pool, v_pool, block_ids, offsets, kv_len, B, base, rotate_keys=True,
                rotary_dim=None):
    """Copy a sequence's blocks into logical order with eager RoPE on keys.

    k_pool, v_pool: uint16 bf16 bits [num_blocks, Hkv, B, D] (or float arrays).
    block_ids, offsets: per-entry physical block id and logical offset of slot 0.
    rotate_keys=False reads a pool whose keys already carry R(L) (the materialised
    baseline the method is compared with): keys are then used as stored.
    rotary_dim: partial rotary (only the first rotary_dim dims rotated; rope.rotate).
    Returns K_hat [Hkv, n, D] float64 (rotated), V_hat [Hkv, n, D], key_pos [n].
    """
    T = len(block_ids)
    if kv_len <= (T - 1) * B or kv_len > T * B:
        raise ValueError("kv_len inconsistent with the number of entries")
    if T == 0:                                   # no entries: no keys
        Hkv, D = k_pool.shape[1], k_pool.shape[3]
        return (np.zeros((Hkv, 0, D)), np.zeros((Hkv, 0, D)), np.zeros(0, dtype=np.int64))
    ks, vs, ps = [], [], []
    for t in range(T):
        n_t = B if t < T - 1 else kv_len - (T - 1) * B
        blk = int(block_ids[t])
        kb = k_pool[blk][:, :n_t, :]
        vb = v_pool[blk][:, :n_t, :]
        if kb.dtype == np.uint16:
            kb = bf16_bits_to_f64(kb)
        if vb.dtype == np.uint16:
            vb = bf16_bits_to_f64(vb)
        pos = int(offsets[t]) + np.arange(n_t, dtype=np.int64)
        ks.append(rotate(kb, pos[None, :], base, rotary_dim) if rotate_keys
                  else np.asarray(kb, dtype=np.float64))
        vs.append(np.asarray(vb, dtype=np.float64))
        ps.append(pos)
    return (np.concatenate(ks, axis=1), np.concatenate(vs, axis=1),
            np.concatenate(ps))


def attend(q_rot, q_pos, K_hat, V_hat, key_pos):
    """Causal softmax attention in float64.

    q_rot: [n_q, Hq, D] already rotated by R(q_pos); K_hat/V_hat [Hkv, n, D].
    """
    n_q, Hq, D = q_rot.shape
    Hkv = K_hat.shape[0]
    G = Hq // Hkv
    out = np.zeros((n_q, Hq, D), dtype=np.float64)
    if K_hat.shape[1] == 0:                      # no key at all: every row sees none
        return out
    visible = key_pos[None, :] <= np.asarray(q_pos, dtype=np.int64)[:, None]
    scale = 1.0 / np.sqrt(D)
    for h in range(Hq):
        g = h // G
        s = (q_rot[:, h, :] @ K_hat[g].T) * scale           # [n_q, n]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        any_vis = np.isfinite(m[:, 0])
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.where(visible, np.exp(s - m), 0.0)
        l = p.sum(axis=1, keepdims=True)
        o = (p @ V_hat[g]) / np.where(l > 0, l, 1.0)
        out[:, h, :] = np.where(any_vis[:, None], o, 0.0)
    return out


def _rot_queries(q, q_pos, base, rotary_dim=None):
    qf = bf16_bits_to_f64(q) if q.dtype == np.uint16 else np.asarray(q, np.float64)
    return rotate(qf, np.asarray(q_pos, dtype=np.int64)[:, None], base, rotary_dim)


def lazy_attention(q, k_pool, v_pool, seq_block_ids, seq_offsets, kv_lens,
                   q_indptr, q_pos, base, B, rotate_keys=True, rotary_dim=None):
    """Whole-batch reference output, float64 [total_q, Hq, D].

    q: bf16 bits [total_q, Hq, D]; seq_block_ids / seq_offsets: one array per
    sequence; q_indptr: CSR rows of q per sequence; q_pos: logical position of
    each query row. One sequence at a time, to bound memory.
    """
    total_q, Hq, D = q.shape
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    for s in range(len(kv_lens)):
        r0, r1 = int(q_indptr[s]), int(q_indptr[s + 1])
        if r1 == r0:
            continue
        K_hat, V_hat, key_pos = materialise(
            k_pool, v_pool, seq_block_ids[s], seq_offsets[s], int(kv_lens[s]), B, base,
            rotate_keys, rotary_dim)
        qr = _rot_queries(q[r0:r1], q_pos[r0:r1], base, rotary_dim)
        out[r0:r1] = attend(qr, q_pos[r0:r1], K_hat, V_hat, key_pos)
    return out


def attention_rows(q, k_pool, v_pool, seq_block_ids, seq_offsets, kv_lens,
                   q_indptr, q_pos, base, B, seq, rows, rotate_keys=True, rotary_dim=None):
    """Reference output of selected query rows (global row indices) of one sequence."""
    rows = np.asarray(rows, dtype=np.int64)
    r0, r1 = int(q_indptr[seq]), int(q_indptr[seq + 1])
    if np.any(rows < r0) or np.any(rows >= r1):
        raise ValueError("rows must belong to the sequence")
    K_hat, V_hat, key_pos = materialise(
        k_pool, v_pool, seq_block_ids[seq], seq_offsets[seq], int(kv_lens[seq]), B, base,
        rotate_keys, rotary_dim)
    qr = _rot_queries(q[rows], q_pos[rows], base, rotary_dim)
    return attend(qr, q_pos[rows], K_hat, V_hat, key_pos)


def rotated_pool(k_pool, seq_block_ids, seq_offsets, kv_lens, B, base):
    """Float64 copy of k_pool in which every referenced key slot holds R(L) k at the
    logical position L it is referenced at (the materialised baseline's pool). Each block
    may be referenced once; unreferenced blocks are copied unrotated."""
    kp = bf16_bits_to_f64(k_pool) if k_pool.dtype == np.uint16 else np.array(k_pool, np.float64)
    out = kp.copy()
    seen = set()
    for s in range(len(kv_lens)):
        T = len(seq_block_ids[s])
        for t in range(T):
            blk = int(seq_block_ids[s][t])
            if blk in seen:
                raise ValueError("a block referenced twice cannot hold one rotation")
            seen.add(blk)
            n_t = B if t < T - 1 else int(kv_lens[s]) - (T - 1) * B
            pos = int(seq_offsets[s][t]) + np.arange(n_t, dtype=np.int64)
            out[blk][:, :n_t, :] = rotate(kp[blk][:, :n_t, :], pos[None, :], base)
    return out
