"""Pool whose keys carry their rotation inside their document, float64 (test
infrastructure only).

The technical summary's "Technical Implementation" contrasts rotating each cached key
twice (back to position zero, then to its target) with rotating it once by the difference,
and lets decode re-rotate the query only where the relative offset changes, at a new
document. Both read naturally for a cache whose keys were stored with RoPE at their
positions INSIDE their document (as a model produces them when it encodes the document on
its own, from position 0). This module states what attention over such a pool must equal,
from the definition of RoPE attention:

  - entry t of a block table has logical offset off_t (slot j at L = off_t + j) and a
    stored offset st_t: slot j of its block holds R(st_t + j) k for the un-rotated key k
    (st_t = 16 b for the b-th block of a document stored from position 0);
  - the logical key is R(L) k. The oracle recovers k by applying R(-(st_t + j)) and then
    rotates it to L (two float64 rotations, exactly the definition);
  - values are stored as they are; queries are rotated by R(p); causal mask, softmax and
    output as in attention.py.
"""
import numpy as np

from .attention import attend, bf16_bits_to_f64, _rot_queries
from .rope import rotate


def materialise_doc_rotated(k_pool, v_pool, block_ids, offsets, stored_offsets, kv_len, B,
                            base):
    """Logical-order K_hat (= R(L) k) and V of one sequence from a document-rotated pool.

    k_pool, v_pool: bf16 bits (or floats) [num_blocks, Hkv, B, D]; block_ids, offsets,
    stored_offsets:
    per-entry physical id, logical offset of slot 0 and stored rotation offset of slot 0.
    Returns K_hat [Hkv, n, D], V_hat [Hkv, n, D], key_pos [n].
    """
    T = len(block_ids)
    Hkv, D = k_pool.shape[1], k_pool.shape[3]
    if T == 0:
        return np.zeros((Hkv, 0, D)), np.zeros((Hkv, 0, D)), np.zeros(0, dtype=np.int64)
    if kv_len <= (T - 1) * B or kv_len > T * B:
        raise ValueError("kv_len inconsistent with the number of entries")
    ks, vs, ps = [], [], []
    for t in range(T):
        n_t = B if t < T - 1 else kv_len - (T - 1) * B
        blk = int(block_ids[t])
        kb, vb = k_pool[blk][:, :n_t, :], v_pool[blk][:, :n_t, :]
        kb = bf16_bits_to_f64(kb) if kb.dtype == np.uint16 else np.asarray(kb, np.float64)
        vb = bf16_bits_to_f64(vb) if vb.dtype == np.uint16 else np.asarray(vb, np.float64)
        j = np.arange(n_t, dtype=np.int64)
        raw = rotate(kb, -(int(stored_offsets[t]) + j)[None, :], base)   # R(-(st + j))
        pos = int(offsets[t]) + j
        ks.append(rotate(raw, pos[None, :], base))                       # R(L)
        vs.append(vb)
        ps.append(pos)
    return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1), np.concatenate(ps)


def doc_rotated_attention(q, k_pool, v_pool, seq_block_ids, seq_offsets, seq_stored,
                          kv_lens, q_indptr, q_pos, base, B):
    """Whole-batch output, float64 [total_q, Hq, D], over a document-rotated pool."""
    total_q, Hq, D = q.shape
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    for s in range(len(kv_lens)):
        r0, r1 = int(q_indptr[s]), int(q_indptr[s + 1])
        if r1 == r0:
            continue
        K, V, key_pos = materialise_doc_rotated(k_pool, v_pool, seq_block_ids[s],
                                                seq_offsets[s], seq_stored[s],
                                                int(kv_lens[s]), B, base)
        out[r0:r1] = attend(_rot_queries(q[r0:r1], q_pos[r0:r1], base), q_pos[r0:r1], K, V,
                            key_pos)
    return out


def doc_rotated_rows(q, k_pool, v_pool, seq_block_ids, seq_offsets, seq_stored, kv_lens,
                     q_indptr, q_pos, base, B, seq, rows):
    """Output of selected query rows (global indices) of one sequence."""
    rows = np.asarray(rows, dtype=np.int64)
    K, V, key_pos = materialise_doc_rotated(k_pool, v_pool, seq_block_ids[seq],
                                            seq_offsets[seq], seq_stored[seq],
                                            int(kv_lens[seq]), B, base)
    return attend(_rot_queries(q[rows], q_pos[rows], base), q_pos[rows], K, V, key_pos)
