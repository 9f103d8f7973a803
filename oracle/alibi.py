"""ALiBi over the position-free pool, float64 (test infrastructure only).

The pages state that deferring position to the attention kernel works for other relative
position encodings as well, ALiBi among them (technical summary, "Key Contributions").
ALiBi (Press, Smith, Lewis, "Train Short, Test Long", 2022) leaves queries and keys
unrotated and adds a per-head linear penalty to each score: for a query of head h at
logical position p and a key at logical position L <= p,

    s = q . k / sqrt(D) - m_h (p - L).

Position again enters only through logical positions, so the same position-free pool and
block tables serve it. Steps, as the definition reads:
  1. gather each sequence's keys and values in logical order from its block table (no
     rotation), with their logical positions L = off_t + j;
  2. score every (query row, key) pair of a head as above, for the key/value head
     floor(h / G);
  3. causal mask on logical positions (L <= p), max-subtracted softmax in float64, output
     sum p_j v_j; a row with no visible key outputs 0.
"""
import numpy as np

from .attention import materialise, bf16_bits_to_f64


def alibi_slopes(H):
    """The geometric slopes of the ALiBi paper: 2^(-8 i / H), i = 1..H, for H a power of
    two; otherwise those of the largest power of two n < H followed by every other slope of
    2n, up to H in all."""
    def pow2(n):
        return [2.0 ** (-8.0 * i / n) for i in range(1, n + 1)]
    n = 1 << (int(H).bit_length() - 1)
    if n == H:
        return np.array(pow2(H))
    return np.array(pow2(n) + pow2(2 * n)[0::2][: H - n])


def attend_alibi(q, q_pos, K, V, key_pos, slopes):
    """q [n_q, Hq, D] float64; K, V [Hkv, n, D]; slopes [Hq]."""
    n_q, Hq, D = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    out = np.zeros((n_q, Hq, D))
    if K.shape[1] == 0:
        return out
    qp = np.asarray(q_pos, dtype=np.int64)[:, None]
    kp = np.asarray(key_pos, dtype=np.int64)[None, :]
    visible = kp <= qp
    dist = (qp - kp).astype(np.float64)
    for h in range(Hq):
        g = h // G
        s = q[:, h, :] @ K[g].T / np.sqrt(D) - float(slopes[h]) * dist
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        any_vis = np.isfinite(m[:, 0])
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.where(visible, np.exp(s - m), 0.0)
        l = p.sum(axis=1, keepdims=True)
        o = (p @ V[g]) / np.where(l > 0, l, 1.0)
        out[:, h, :] = np.where(any_vis[:, None], o, 0.0)
    return out


def alibi_attention(q, k_pool, v_pool, seq_block_ids, seq_offsets, kv_lens, q_indptr, q_pos,
                    slopes, B):
    """Whole-batch output [total_q, Hq, D] float64 (bf16 bit inputs as for lazy_attention)."""
    total_q, Hq, D = q.shape
    out = np.zeros((total_q, Hq, D))
    for s in range(len(kv_lens)):
        r0, r1 = int(q_indptr[s]), int(q_indptr[s + 1])
        if r1 == r0:
            continue
        K, V, key_pos = materialise(k_pool, v_pool, seq_block_ids[s], seq_offsets[s],
                                    int(kv_lens[s]), B, 10000.0, rotate_keys=False)
        qf = bf16_bits_to_f64(q[r0:r1]) if q.dtype == np.uint16 else np.asarray(q[r0:r1], float)
        out[r0:r1] = attend_alibi(qf, q_pos[r0:r1], K, V, key_pos, slopes)
    return out


def alibi_rows(q, k_pool, v_pool, seq_block_ids, seq_offsets, kv_lens, q_indptr, q_pos,
               slopes, B, seq, rows):
    """Output rows `rows` (global row indices of sequence `seq`), float64 [len(rows), Hq, D]."""
    rows = np.asarray(rows, dtype=np.int64)
    K, V, key_pos = materialise(k_pool, v_pool, seq_block_ids[seq], seq_offsets[seq],
                                int(kv_lens[seq]), B, 10000.0, rotate_keys=False)
    qf = bf16_bits_to_f64(q[rows]) if q.dtype == np.uint16 else np.asarray(q[rows], float)
    return attend_alibi(qf, q_pos[rows], K, V, key_pos, slopes)
