"""Brute-force attention for tiny inputs, written independently of oracle/.

Every step is spelled out with Python loops: an explicit D x D RoPE matrix per
position (2 x 2 rotations of the (k, k + D/2) pairs with angle n * base^(-2k/D)),
an explicit boolean mask matrix over logical positions, explicit exp/sum
softmax. Only used on inputs of a few dozen keys.
"""
import math

import numpy as np


def bits_to_float(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rope_matrix(n, D, base):
    h = D // 2
    M = np.zeros((D, D))
    for k in range(h):
        ang = n * math.pow(base, -2.0 * k / D)
        c, s = math.cos(ang), math.sin(ang)
        M[k, k] = c
        M[k, k + h] = -s
        M[k + h, k] = s
        M[k + h, k + h] = c
    return M


def brute_attention(wl):
    """Output [total_q, Hq, D] float64 of a workload.Workload, by explicit loops."""
    D, B, base = wl.D, wl.B, wl.rope_base
    G = wl.Hq // wl.Hkv
    lookup = {int(pid): i for i, pid in enumerate(wl.pool_ids)}
    out = np.zeros((wl.total_q, wl.Hq, D))
    for s in range(wl.num_seqs):
        keys, vals, kpos = [], [], []       # per key: [Hkv, D]
        T = len(wl.seq_block_ids[s])
        for t in range(T):
            nslots = B if t < T - 1 else int(wl.kv_lens[s]) - (T - 1) * B
            blk = lookup[int(wl.seq_block_ids[s][t])]
            for j in range(nslots):
                L = int(wl.seq_offsets[s][t]) + j
                kv = bits_to_float(wl.k_bits[blk, :, j, :])
                vv = bits_to_float(wl.v_bits[blk, :, j, :])
                R = rope_matrix(L, D, base)
                keys.append(np.stack([R @ kv[g] for g in range(wl.Hkv)]))
                vals.append(vv)
                kpos.append(L)
        n = len(keys)
        for r in range(int(wl.q_indptr[s]), int(wl.q_indptr[s + 1])):
            p = int(wl.q_pos[r])
            mask = [kpos[i] <= p for i in range(n)]
            R = rope_matrix(p, D, base)
            for h in range(wl.Hq):
                g = h // G
                qv = R @ bits_to_float(wl.q_bits[r, h])
                scores = [float(qv @ keys[i][g]) / math.sqrt(D) if mask[i] else None
                          for i in range(n)]
                vis = [x for x in scores if x is not None]
                if not vis:
                    continue
                m = max(vis)
                w = [math.exp(x - m) if x is not None else 0.0 for x in scores]
                tot = sum(w)
                o = np.zeros(D)
                for i in range(n):
                    if w[i]:
                        o += (w[i] / tot) * vals[i][g]
                out[r, h] = o
    return out
