"""Small-workload builders shared by CPU and GPU tests (no attention arithmetic)."""
import numpy as np

from workload import RequestLayout, Segment, build


def oracle_out(wl, rows=None, seq=None, base=None, rotary_dim=None):
    """The oracle on a workload; `base` overrides its RoPE base (a number or a table),
    `rotary_dim` selects partial rotary."""
    import oracle
    if rows is None:
        return oracle.lazy_attention(wl.q_bits, wl.k_bits, wl.v_bits,
                                     [wl.compact_ids(s) for s in range(wl.num_seqs)],
                                     wl.seq_offsets, wl.kv_lens, wl.q_indptr, wl.q_pos,
                                     wl.rope_base if base is None else base, wl.B,
                                     rotary_dim=rotary_dim)
    return oracle.attention_rows(wl.q_bits, wl.k_bits, wl.v_bits,
                                 [wl.compact_ids(s) if s == seq else None
                                  for s in range(wl.num_seqs)],
                                 wl.seq_offsets, wl.kv_lens, wl.q_indptr, wl.q_pos,
                                 wl.rope_base if base is None else base, wl.B, seq, rows,
                                 rotary_dim=rotary_dim)


def small(Hq=4, Hkv=2, D=16, B=16, base=10000.0, seed=7, segs=None, q_len=None,
          q_pos=None, n_docs=3, doc_tokens=32, q_scale=1.0, requests=None):
    """One or more requests from explicit segment lists (default: 2 docs + 20 new tokens)."""
    if requests is None:
        if segs is None:
            segs = [Segment("doc", 5, doc=0), Segment("doc", 40, doc=2),
                    Segment("private", 72, tokens=20)]
        last = segs[-1]
        ntok = last.tokens if last.kind == "private" else doc_tokens
        requests = [RequestLayout(segs, q_len if q_len is not None else ntok, q_pos)]
    return build("small", Hq, Hkv, D, B, base, n_docs, doc_tokens, requests, seed,
                 q_scale=q_scale)


def dense_request(n_tokens, start=0):
    """A request whose tokens are all new and all queried, positions start..start+n-1."""
    return RequestLayout([Segment("private", start, tokens=n_tokens)], n_tokens)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def doc_stored_offsets(wl):
    """Stored offsets of a pool whose document keys were encoded per document."""
    return wl.doc_stored_offsets()


def doc_rotated_pool(wl, stored, as_bits=True):
    """wl's compact K pool with every block's keys rotated by R(stored + j) (the oracle's
    rotation); bf16 bits (round to nearest even) or float64. A block must have one stored
    offset wherever it is referenced."""
    from oracle.attention import bf16_bits_to_f64
    from oracle.rope import rotate
    from workload.rag import f32_to_bf16_bits
    st_of = {}
    for s in range(wl.num_seqs):
        for c, st in zip(wl.compact_ids(s), stored[s]):
            if st_of.setdefault(int(c), int(st)) != int(st):
                raise ValueError("a block is referenced with two stored offsets")
    k = bf16_bits_to_f64(wl.k_bits)
    j = np.arange(wl.B, dtype=np.int64)
    for c, st in st_of.items():
        k[c] = rotate(k[c], (st + j)[None, :], wl.rope_base)
    if not as_bits:
        return k
    nan = np.isnan(k)                       # padding slots stay NaN
    bits = f32_to_bf16_bits(np.where(nan, 0.0, k).astype(np.float32))
    return np.where(nan, np.uint16(0x7FC0), bits).astype(np.uint16)
