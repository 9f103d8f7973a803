"""Synthetic RAG-shaped inputs for position-agnostic paged attention.

Stand-in for the RAG benchmarks the LazyAttention paper evaluates on (its
"Experimental Results": 2WikiMQA, HotpotQA, TriviaQA, NarrativeQA), which are
not available here: only the shapes matter for the attention path, so every
tensor is seeded N(0, 1) data rounded to bf16, and documents are drawn with the
skewed (Zipf) reuse the paper's problem statement describes.

Pool layout: `n_docs` documents of `doc_tokens` tokens, each split into
`doc_tokens / B` blocks whose physical ids are a seeded permutation of the pool,
followed by private blocks (question / suffix / decode-token K/V) of every
request, also scattered by the same permutation. Only referenced blocks carry
data; the device pool is pre-filled with bf16 NaN elsewhere, and padding slots
of a request's partial last block are NaN too, so a kernel that reads outside
the visible keys produces NaN.

Seeded streams (numpy default_rng with a SeedSequence list):
  [seed, 0]            layout: rank->doc permutation, Zipf draws, starts, gaps
  [seed, 1, doc]       K then V of one document
  [seed, 2]            all query rows
  [seed, 3, req, seg]  K then V of a request's private segment
  [seed, 4]            physical block-id permutation
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BF16_NAN = 0x7FC0


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 to bf16 (round to nearest even), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any((u & 0x7FFFFFFF) > 0x7F800000):
        raise ValueError("NaN input")
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def _to_bf16_fast(x: np.ndarray) -> np.ndarray:
    """Same rounding as f32_to_bf16_bits (checked by a test), via torch's CPU cast."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        return f32_to_bf16_bits(x)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def harmonic(N: int, s: float) -> float:
    return float(np.sum(np.arange(1, N + 1, dtype=np.float64) ** (-s)))


def _zipf_cdf(N: int, s: float) -> np.ndarray:
    w = np.arange(1, N + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    return cdf / cdf[-1]


def zipf_ranks(rng, n: int, N: int, s: float, cdf=None) -> np.ndarray:
    """n iid draws of a finite Zipf(s) over ranks 1..N, P(k) ~ k^-s (inverse CDF)."""
    if cdf is None:
        cdf = _zipf_cdf(N, s)
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), N - 1) + 1


@dataclass
class Segment:
    kind: str            # "doc" or "private"
    start: int           # logical position of the segment's first token
    doc: int = -1        # document id for kind == "doc"
    tokens: int = 0      # token count for kind == "private"


@dataclass
class RequestLayout:
    segments: List[Segment]
    q_len: int                            # queries = last q_len tokens of the request
    q_pos: Optional[np.ndarray] = None    # explicit query positions (overrides)


@dataclass
class Workload:
    name: str
    Hq: int
    Hkv: int
    D: int
    B: int
    rope_base: float
    num_blocks: int
    seq_block_ids: List[np.ndarray]       # per sequence: int32 physical id per entry
    seq_offsets: List[np.ndarray]         # per sequence: int64 logical offset of slot 0
    kv_lens: np.ndarray                   # int32 [S]
    q_indptr: np.ndarray                  # int32 [S+1]
    q_pos: np.ndarray                     # int32 [total_q]
    q_bits: np.ndarray                    # uint16 [total_q, Hq, D]
    pool_ids: np.ndarray                  # int32 [R] sorted referenced physical ids
    k_bits: np.ndarray                    # uint16 [R, Hkv, B, D]
    v_bits: np.ndarray                    # uint16 [R, Hkv, B, D]
    layouts: List[RequestLayout] = field(default_factory=list)
    info: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.kv_lens)

    @property
    def total_q(self) -> int:
        return int(self.q_indptr[-1])

    @property
    def block_table(self) -> np.ndarray:
        """CSR row pointers (int32 [S+1]) into the flat entry arrays."""
        n = np.array([len(x) for x in self.seq_block_ids], dtype=np.int64)
        return np.concatenate([[0], np.cumsum(n)]).astype(np.int32)

    @property
    def flat_block_ids(self) -> np.ndarray:
        return np.concatenate(self.seq_block_ids).astype(np.int32)

    @property
    def flat_offsets(self) -> np.ndarray:
        return np.concatenate(self.seq_offsets).astype(np.int64)

    def compact_ids(self, seq: int) -> np.ndarray:
        """Entry block ids of `seq` re-indexed into the compact k_bits/v_bits arrays."""
        return np.searchsorted(self.pool_ids, self.seq_block_ids[seq]).astype(np.int64)

    def doc_stored_offsets(self) -> List[np.ndarray]:
        """Per sequence and entry, where slot 0 of the entry's block sits in the sequence the
        block was first laid out in: 16 b for the b-th block of a document (its position
        inside the document), the logical offset for a private block. This is the stored
        offset of a pool whose document keys were encoded per document from position 0."""
        doc_blocks = self.info["doc_tokens"] // self.B
        out = []
        for lay in self.layouts:
            st = []
            for sg in lay.segments:
                if sg.kind == "doc":
                    st += [self.B * b for b in range(doc_blocks)]
                else:
                    st += [sg.start + self.B * b for b in range(-(-sg.tokens // self.B))]
            out.append(np.array(st, dtype=np.int64))
        return out

    def compact_views(self):
        """(k_pool, v_pool, per-seq compact ids) for host-side references."""
        return self.k_bits, self.v_bits, [self.compact_ids(s) for s in range(self.num_seqs)]

    def to_device(self, device="cuda"):
        """Device tensors: q, full NaN-filled pools holding the referenced blocks, CSR arrays."""
        import torch
        shape = (self.num_blocks, self.Hkv, self.B, self.D)
        k_pool = torch.empty(shape, dtype=torch.int16, device=device)
        v_pool = torch.empty(shape, dtype=torch.int16, device=device)
        k_pool.fill_(BF16_NAN)
        v_pool.fill_(BF16_NAN)
        idx = torch.from_numpy(self.pool_ids.astype(np.int64)).to(device)
        k_pool.index_copy_(0, idx, torch.from_numpy(self.k_bits.view(np.int16)).to(device))
        v_pool.index_copy_(0, idx, torch.from_numpy(self.v_bits.view(np.int16)).to(device))
        q = torch.from_numpy(self.q_bits.view(np.int16)).to(device).view(torch.bfloat16)

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
        return dict(q=q, k_pool=k_pool.view(torch.bfloat16), v_pool=v_pool.view(torch.bfloat16),
                    kv_lens=i32(self.kv_lens), q_indptr=i32(self.q_indptr),
                    q_pos=i32(self.q_pos), block_table=i32(self.block_table))


def build(name, Hq, Hkv, D, B, rope_base, n_docs, doc_tokens, layouts, seed,
          q_scale: float = 1.0) -> Workload:
    """Materialise tensors for explicit request layouts (seeded, deterministic)."""
    if doc_tokens % B:
        raise ValueError("documents must be whole blocks")
    doc_blocks = doc_tokens // B
    priv = []                               # (request, segment, block count)
    for r, lay in enumerate(layouts):
        for i, sg in enumerate(lay.segments):
            if sg.kind == "private":
                if i != len(lay.segments) - 1 and sg.tokens % B:
                    raise ValueError("only a request's last segment may end in a partial block")
                priv.append((r, i, -(-sg.tokens // B)))
    n_priv = sum(p[2] for p in priv)
    num_blocks = n_docs * doc_blocks + n_priv
    perm = np.random.default_rng([seed, 4]).permutation(num_blocks).astype(np.int64)
    doc_phys = perm[: n_docs * doc_blocks].reshape(n_docs, doc_blocks)
    priv_phys, cur = {}, n_docs * doc_blocks
    for r, i, nb in priv:
        priv_phys[(r, i)] = perm[cur: cur + nb]
        cur += nb

    seq_ids, seq_offs, kv_lens, q_counts, q_pos_all = [], [], [], [], []
    for r, lay in enumerate(layouts):
        ids, offs, toks, last_pos = [], [], 0, []
        for i, sg in enumerate(lay.segments):
            if sg.kind == "doc":
                for b in range(doc_blocks):
                    ids.append(doc_phys[sg.doc, b])
                    offs.append(sg.start + b * B)
                toks += doc_tokens
                last_pos = list(range(sg.start, sg.start + doc_tokens))
            else:
                pb = priv_phys[(r, i)]
                for b in range(len(pb)):
                    ids.append(pb[b])
                    offs.append(sg.start + b * B)
                toks += sg.tokens
                last_pos = list(range(sg.start, sg.start + sg.tokens))
        seq_ids.append(np.array(ids, dtype=np.int32))
        seq_offs.append(np.array(offs, dtype=np.int64))
        kv_lens.append(toks)
        if lay.q_pos is not None:
            qp = np.asarray(lay.q_pos, dtype=np.int64)
        else:
            if lay.q_len > len(last_pos):
                raise ValueError("queries must fit in the last segment")
            qp = np.array(last_pos[len(last_pos) - lay.q_len:], dtype=np.int64)
        q_counts.append(len(qp))
        q_pos_all.append(qp)

    # referenced pool content (one seeded stream per document / private segment)
    ref_docs = sorted({sg.doc for lay in layouts for sg in lay.segments if sg.kind == "doc"})
    shape_doc = (doc_blocks, Hkv, B, D)

    def _doc(d):
        g = np.random.default_rng([seed, 1, d])
        kf = g.standard_normal(shape_doc, dtype=np.float32)
        vf = g.standard_normal(shape_doc, dtype=np.float32)
        return _to_bf16_fast(kf), _to_bf16_fast(vf)

    def _priv(item):
        r, i, nb = item
        g = np.random.default_rng([seed, 3, r, i])
        shp = (nb, Hkv, B, D)
        kb = _to_bf16_fast(g.standard_normal(shp, dtype=np.float32))
        vb = _to_bf16_fast(g.standard_normal(shp, dtype=np.float32))
        pad = nb * B - layouts[r].segments[i].tokens
        if pad:
            kb[-1, :, B - pad:, :] = BF16_NAN
            vb[-1, :, B - pad:, :] = BF16_NAN
        return kb, vb

    with ThreadPoolExecutor(max_workers=8) as ex:
        doc_kv = list(ex.map(_doc, ref_docs))
        priv_kv = list(ex.map(_priv, priv))
    k_parts = [k for k, _ in doc_kv] + [k for k, _ in priv_kv]
    v_parts = [v for _, v in doc_kv] + [v for _, v in priv_kv]
    blocks_ids = [doc_phys[d] for d in ref_docs] + [priv_phys[(r, i)] for r, i, _ in priv]
    all_ids = np.concatenate(blocks_ids) if blocks_ids else np.zeros(0, np.int64)
    order = np.argsort(all_ids, kind="stable")
    empty = np.zeros((0, Hkv, B, D), np.uint16)
    k_bits = np.concatenate(k_parts)[order] if k_parts else empty
    v_bits = np.concatenate(v_parts)[order] if v_parts else empty

    total_q = int(sum(q_counts))
    q = np.random.default_rng([seed, 2]).standard_normal((total_q, Hq, D), dtype=np.float32)
    q_bits = _to_bf16_fast(q * np.float32(q_scale))
    q_indptr = np.concatenate([[0], np.cumsum(q_counts)]).astype(np.int32)
    return Workload(
        name=name, Hq=Hq, Hkv=Hkv, D=D, B=B, rope_base=float(rope_base),
        num_blocks=num_blocks, seq_block_ids=seq_ids, seq_offsets=seq_offs,
        kv_lens=np.array(kv_lens, dtype=np.int32), q_indptr=q_indptr,
        q_pos=np.concatenate(q_pos_all).astype(np.int32) if q_pos_all else np.zeros(0, np.int32),
        q_bits=q_bits, pool_ids=all_ids[order].astype(np.int32),
        k_bits=k_bits, v_bits=v_bits, layouts=list(layouts),
        info=dict(seed=seed, n_docs=n_docs, doc_tokens=doc_tokens,
                  referenced_docs=len(ref_docs)))


def _draw_docs(rng, n, n_docs, s, replace, rank_to_doc, cdf):
    """Zipf draws; without replacement, repeats are rejected and redrawn."""
    if replace:
        return [int(d) for d in rank_to_doc[zipf_ranks(rng, n, n_docs, s, cdf) - 1]]
    out, seen = [], set()
    while len(out) < n:
        d = int(rank_to_doc[zipf_ranks(rng, 1, n_docs, s, cdf)[0] - 1])
        if d not in seen:
            seen.add(d)
            out.append(d)
    return out


@dataclass(frozen=True)
class Group:
    count: int            # requests in this group
    n_docs: int           # documents per request
    private_tokens: int   # new tokens after the documents (question/suffix/decode token)
    q_len: int            # query rows (the last q_len private tokens)
    replace: bool = False  # draw documents with replacement within a request
    gap_max: int = 0      # gap ~ U{0..gap_max} before every document and the suffix


@dataclass(frozen=True)
class Config:
    name: str
    Hq: int
    Hkv: int
    D: int
    B: int
    rope_base: float
    n_docs: int
    doc_tokens: int
    zipf_s: float
    groups: tuple
    start_max: int = 511
    description: str = ""


def layouts_for(cfg: Config, seed: int, no_reuse: bool = False) -> List[RequestLayout]:
    """Request layouts of a configuration. no_reuse builds the control of the same shape in
    which every document appears once in the whole batch (documents taken in the order of a
    seeded permutation instead of Zipf draws), so no K/V block is read twice."""
    rng = np.random.default_rng([seed, 0])
    rank_to_doc = rng.permutation(cfg.n_docs)
    cdf = _zipf_cdf(cfg.n_docs, cfg.zipf_s)
    distinct = np.random.default_rng([seed, 5]).permutation(cfg.n_docs)
    if no_reuse and sum(g.count * g.n_docs for g in cfg.groups) > cfg.n_docs:
        raise ValueError(f"{cfg.name}: not enough documents for a no-reuse batch")
    used = 0
    lays = []
    for grp in cfg.groups:
        for _ in range(grp.count):
            if no_reuse:
                docs = [int(d) for d in distinct[used:used + grp.n_docs]]
                used += grp.n_docs
            else:
                docs = _draw_docs(rng, grp.n_docs, cfg.n_docs, cfg.zipf_s, grp.replace,
                                  rank_to_doc, cdf)
            pos = int(rng.integers(0, cfg.start_max + 1)) if cfg.start_max > 0 else 0
            segs = []
            for d in docs:
                if grp.gap_max:
                    pos += int(rng.integers(0, grp.gap_max + 1))
                segs.append(Segment("doc", pos, doc=int(d)))
                pos += cfg.doc_tokens
            if grp.gap_max:
                pos += int(rng.integers(0, grp.gap_max + 1))
            segs.append(Segment("private", pos, tokens=grp.private_tokens))
            lays.append(RequestLayout(segs, grp.q_len))
    return lays


CONFIGS = {
    "tiny-prefill-4q1kv-d64": Config(
        "tiny-prefill-4q1kv-d64", Hq=4, Hkv=1, D=64, B=16, rope_base=10000.0,
        n_docs=2, doc_tokens=64, zipf_s=0.0, groups=(), start_max=0,
        description="1 request: docs at 0 and 64 (4 blocks each), 32 query tokens at 128..159"),
    "decode-32q8kv-b64-ctx4161": Config(
        "decode-32q8kv-b64-ctx4161", Hq=32, Hkv=8, D=128, B=16, rope_base=10000.0,
        n_docs=1000, doc_tokens=512, zipf_s=1.1,
        groups=(Group(64, 8, 65, 1),),
        description="64 requests x (8 Zipf(1.1) docs x 512 + 64 question + 1 decode token)"),
    "prefill-32q8kv-b16-ctx5376": Config(
        "prefill-32q8kv-b16-ctx5376", Hq=32, Hkv=8, D=128, B=16, rope_base=10000.0,
        n_docs=1000, doc_tokens=512, zipf_s=1.1,
        groups=(Group(16, 10, 256, 256, gap_max=63),),
        description="16 requests x (10 Zipf(1.1) docs x 512 with gaps + 256-token suffix prefill)"),
    "decode-32q8kv-b8-ctx32769": Config(
        "decode-32q8kv-b8-ctx32769", Hq=32, Hkv=8, D=128, B=16, rope_base=10000.0,
        n_docs=4000, doc_tokens=512, zipf_s=1.2,
        groups=(Group(8, 64, 1, 1, replace=True),),
        description="8 requests x (64 Zipf(1.2) docs x 512 with replacement + 1 decode token)"),
    "mixed-64q8kv-4p96d": Config(
        "mixed-64q8kv-4p96d", Hq=64, Hkv=8, D=128, B=16, rope_base=10000.0,
        n_docs=2000, doc_tokens=1024, zipf_s=1.1,
        groups=(Group(4, 16, 512, 512), Group(96, 12, 1, 1)),
        description="4 prefill (16 docs x 1024 + 512 suffix) + 96 decode (12 docs x 1024 + 1)"),
}

CONFIG_ORDER = list(CONFIGS)

# Not one of the five named workloads: one long request whose 256-query prefill has too few
# query tiles to fill the GPU, so the prefill key range is split (KV split). Seeded as if it
# were the sixth configuration.
EXTRA_CONFIGS = {
    "prefill-32q8kv-b1-ctx32512": Config(
        "prefill-32q8kv-b1-ctx32512", Hq=32, Hkv=8, D=128, B=16, rope_base=10000.0,
        n_docs=4000, doc_tokens=512, zipf_s=1.2,
        groups=(Group(1, 63, 256, 256, gap_max=63),),
        description="1 request x (63 Zipf(1.2) docs x 512 with gaps + 256-token suffix "
                    "prefill): 32,512 keys"),
}


def _tiny_layouts(decode: bool) -> List[RequestLayout]:
    segs = [Segment("doc", 0, doc=0), Segment("doc", 64, doc=1)]
    if decode:
        segs.append(Segment("private", 128, tokens=33))
        return [RequestLayout(segs, 1)]
    segs.append(Segment("private", 128, tokens=32))
    return [RequestLayout(segs, 32)]


def make(name: str, seed: Optional[int] = None, decode_variant: bool = False,
         no_reuse: bool = False, q_scale: float = 1.0) -> Workload:
    """Build a named configuration. Master seed defaults to 1000 + its 1-based index.
    q_scale multiplies the N(0, 1) queries before rounding (q_scale 4 gives the peaky
    softmax of the stress variants)."""
    cfg = CONFIGS[name] if name in CONFIGS else EXTRA_CONFIGS[name]
    if seed is None:
        seed = 1000 + (CONFIG_ORDER.index(name) + 1 if name in CONFIGS
                       else len(CONFIG_ORDER) + 1 + list(EXTRA_CONFIGS).index(name))
    if name.startswith("tiny-prefill"):
        lays = _tiny_layouts(decode_variant)
    else:
        lays = layouts_for(cfg, seed, no_reuse)
    suffix = ("-decode" if decode_variant else "") + ("-noreuse" if no_reuse else "") + \
        (f"-q{q_scale:g}" if q_scale != 1.0 else "")
    wl = build(cfg.name + suffix, cfg.Hq, cfg.Hkv, cfg.D, cfg.B,
               cfg.rope_base, cfg.n_docs, cfg.doc_tokens, lays, seed, q_scale=q_scale)
    wl.info["description"] = cfg.description
    return wl
