"""Float64 CPU oracle for LazyAttention (deferred-RoPE paged attention).

TEST INFRASTRUCTURE ONLY. Nothing in the product library imports, links or runs
this package; only the tests, the smoke check and the benchmark's CPU-baseline
leg do. It is a plain, slow, obviously-correct statement of what the attention
path computes, written from:

  Xia, Pamnani, Fang, Chockchowwat, Park, "LazyAttention: Efficient
  Retrieval-Augmented Generation with Deferred Positional Encoding",
  arXiv 2606.04302 -- the authors' abstract, and the gist.science technical
  summary of it (sections "Core Concept: Deferred Positional Encoding",
  "Technical Implementation", "Mathematical Equivalence").

The summary states that the deferred (lazy) method gives the same scores and
outputs as materialising position-adjusted KV copies, because RoPE attention
depends only on the relative offset n - m. The oracle therefore computes the
plain definition -- it materialises each logical prompt by copying the
un-rotated key blocks, applies RoPE at absolute logical positions (float64),
and runs causal softmax attention in float64 -- rather than the lazy algorithm.

Modules
  rope       RoPE frequencies and rotation R(n) in float64.
  meta       independent encoder/decoder of the packed (block id, offset) word.
  attention  materialise + attend; sampled-row variant for large batches.
  overhead   the rotation-FLOP accounting of the prefill tile (3/(4M)).
  pool       ingest of new keys/values into pool slots; a plain model of the
             document-keyed block index (LRU among unreferenced documents).
  alibi      ALiBi (linear bias on logical distances, no rotation) over the same pool.
  docrot     a pool whose keys carry RoPE at their positions inside their document.

Pins (tests marked "not gpu"): closed-form rotation identities and the complex
(RoFormer) form of RoPE, a brute-force attention with explicit D x D rotation
matrices and an explicit mask matrix, torch's scaled_dot_product_attention on a
dense layout, single-key / equal-key closed forms, the reuse-vs-copy invariant,
translation and permutation invariance, bit patterns of the packed word, and
the summary's printed 0.59% overhead at M = 128. No function here is
"parity unpinned".
"""
from . import rope, meta, attention, overhead, pool, alibi, docrot  # noqa: F401
from .attention import lazy_attention, attention_rows, bf16_bits_to_f64, rotated_pool  # noqa: F401
from .meta import encode_meta, decode_meta  # noqa: F401
