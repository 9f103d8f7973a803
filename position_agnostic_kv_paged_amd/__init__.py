"""LazyAttention on AMD Instinct MI355X: deferred-RoPE paged attention over a
position-free KV pool (HIP/gfx950 kernels behind a C ABI, include/lazyattn.h)."""
from ._lib import lib, LazyAttnError, EXPORTED, LIB_PATH  # noqa: F401
from .api import (prefill, decode, prefill_rotated_pool, decode_rotated_pool,  # noqa: F401
                  materialize_rotated, encode_meta, debug_decode_meta,
                  workspace_bytes, probe_cus, probe_mfma, probe_read, probe_gather,
                  ingest_kv,
                  PoolIndex, llama31_inv_freq, decode_noalloc, decode_share_plan,
                  decode_shared, prefill_shared, shared_workspace_bytes, BLOCK)
