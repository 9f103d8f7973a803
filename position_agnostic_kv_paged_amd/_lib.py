"""ctypes loader for liblazyattn.so (the HIP/gfx950 library); argument marshalling only."""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblazyattn.so")

OK, ERR_NULL, ERR_ALIGN, ERR_SHAPE, ERR_RANGE, ERR_WORKSPACE, ERR_LAUNCH, ERR_ARG = \
    0, -1, -2, -3, -4, -5, -6, -7
ERR_NOSPACE, ERR_STATE = -8, -9
NOALLOC_SCRATCH_BYTES = 32 << 20   # LAZYATTN_NOALLOC_SCRATCH_BYTES

# every symbol include/lazyattn.h declares
EXPORTED = [
    "lazyattn_prefill", "lazyattn_decode", "lazyattn_prefill_rotated_pool",
    "lazyattn_decode_rotated_pool", "lazyattn_prefill_freqs", "lazyattn_decode_freqs",
    "lazyattn_prefill_alibi", "lazyattn_decode_alibi", "lazyattn_prefill_partial",
    "lazyattn_decode_partial", "lazyattn_prefill_doc_rotated", "lazyattn_decode_doc_rotated",
    "lazyattn_materialize_rotated", "lazyattn_probe_cus",
    "lazyattn_probe_mfma", "lazyattn_probe_read", "lazyattn_probe_gather", "lazyattn_ingest_kv",
    "lazyattn_pool_create",
    "lazyattn_pool_destroy", "lazyattn_pool_acquire", "lazyattn_pool_release",
    "lazyattn_pool_alloc_private", "lazyattn_pool_free_private", "lazyattn_pool_stats",
    "lazyattn_prefill_workspace_bytes",
    "lazyattn_decode_workspace_bytes", "lazyattn_encode_meta", "lazyattn_debug_decode_meta",
    "lazyattn_llama31_inv_freq", "lazyattn_decode_noalloc", "lazyattn_decode_share_plan",
    "lazyattn_decode_shared", "lazyattn_decode_shared_workspace_bytes",
    "lazyattn_prefill_shared", "lazyattn_prefill_shared_workspace_bytes",
    "lazyattn_status_str", "lazyattn_version",
]

_lib = None


class PoolStats(ctypes.Structure):
    """LazyattnPoolStats (include/lazyattn.h)."""
    _fields_ = [("hits", ctypes.c_int64), ("misses", ctypes.c_int64),
                ("evictions", ctypes.c_int64), ("evicted_blocks", ctypes.c_int64),
                ("num_blocks", ctypes.c_int32), ("free_blocks", ctypes.c_int32),
                ("cached_docs", ctypes.c_int32), ("pinned_docs", ctypes.c_int32),
                ("private_blocks", ctypes.c_int32), ("evictable_blocks", ctypes.c_int32)]


class LazyAttnError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {status_str(code)} ({code})")


def lib():
    """Load the library once; fail loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "python position_agnostic_kv_paged_amd/build.py (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, u64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
    attn = [vp, vp, vp, vp, vp, vp, vp, vp, dbl, i32, i32, i32, i32, i32, i32, i32, i32,
            vp, vp, u64, vp]
    for name in ("lazyattn_prefill", "lazyattn_decode", "lazyattn_prefill_rotated_pool",
                 "lazyattn_decode_rotated_pool"):
        f = getattr(L, name)
        f.argtypes, f.restype = attn, ctypes.c_int
    for name in ("lazyattn_prefill_freqs", "lazyattn_decode_freqs", "lazyattn_prefill_alibi",
                 "lazyattn_decode_alibi"):
        f = getattr(L, name)
        f.argtypes, f.restype = attn[:8] + [vp] + attn[9:], ctypes.c_int
    L.lazyattn_decode_noalloc.argtypes = attn[:17] + [vp, vp]
    L.lazyattn_decode_noalloc.restype = ctypes.c_int
    L.lazyattn_decode_shared.argtypes = attn[:17] + [vp, i32, i32] + attn[17:]
    L.lazyattn_decode_shared.restype = ctypes.c_int
    L.lazyattn_decode_shared_workspace_bytes.argtypes = [i32] * 6
    L.lazyattn_decode_shared_workspace_bytes.restype = ctypes.c_size_t
    L.lazyattn_prefill_shared.argtypes = attn[:17] + [vp, i32, i32] + attn[17:]
    L.lazyattn_prefill_shared.restype = ctypes.c_int
    L.lazyattn_prefill_shared_workspace_bytes.argtypes = [i32] * 7
    L.lazyattn_prefill_shared_workspace_bytes.restype = ctypes.c_size_t
    L.lazyattn_decode_share_plan.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp,
                                             ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
    L.lazyattn_decode_share_plan.restype = ctypes.c_int
    for name in ("lazyattn_prefill_workspace_bytes", "lazyattn_decode_workspace_bytes"):
        f = getattr(L, name)
        f.argtypes, f.restype = [i32] * 6, ctypes.c_size_t
    for name in ("lazyattn_prefill_partial", "lazyattn_decode_partial"):
        f = getattr(L, name)
        f.argtypes, f.restype = attn[:9] + [i32] + attn[9:], ctypes.c_int
    for name in ("lazyattn_prefill_doc_rotated", "lazyattn_decode_doc_rotated"):
        f = getattr(L, name)
        f.argtypes, f.restype = attn[:8] + [vp] + attn[8:], ctypes.c_int
    L.lazyattn_materialize_rotated.argtypes = [vp, vp, vp, vp, vp, dbl, i32, i32, i32, i32, i32,
                                               i32, vp, vp, vp, vp]
    L.lazyattn_materialize_rotated.restype = ctypes.c_int
    L.lazyattn_probe_cus.argtypes, L.lazyattn_probe_cus.restype = [], i32
    L.lazyattn_probe_mfma.argtypes, L.lazyattn_probe_mfma.restype = [i32, vp, vp, vp], ctypes.c_int
    L.lazyattn_probe_read.argtypes, L.lazyattn_probe_read.restype = [vp, u64, vp, vp], ctypes.c_int
    L.lazyattn_probe_gather.argtypes = [vp, u64, vp, i32, i32, vp, vp]
    L.lazyattn_probe_gather.restype = ctypes.c_int
    L.lazyattn_ingest_kv.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    L.lazyattn_ingest_kv.restype = ctypes.c_int
    P32 = ctypes.POINTER(ctypes.c_int32)
    for name, args in (("lazyattn_pool_create", [i32, i32, ctypes.POINTER(vp)]),
                       ("lazyattn_pool_destroy", [vp]),
                       ("lazyattn_pool_acquire", [vp, ctypes.c_uint64, i32, P32, i32, P32, P32]),
                       ("lazyattn_pool_release", [vp, ctypes.c_uint64]),
                       ("lazyattn_pool_alloc_private", [vp, i32, P32]),
                       ("lazyattn_pool_free_private", [vp, P32, i32]),
                       ("lazyattn_pool_stats", [vp, ctypes.POINTER(PoolStats)])):
        f = getattr(L, name)
        f.argtypes, f.restype = args, ctypes.c_int
    L.lazyattn_llama31_inv_freq.argtypes = [i32, dbl, dbl, dbl, dbl, dbl, vp]
    L.lazyattn_llama31_inv_freq.restype = ctypes.c_int
    L.lazyattn_encode_meta.argtypes = [vp, vp, vp, i32, i32, vp, vp]
    L.lazyattn_encode_meta.restype = ctypes.c_int
    L.lazyattn_debug_decode_meta.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    L.lazyattn_debug_decode_meta.restype = ctypes.c_int
    L.lazyattn_status_str.argtypes, L.lazyattn_status_str.restype = [ctypes.c_int], ctypes.c_char_p
    L.lazyattn_version.argtypes, L.lazyattn_version.restype = [], ctypes.c_char_p
    _lib = L
    return L


def status_str(code: int) -> str:
    return lib().lazyattn_status_str(int(code)).decode()


def check(code: int, where: str):
    if code != OK:
        raise LazyAttnError(code, where)
