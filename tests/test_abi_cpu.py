"""Host-side checks of the C ABI library (no GPU needed): load, exports, encoder, validation."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from workload import make

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import position_agnostic_kv_paged_amd as pkg
    if not os.path.exists(pkg.LIB_PATH):
        pytest.skip("library not built")
    pkg.lib()
    return pkg


def test_exports_every_declared_symbol(L):
    hdr = open(os.path.join(ROOT, "include", "lazyattn.h")).read()
    declared = sorted(set(re.findall(r"^(?:int|int32_t|size_t|const char\*)\s+(lazyattn_\w+)\(",
                                     hdr, flags=re.M)))
    assert declared == sorted(L.EXPORTED)
    raw = ctypes.CDLL(L.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), name


def test_host_encoder_matches_oracle_bit_exact(L):
    for name in ("decode-32q8kv-b64-ctx4161", "prefill-32q8kv-b16-ctx5376"):
        wl = make(name)
        got = L.encode_meta(wl.flat_block_ids, wl.flat_offsets, wl.block_table)
        want = oracle.encode_meta(wl.flat_block_ids, wl.flat_offsets, wl.block_table, 16)
        assert np.array_equal(got, want)


def test_host_encoder_boundaries_and_errors(L):
    ids = np.array([0, 131071, 7, 1], np.int32)
    offs = np.array([-16384, 16 + 16383, 32, 48 - 1], np.int64)
    bt = np.array([0, 4], np.int32)
    assert np.array_equal(L.encode_meta(ids, offs, bt), oracle.encode_meta(ids, offs, bt, 16))
    from position_agnostic_kv_paged_amd import LazyAttnError
    for bad_ids, bad_offs in (([131072], [0]), ([0], [16384]), ([0], [-16385]), ([-1], [0])):
        with pytest.raises(LazyAttnError) as e:
            L.encode_meta(np.array(bad_ids, np.int32), np.array(bad_offs, np.int64),
                          np.array([0, 1], np.int32))
        assert e.value.code == -4
    # first bad entry is reported
    lib = L.lib()
    words = np.zeros(3, np.uint32)
    bad = ctypes.c_int64(0)
    ids3 = np.array([1, 2, 1 << 17], np.int32)
    offs3 = np.array([0, 16, 32], np.int64)
    bt3 = np.array([0, 3], np.int32)
    rc = lib.lazyattn_encode_meta(ids3.ctypes.data, offs3.ctypes.data, bt3.ctypes.data, 1, 16,
                                  words.ctypes.data, ctypes.byref(bad))
    assert rc == -4 and bad.value == 2 and words[2] == 0 and words[1] == 2


def _call(lib, fn, **over):
    a = dict(q=16, k=16, v=16, bt=16, meta=16, kvl=16, qi=16, qp=16, base=10000.0, S=1, TQ=1,
             Hq=32, Hkv=8, D=128, B=16, NB=10, ME=4, out=16, ws=16, wsb=1 << 30, st=0)
    a.update(over)
    vp = lambda x: ctypes.c_void_p(x) if x else None
    return getattr(lib, fn)(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["bt"]), vp(a["meta"]),
                            vp(a["kvl"]), vp(a["qi"]), vp(a["qp"]), a["base"], a["S"], a["TQ"],
                            a["Hq"], a["Hkv"], a["D"], a["B"], a["NB"], a["ME"], vp(a["out"]),
                            vp(a["ws"]), a["wsb"], vp(a["st"]))


@pytest.mark.parametrize("fn", ["lazyattn_prefill", "lazyattn_decode"])
def test_argument_validation_without_gpu(L, fn):
    lib = L.lib()
    assert _call(lib, fn, q=0) == -1
    assert _call(lib, fn, out=0) == -1
    assert _call(lib, fn, D=96) == -3
    assert _call(lib, fn, B=32) == -3
    assert _call(lib, fn, Hq=12, Hkv=8) == -3
    assert _call(lib, fn, Hq=24, Hkv=1) == -3          # G = 24: not 1, 2, 4, 8 or 16 S
    assert _call(lib, fn, Hq=96, Hkv=2, D=96) == -3    # G = 48 is fine, D = 96 is not
    assert _call(lib, fn, S=-1) == -3
    assert _call(lib, fn, NB=(1 << 17) + 1) == -3
    assert _call(lib, fn, base=1.0) == -7
    assert _call(lib, fn, base=float("nan")) == -7
    assert _call(lib, fn, q=24) == -2
    assert _call(lib, fn, ws=40) == -2
    assert _call(lib, fn, wsb=8) == -5
    # nothing to do: returns OK before any device work
    assert _call(lib, fn, S=0, TQ=0) == 0


@pytest.mark.parametrize("fn", ["lazyattn_prefill_partial", "lazyattn_decode_partial"])
def test_partial_rotary_validation_without_gpu(L, fn):
    """rotary_dim must be a multiple of 16 in [16, D]; errors return before any launch."""
    lib = L.lib()
    f = getattr(lib, fn)
    vp = ctypes.c_void_p

    def call(r, D=128, q=16, base=10000.0):
        return f(vp(q) if q else None, vp(16), vp(16), vp(16), vp(16), vp(16), vp(16), vp(16),
                 base, r, 1, 1, 32, 8, D, 16, 10, 4, vp(16), vp(16), 1 << 30, None)
    for r in (0, 8, 24, 144, -16):
        assert call(r) == -7
    assert call(80, D=64) == -7
    assert call(32, q=0) == -1
    assert call(32, base=0.5) == -7
    assert call(32, D=96) == -3


def test_workspace_sizes(L):
    lib = L.lib()
    assert lib.lazyattn_prefill_workspace_bytes(4, 100, 10, 32, 8, 96) == 0
    a = lib.lazyattn_decode_workspace_bytes(64, 64, 261, 32, 8, 128)
    b = lib.lazyattn_prefill_workspace_bytes(64, 64 * 256, 261, 32, 8, 128)
    assert a > 0 and b > 0
    assert L.lib().lazyattn_status_str(-5) == b"workspace too small"


def test_binding_rejects_mixed_or_malformed_variant_arguments(L):
    """The torch binding checks variant arguments before any library call (CPU tensors)."""
    torch = pytest.importorskip("torch")
    q = torch.zeros((4, 8, 128), dtype=torch.bfloat16)
    pool = torch.zeros((6, 2, 16, 128), dtype=torch.bfloat16)
    i32 = lambda *v: torch.tensor(v, dtype=torch.int32)
    args = (q, pool, pool, i32(0, 2), i32(0, 0), i32(20), i32(0, 4), i32(16, 17, 18, 19),
            10000.0, 2)
    with pytest.raises(ValueError):                     # stored offsets must be int32
        L.prefill(*args, stored_offsets=torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError):                     # one stored offset per entry
        L.prefill(*args, stored_offsets=i32(0))
    with pytest.raises(ValueError):
        L.decode(*args, stored_offsets=i32(0, 16), rotary_dim=32)
    with pytest.raises(ValueError):
        L.prefill(*args, rotary_dim=32, slopes=torch.zeros(8))
    with pytest.raises(ValueError):                     # D/2 frequencies
        L.prefill(*args, inv_freq=np.ones(10))
    with pytest.raises(ValueError):                     # slopes: float32 [Hq]
        L.decode(*args, slopes=torch.zeros(4))
