"""lazyattn_decode_noalloc: the decode entry point that allocates nothing (its workspace is a
fixed per-device buffer inside the library) against lazyattn_decode, which takes a
caller-allocated workspace, and against the oracle; two calls in a row, the second smaller;
a batch whose default split does not fit the buffer (coarsened split); a batch that cannot
fit at all (error before any launch)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from workload import make, build, Segment, RequestLayout  # noqa: E402
from tests.util import small, oracle_out  # noqa: E402
from tests.gpu_util import compare, say, words_for  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import position_agnostic_kv_paged_amd as L
    L.lib()


def _both(wl):
    """(lazyattn_decode output, lazyattn_decode_noalloc output) as float64 arrays."""
    import position_agnostic_kv_paged_amd as L
    t = wl.to_device("cuda")
    meta = torch.from_numpy(np.ascontiguousarray(words_for(wl)).view(np.int32)).to("cuda")
    me = max(len(x) for x in wl.seq_block_ids)
    args = (t["q"], t["k_pool"], t["v_pool"], t["block_table"], meta, t["kv_lens"],
            t["q_indptr"], t["q_pos"], wl.rope_base, me)
    ref = L.decode(*args)
    out = torch.full_like(t["q"], float("nan"))
    L.decode_noalloc(*args, out=out)
    torch.cuda.synchronize()
    f = lambda x: x.float().cpu().numpy().astype(np.float64)  # noqa: E731
    return f(ref), f(out)


def test_noalloc_two_calls_second_smaller():
    big = make("decode-32q8kv-b64-ctx4161")
    sm = small(Hq=8, Hkv=2, D=128, seed=5, q_len=1)
    for wl in (big, sm):
        say(f"no-alloc decode on {wl.name}: {wl.total_q} rows")
        ref, got = _both(wl)
        assert np.array_equal(got, ref), "no-alloc output differs from lazyattn_decode"
        compare(got, oracle_out(wl), f"noalloc/{wl.name}")


def test_noalloc_coarsened_split():
    """800 decode rows x 64 heads: the default split (two splits per row) needs ~54 MB of
    partials, more than the 32 MiB buffer, so the call takes one split per row; same result
    within tolerance."""
    rng = np.random.default_rng(9)
    reqs = []
    for r in range(800):
        start = int(rng.integers(0, 200))
        reqs.append(RequestLayout([Segment("doc", start, doc=int(rng.integers(0, 50))),
                                   Segment("private", start + 256, tokens=65)], 1))
    wl = build("noalloc-800", 64, 8, 128, 16, 10000.0, 50, 256, reqs, seed=10)
    say("no-alloc decode, 800 rows (coarsened split)")
    ref, got = _both(wl)
    want = oracle_out(wl)
    compare(got, want, "noalloc/800-rows")
    compare(ref, want, "decode/800-rows")


def test_noalloc_rejects_batch_that_cannot_fit():
    """2000 rows x 64 heads need ~68 MB of partials even with one split per row: the call
    returns LAZYATTN_ERR_WORKSPACE before launching anything."""
    import position_agnostic_kv_paged_amd as L
    from position_agnostic_kv_paged_amd._lib import ERR_WORKSPACE, LazyAttnError
    n, Hq, Hkv, D = 2000, 64, 8, 128
    q = torch.zeros((n, Hq, D), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((4, Hkv, 16, D), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    meta = torch.zeros(1, dtype=torch.int32, device="cuda")
    kv = torch.zeros(n, dtype=torch.int32, device="cuda")
    qi = torch.arange(n + 1, dtype=torch.int32, device="cuda")
    qp = torch.zeros(n, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(LazyAttnError) as e:
        L.decode_noalloc(q, pool, pool, bt, meta, kv, qi, qp, 10000.0, 1, out=out)
    assert e.value.code == ERR_WORKSPACE
