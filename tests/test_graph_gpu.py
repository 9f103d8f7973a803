"""The attention calls captured into a HIP graph (torch.cuda.CUDAGraph on the ROCm build).
With the output and the workspace given, a call only enqueues kernels on the caller's
stream (no allocation, no memset, no host read of device memory), so a serving loop can
capture it once and replay it. Every replay, with eager work on the device between the
replays, must reproduce the eager result bit for bit."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from workload import Segment, RequestLayout, build  # noqa: E402
from tests.gpu_util import words_for, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import position_agnostic_kv_paged_amd as L
    L.lib()


def _mixed_batch():
    """A prefill request, two decode requests (one with a reused document at two offsets)."""
    reqs = [RequestLayout([Segment("doc", 11, doc=0), Segment("doc", 60, doc=1),
                           Segment("private", 100, tokens=70)], 70),
            RequestLayout([Segment("doc", 0, doc=2), Segment("private", 32, tokens=5)], 1),
            RequestLayout([Segment("doc", 500, doc=2), Segment("doc", 5, doc=0),
                           Segment("doc", 700, doc=2), Segment("private", 800, tokens=17)], 1)]
    return build("graph-mixed", 8, 2, 128, 16, 10000.0, 3, 64, reqs, seed=21)


@pytest.mark.parametrize("variant", ["rope", "llama31"])
@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_graph_replays_equal_eager(kind, variant):
    import position_agnostic_kv_paged_amd as L
    wl = _mixed_batch()
    t = wl.to_device("cuda")
    meta = torch.from_numpy(np.ascontiguousarray(words_for(wl)).view(np.int32)).to("cuda")
    max_e = max(len(x) for x in wl.seq_block_ids)
    fn = L.prefill if kind == "prefill" else L.decode
    inv_freq = L.llama31_inv_freq(wl.D) if variant == "llama31" else None
    ws = torch.empty(L.workspace_bytes(kind, wl.num_seqs, t["q"].shape[0], max_e, wl.Hq,
                                       wl.Hkv, wl.D), dtype=torch.uint8, device="cuda")

    def call(out):
        fn(t["q"], t["k_pool"], t["v_pool"], t["block_table"], meta, t["kv_lens"],
           t["q_indptr"], t["q_pos"], wl.rope_base, max_e, out=out, workspace=ws,
           inv_freq=inv_freq)

    say(f"graph capture {kind}/{variant}")
    eager = torch.empty_like(t["q"])
    call(eager)
    torch.cuda.synchronize()
    static = torch.empty_like(t["q"])
    side = torch.cuda.Stream()                       # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(static)                                 # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(static)
    other = torch.empty_like(t["q"])
    for i in range(4):
        static.fill_(float("nan"))                   # eager fill kernel, not part of the graph
        call(other)                                  # eager call between replays (same workspace)
        noise = torch.randn(1 << 18, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(static.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        assert torch.equal(other.view(torch.int16), eager.view(torch.int16))
        del noise


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_graph_replays_equal_eager_shared(kind):
    """The calls over a shared-document plan (plan built on the host before the capture, its
    device copy a captured kernel argument) replay bit for bit too."""
    import position_agnostic_kv_paged_amd as L
    wl = _mixed_batch()
    t = wl.to_device("cuda")
    words = words_for(wl)
    meta = torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to("cuda")
    max_e = max(len(x) for x in wl.seq_block_ids)
    plan = L.decode_share_plan(wl.q_indptr, wl.block_table, words, wl.Hq, wl.Hkv,
                               single_row_only=kind == "prefill", max_chunk=4)
    n_items, n_slots = int(plan[4]), int(plan[5])
    d_plan = torch.from_numpy(plan).cuda()
    ws = torch.empty(max(16, L.shared_workspace_bytes(kind, wl.num_seqs, t["q"].shape[0], max_e,
                                                      n_slots, wl.Hq, wl.Hkv, wl.D)),
                     dtype=torch.uint8, device="cuda")
    fn = L.prefill_shared if kind == "prefill" else L.decode_shared

    def call(out):
        fn(t["q"], t["k_pool"], t["v_pool"], t["block_table"], meta, t["kv_lens"],
           t["q_indptr"], t["q_pos"], wl.rope_base, max_e, d_plan, n_items, n_slots, out=out,
           workspace=ws)

    say(f"graph capture {kind}/shared plan ({n_items} items)")
    eager = torch.empty_like(t["q"])
    call(eager)
    torch.cuda.synchronize()
    static = torch.empty_like(t["q"])
    side = torch.cuda.Stream()                       # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(static)
    other = torch.empty_like(t["q"])
    for i in range(4):
        static.fill_(float("nan"))
        call(other)
        noise = torch.randn(1 << 18, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(static.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        assert torch.equal(other.view(torch.int16), eager.view(torch.int16))
        del noise
