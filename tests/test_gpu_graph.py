"""HIP graph capture of the attention calls: each call is captured once (torch.cuda.CUDAGraph is a
hipGraph on ROCm) and replayed several times, with eager work and synchronizations between the
replays; every replay must equal the eager call bitwise.  Between replays the inputs are changed in
place, so that a replay that re-ran nothing (or a stale plan) would fail.  The single launch plans
in-kernel and leaves its arrival counters zero, and the library enqueues no hipMemset, so the
captured launches are self-contained."""
import numpy as np
import pytest

from paged_kv_cache_gqa_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only container
    pytest.skip("no GPU", allow_module_level=True)

import paged_kv_cache_gqa_amd as pa  # noqa: E402

REPLAYS = 3


def _replay_and_compare(call, inputs, outs, fresh):
    """call(): enqueue the call on the current stream writing into `outs`; fresh(i): new input
    values (in place) for replay i.  Returns nothing; asserts replay == eager for every replay."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream (first-call set-up stays out of the graph)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        fresh(i)
        torch.cuda.synchronize()
        call()  # eager reference on the same inputs
        torch.cuda.synchronize()
        ref = [o.clone() for o in outs]
        for o in outs:
            o.fill_(float("nan"))  # eager work between the two runs
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {i} differs from the eager call"
        assert all(torch.isfinite(o.float()).all() for o in outs)


def _fresh_q(t, seed):
    gen = torch.Generator(device="cuda")

    def fresh(i):
        gen.manual_seed(seed + i)
        t["q"].copy_(torch.randn(t["q"].shape, generator=gen, device="cuda").to(t["q"].dtype))
    return fresh


@pytest.mark.parametrize("seed", [401, 402])
def test_attention_graph_replays(seed):
    w = W.make_interleaved_mixed(seed, "bf16")
    t = pa.to_device(w)
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    ws = pa.alloc_workspace(desc)
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")

    def call():
        pa.attention(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], t["query_start_loc"],
                     w.scale, out=out, lse=lse, workspace=ws)
    _replay_and_compare(call, t, [out, lse], _fresh_q(t, seed))


def test_noalloc_graph_replays():
    w = W.make_config(3)
    t = pa.to_device(w)
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")

    def call():
        pa.attention_noalloc(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                             t["query_start_loc"], w.scale, out, lse)
    _replay_and_compare(call, t, [out, lse], _fresh_q(t, 403))


def test_fp8_graph_replays():
    w = W.to_fp8(W.make_interleaved_mixed(404, "bf16"))
    t = pa.to_device(w)
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    ws = pa.alloc_workspace(desc)
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")

    def call():
        pa.attention_fp8kv(t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["block_table"],
                           t["seq_lens"], t["query_start_loc"], w.scale, out=out, lse=lse, workspace=ws)
    _replay_and_compare(call, t, [out, lse], _fresh_q(t, 405))


def test_shared_prefix_graph_replays():
    w = W.make_shared_prefix(406, [5, 3, 4], [512, 256, 1024], 300, 2, 32, 8, 128, "bf16")
    t = pa.to_device(w)
    gs = torch.from_numpy(w.meta["group_start"].astype(np.int32)).cuda()
    pl = torch.from_numpy(w.meta["prefix_len"].astype(np.int32)).cuda()
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    ws = pa.shared_prefix_workspace(desc, int(pl.shape[0]))
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")

    def call():
        pa.attention_shared_prefix(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                   t["query_start_loc"], gs, pl, w.scale, out=out, lse=lse, workspace=ws)
    _replay_and_compare(call, t, [out, lse], _fresh_q(t, 407))
