"""GPU test of pa_attention_noalloc (the entry point that allocates nothing: its scratch is a
static device array of the library) through the C ABI: its result equals pa_attention's bitwise
on two calls in a row, the second with a smaller batch, and both match the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
from paged_kv_cache_gqa_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only container
    pytest.skip("no GPU", allow_module_level=True)

import paged_kv_cache_gqa_amd as pa  # noqa: E402

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 2e-3)}


def _check_oracle(w, out, lse):
    ref_o, ref_l = oracle.attention_workload(w)
    eo = np.abs(out.float().cpu().numpy() - ref_o)
    el = np.abs(lse.cpu().numpy() - ref_l)
    mx, mean = TOL[w.dtype]
    msg = f"{w.name}: max|dout|={eo.max():.3e} mean={eo.mean():.3e} max|dlse|={el.max():.3e}"
    print(msg, flush=True)
    assert eo.max() <= mx and el.max() <= mx, msg
    if w.dtype == "bf16":
        assert eo.mean() <= mean and el.mean() <= mean, msg


def _noalloc_abi(t, w, out, lse):
    """pa_attention_noalloc called through ctypes with preallocated outputs (no workspace argument)."""
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    L = pa.lib()
    vp = ctypes.c_void_p
    rc = L.pa_attention_noalloc(ctypes.byref(desc), vp(t["q"].data_ptr()), vp(t["k_pool"].data_ptr()),
                                vp(t["v_pool"].data_ptr()), vp(t["block_table"].data_ptr()),
                                vp(t["seq_lens"].data_ptr()), vp(t["query_start_loc"].data_ptr()),
                                vp(out.data_ptr()), vp(lse.data_ptr()),
                                vp(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, pa.status_str(rc)


@pytest.mark.parametrize("first,second", [(3, 2), (4, 1), ("tile", 3)])
def test_noalloc_equals_attention_on_two_calls(first, second):
    """Two calls in a row on the shared scratch, the second with a smaller batch: each equals
    pa_attention (bitwise) and matches the oracle.  The mixed batch (configuration 3) and the
    llama3-8b decode batch (configuration 2) both have key-split units merged through the scratch;
    the long prefill tile runs 128-row blocks, whose split pieces fill the scratch's largest slots."""
    for c in (first, second):
        w = W.make_long_prefill() if c == "tile" else W.make_config(c)
        t = pa.to_device(w)
        ref_o, ref_l = pa.attention(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    t["query_start_loc"], w.scale)
        out = torch.empty_like(t["q"])
        lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
        _noalloc_abi(t, w, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"configuration {c}"
        _check_oracle(w, out, lse)


def test_noalloc_binding_and_errors():
    w = W.make_random(44, 6, 500, 32, 8, 128, "bf16", max_q=70)
    t = pa.to_device(w)
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    for _ in range(2):
        pa.attention_noalloc(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                             t["query_start_loc"], w.scale, out, lse)
        torch.cuda.synchronize()
        _check_oracle(w, out, lse)
    L = pa.lib()
    assert L.pa_attention_noalloc(None, None, None, None, None, None, None, None, None, None) == 1
    bad = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    bad.head_dim = 96
    assert L.pa_attention_noalloc(ctypes.byref(bad), None, None, None, None, None, None, None, None, None) == 3
