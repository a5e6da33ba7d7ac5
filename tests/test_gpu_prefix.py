"""GPU parity of shared-prefix attention (pa_attention_shared_prefix) against the oracle.  The
cascade (prefix pass over each group's shared pages, suffix pass per sequence, log-sum-exp merge)
is an exact rearrangement, so the oracle is plain attention on the same batch.  Tolerances as for
pa_attention: fp32 1e-5 max-abs; bf16 2e-2 max-abs and 2e-3 mean-abs, for out and lse."""
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


def run_prefix(w):
    t = pa.to_device(w)
    gs = torch.from_numpy(w.meta["group_start"].astype(np.int32)).cuda()
    pl = torch.from_numpy(w.meta["prefix_len"].astype(np.int32)).cuda()
    out, lse = pa.attention_shared_prefix(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                          t["query_start_loc"], gs, pl, w.scale)
    torch.cuda.synchronize()
    return out, lse


def check(w, out, lse, ref=None):
    ref_o, ref_l = ref if ref is not None else oracle.attention_workload(w)
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    eo, el = np.abs(o - ref_o), np.abs(l - ref_l)
    mx, mean = TOL[w.dtype]
    msg = f"{w.name}: max|dout|={eo.max():.3e} mean={eo.mean():.3e} max|dlse|={el.max():.3e}"
    print(msg, flush=True)
    assert np.isfinite(o).all() and np.isfinite(l).all(), msg
    assert eo.max() <= mx and el.max() <= mx, msg
    if w.dtype == "bf16":
        assert eo.mean() <= mean and el.mean() <= mean, msg


CASES = [
    # seed, group sizes, prefix lens, suffix max, max q, Hq, Hkv, D, dtype
    (121, [3, 1, 4, 2], [64, 0, 128, 16], 200, 5, 8, 2, 64, "f32"),
    (122, [5, 3], [512, 256], 300, 1, 32, 8, 128, "bf16"),      # decode groups: key-split prefix units
    (123, [2, 3], [512, 1024], 400, 300, 8, 1, 128, "bf16"),    # prefill windows: 64-row units in both passes
    (124, [16], [2048], 500, 4, 32, 8, 128, "bf16"),            # one big group, verify-sized windows
    (126, [6, 6], [1024, 512], 1500, 1500, 8, 1, 128, "bf16"),  # long windows: 128-row blocks in both passes
    (125, [1, 1, 1, 1], [0, 0, 0, 0], 300, 6, 12, 3, 64, "bf16"),  # no sharing at all
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}-{c[8]}-D{c[7]}-g{len(c[1])}" for c in CASES])
def test_shared_prefix_random(case):
    seed, sizes, plens, smax, mq, Hq, Hkv, D, dt = case
    w = W.make_shared_prefix(seed, sizes, plens, smax, mq, Hq, Hkv, D, dt)
    out, lse = run_prefix(w)
    check(w, out, lse)


def test_shared_prefix_system_prompt_configuration():
    """8 groups of 16 decode sequences over a shared 4096-token prefix: every sequence against the
    oracle (max and mean bounds), and against plain pa_attention on the same batch."""
    w = W.make_shared_prefix_config()
    out, lse = run_prefix(w)
    check(w, out, lse)
    t = pa.to_device(w)
    po, pl = pa.attention(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], t["query_start_loc"],
                          w.scale)
    torch.cuda.synchronize()
    assert (out.float() - po.float()).abs().max().item() <= 2e-2
    assert (lse - pl).abs().max().item() <= 2e-2


def test_shared_prefix_rejects_bad_group_counts():
    w = W.make_shared_prefix(126, [2, 2], [32, 32], 100, 2, 8, 2, 64, "bf16")
    t = pa.to_device(w)
    gs = torch.tensor([0, 2, 4, 4], dtype=torch.int32, device="cuda")
    pl = torch.tensor([32, 32, 0], dtype=torch.int32, device="cuda")
    with pytest.raises(pa.PagedAttentionError):  # 5 groups for 4 sequences
        pa.attention_shared_prefix(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                   t["query_start_loc"], torch.zeros(6, dtype=torch.int32, device="cuda"),
                                   torch.zeros(5, dtype=torch.int32, device="cuda"), w.scale)
    out, lse = pa.attention_shared_prefix(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                          t["query_start_loc"], gs, pl, w.scale)  # an empty third group
    torch.cuda.synchronize()
    check(w, out, lse)
