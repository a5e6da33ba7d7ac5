"""GPU parity of tree-structured verify windows (pa_attention_tree) against the oracle's
attention_tree, through the C ABI.  Tolerances as for pa_attention: fp32 1e-5 max-abs; bf16 2e-2
max-abs and 2e-3 mean-abs, for out and lse."""
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


def run_tree(w, masks):
    t = pa.to_device(w)
    tm = torch.from_numpy(np.ascontiguousarray(masks, dtype=np.uint64).view(np.int64)).cuda()
    out, lse = pa.attention_tree(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                 t["query_start_loc"], tm, w.scale)
    torch.cuda.synchronize()
    return out, lse


def check(w, masks, out, lse):
    ref_o, ref_l = oracle.attention_tree(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, w.query_start_loc,
                                         masks, w.scale)
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(l), empty), "rows that see no key"
    assert np.all(o[empty] == 0.0)
    mx, mean = TOL[w.dtype]
    eo, el = np.abs(o - ref_o), np.abs(l[~empty] - ref_l[~empty])
    msg = f"{w.name}: max|dout|={eo.max():.3e} mean={eo.mean():.3e} max|dlse|={el.max():.3e}"
    print(msg, flush=True)
    assert np.isfinite(o).all() and eo.max() <= mx and el.max() <= mx, msg
    if w.dtype == "bf16":
        assert eo.mean() <= mean and el.mean() <= mean, msg


def test_causal_masks_equal_plain_attention_bitwise():
    w = W.make_random(91, 8, 600, 32, 8, 128, "bf16", max_q=40)
    t = pa.to_device(w)
    o1, l1 = pa.attention(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], t["query_start_loc"],
                          w.scale)
    o2, l2 = run_tree(w, W.causal_masks(w.q_lens()))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


CASES = [
    # seed, B, max_len, Hq, Hkv, D, dtype, max_q
    (92, 12, 900, 32, 8, 128, "bf16", 5),    # verify windows: key-split units (q * G <= 32)
    (93, 6, 700, 8, 1, 128, "bf16", 64),     # up to 64-token trees: 64-row units
    (94, 7, 300, 8, 2, 64, "f32", 16),
    (95, 5, 400, 12, 3, 64, "bf16", 100),    # some windows longer than 64: causal there
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}-{c[6]}-D{c[5]}-q{c[7]}" for c in CASES])
def test_random_trees(case):
    seed, B, L, Hq, Hkv, D, dt, mq = case
    w = W.make_random(seed, B, L, Hq, Hkv, D, dt, max_q=mq)
    masks, _ = W.random_trees(w.q_lens(), seed)
    if mq > 64:  # garbage in the masks of long windows must be ignored
        qsl = w.query_start_loc
        for s in range(w.num_seqs):
            if qsl[s + 1] - qsl[s] > 64:
                masks[qsl[s]:qsl[s + 1]] = np.random.default_rng(seed).integers(
                    0, 2**63, size=int(qsl[s + 1] - qsl[s]), dtype=np.int64).astype(np.uint64)
    out, lse = run_tree(w, masks)
    check(w, masks, out, lse)


def test_verify_configuration_with_trees():
    """The whole speculative-verify configuration (32 sequences, 5-token windows over 2k-16k keys) with
    random draft trees over the 4 draft tokens."""
    w = W.make_config(4)
    masks, _ = W.random_trees(w.q_lens(), 4004)
    out, lse = run_tree(w, masks)
    check(w, masks, out, lse)


def test_row_that_sees_nothing():
    w = W.make_random(96, 3, 60, 8, 2, 64, "f32", max_q=3)
    w.seq_lens = w.q_lens().astype(np.int32)  # no context: every key is a window token
    masks = W.causal_masks(w.q_lens())
    masks[0] = 0  # the first row hides even itself
    out, lse = run_tree(w, masks)
    check(w, masks, out, lse)
