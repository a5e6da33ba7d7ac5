"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Tolerances: float32 inputs 1e-5 max-abs; bf16 inputs
2e-2 max-abs and 2e-3 mean-abs (fp32 accumulation), for both out and lse.
Indexing outputs (gather, plan coverage) are compared bit-exactly."""
import bisect
import math

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


def run_gpu(w, **kw):
    t = pa.to_device(w)
    out, lse = pa.attention(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                            t["query_start_loc"], w.scale, **kw)
    torch.cuda.synchronize()
    return out, lse


def check(w, out, lse, ref=None, rows=None, tol=None):
    ref_o, ref_l = ref if ref is not None else oracle.attention_workload(w)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    if rows is not None:
        o, l = o[rows], l[rows]
    mx, mean = tol if tol is not None else TOL[w.dtype]
    eo, el = np.abs(o - ref_o), np.abs(l - ref_l)
    msg = (f"{w.name}: max|dout|={eo.max() if eo.size else 0:.3e} mean={eo.mean() if eo.size else 0:.3e} "
           f"max|dlse|={el.max() if el.size else 0:.3e} mean={el.mean() if el.size else 0:.3e}")
    print(msg, flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), msg
    if eo.size:
        assert eo.max() <= mx and el.max() <= mx, msg
        if w.dtype == "bf16":
            assert eo.mean() <= mean and el.mean() <= mean, msg


@pytest.mark.parametrize("seed", [301, 305, 310, 317])
def test_interleaved_mixed_batch(seed):
    w = W.make_interleaved_mixed(seed, "bf16")
    out, lse = run_gpu(w)
    check(w, out, lse)


# ---------------------------------------------------------------------------
# small shapes: several tiles, ragged tails, windows, both dtypes and head dims
# ---------------------------------------------------------------------------
SMALL = [
    # seed, B, max_len, Hq, Hkv, D, dtype, max_q
    (1, 5, 100, 8, 2, 64, "f32", 1),
    (2, 7, 300, 8, 2, 128, "bf16", 1),
    (3, 6, 257, 32, 8, 128, "bf16", 5),
    (4, 4, 700, 8, 1, 128, "bf16", 200),
    (5, 9, 90, 4, 4, 64, "bf16", 3),
    (6, 3, 520, 16, 1, 64, "f32", 40),
    (7, 5, 1200, 64, 8, 128, "bf16", 1),
    (8, 4, 400, 64, 1, 128, "bf16", 2),
    (9, 6, 333, 8, 2, 128, "f32", 17),
    (10, 8, 64, 12, 3, 64, "bf16", 64),
    # group sizes that do not divide a 64-row block: row blocks end mid-token
    (11, 5, 600, 28, 4, 128, "bf16", 150),   # G = 7
    (12, 4, 400, 24, 8, 64, "f32", 90),      # G = 3
    (13, 3, 900, 40, 8, 128, "bf16", 300),   # G = 5
    (14, 3, 500, 96, 8, 128, "bf16", 70),    # G = 12
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}-{c[6]}-D{c[5]}-G{c[3] // c[4]}-q{c[7]}" for c in SMALL])
def test_small_random(case):
    seed, B, maxlen, Hq, Hkv, D, dt, maxq = case
    w = W.make_random(seed, B, maxlen, Hq, Hkv, D, dt, max_q=maxq)
    out, lse = run_gpu(w)
    check(w, out, lse)


def test_config1_tiny_decode_f32():
    w = W.make_config(1)
    out, lse = run_gpu(w)
    check(w, out, lse)


@pytest.mark.parametrize("c", [2, 3, 4])
def test_full_config(c):
    w = W.make_config(c)
    out, lse = run_gpu(w)
    check(w, out, lse)


def test_config5_full_batch():
    """Full-size long-context batch (256 sequences, lognormal lengths up to 32768, 1% of keys x4):
    every row of every head against the oracle."""
    w = W.make_config(5)
    out, lse = run_gpu(w)
    check(w, out, lse)


def test_long_prefill_tile_workload():
    """The long chunked prefill that bench.py --op tile times (2 x 2048-token windows on 2048 keys of
    context, 32/8 heads): every row against the oracle."""
    w = W.make_long_prefill()
    out, lse = run_gpu(w)
    check(w, out, lse)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def test_edge_lengths_and_empty_windows():
    # n = 1, n = 16, 17, 31, 32, 33 (page and chunk boundaries), zero-query sequences, a full prefill (q = n)
    n = [1, 16, 17, 31, 32, 33, 48, 5, 64, 97]
    q = [1, 1, 0, 3, 32, 1, 0, 5, 64, 1]
    for dt, D in (("bf16", 128), ("f32", 64), ("bf16", 64)):
        w = W.build(f"edges-{dt}-{D}", 42, n, q, 8, 2, D, dt, num_pages=40)
        out, lse = run_gpu(w)
        check(w, out, lse)


def test_empty_batch():
    w = W.build("empty", 3, [5, 9], [0, 0], 8, 2, 128, "bf16", num_pages=4)
    out, lse = run_gpu(w)
    assert out.shape == (0, 8, 128)


def test_single_long_sequence_max_length():
    w = W.build("long", 5, [32768], [1], 64, 8, 128, "bf16", num_pages=2048)
    out, lse = run_gpu(w)
    check(w, out, lse)


# Batches with T_q * Hq >= 64 x (workgroups) run 128-row row blocks (two row tiles per wave); these
# keep T_q * Hq above 64 x 1024, past the threshold for any grid up to 1024 workgroups.
TALL_CASES = [
    # name, seed, seq_lens, q_lens, Hq, Hkv
    ("g4", 84, [2500, 1700, 2048, 900], [2000, 1200, 2048, 900], 32, 8),
    ("g7", 85, [3000, 2222, 1500], [2900, 1400, 1500], 28, 4),  # 128-row blocks end mid-token
    ("g8-mixed", 86, [6000, 9000] + [700 + 37 * i for i in range(40)] + [1200 + 91 * i for i in range(10)],
     [6000, 3000] + [1] * 40 + [5] * 10, 8, 1),  # with decode rows and verify windows
]


@pytest.mark.parametrize("case", TALL_CASES, ids=[c[0] for c in TALL_CASES])
def test_tall_row_blocks(case):
    name, seed, n, q, hq, hkv = case
    assert sum(q) * hq >= 64 * 1024
    w = W.build(f"tall-{name}", seed, n, q, hq, hkv, 128, "bf16")
    out, lse = run_gpu(w)
    check(w, out, lse)


def test_million_key_sequences_split_over_hundreds_of_grains():
    """2^20 + 3 keys (65537 pages per sequence): a decode row group (one key-split unit of 32769
    chunks) and a 64-row prefill block over almost the same length (one row-split unit).  The grid's
    512 grains cut each unit into ~256 pieces, merged inside the launch (the row-split merge past
    its 8-piece fast path)."""
    n = (1 << 20) + 3
    w = W.build("million", 6, [n, n - 5], [1, 8], 8, 1, 128, "bf16")
    out, lse = run_gpu(w)
    check(w, out, lse)


# ---------------------------------------------------------------------------
# invariants of the GPU result
# ---------------------------------------------------------------------------
def _poison(w):
    import oracle_pins as P
    return P.poison_unused(w)


def _permute(w, seed):
    import oracle_pins as P
    return P.permute_pages(w, seed)


@pytest.mark.parametrize("case", [(21, 6, 300, 32, 8, 128, "bf16", 5), (22, 3, 600, 8, 1, 128, "bf16", 100),
                                  (23, 5, 200, 8, 2, 64, "f32", 3)])
def test_bitwise_invariance_poison_permutation(case):
    seed, B, maxlen, Hq, Hkv, D, dt, maxq = case
    w = W.make_random(seed, B, maxlen, Hq, Hkv, D, dt, max_q=maxq, slack_pages=5)
    o1, l1 = run_gpu(w)
    o2, l2 = run_gpu(_poison(w))
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "NaN in unused slots reached the result"
    o3, l3 = run_gpu(_permute(w, 9))
    assert torch.equal(o1, o3) and torch.equal(l1, l3), "physical page placement changed the result"


def test_deterministic_and_staged_equals_one_shot():
    w = W.make_config(3)
    t = pa.to_device(w)
    o1, l1 = run_gpu(w)
    o2, l2 = run_gpu(w)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    ws = pa.alloc_workspace(desc)
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    pa.plan(desc, t["seq_lens"], t["query_start_loc"], ws)
    pa.attention_planned(desc, t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                         t["query_start_loc"], out, lse, ws)
    pa.merge_planned(desc, t["seq_lens"], t["query_start_loc"], out, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, out) and torch.equal(l1, lse)


def test_repeated_launches_bitwise_equal_under_merge_contention():
    """128 decode units of 1024 chunks on a grid of a few hundred grains: every unit is split, so
    about a hundred merges complete concurrently in each launch, through arrival counters that every
    launch re-zeroes.  Twenty launches back to back (no synchronization between them) must give
    bitwise identical results, and the first must match the oracle."""
    n = [32768 - 37 * i for i in range(16)]
    w = W.build("merge-contention", 87, n, [1] * 16, 64, 8, 128, "bf16")
    t = pa.to_device(w)
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    ws = pa.alloc_workspace(desc)
    outs = []
    for _ in range(20):
        o = torch.empty_like(t["q"])
        l = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
        pa.attention(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], t["query_start_loc"],
                     w.scale, out=o, lse=l, workspace=ws)
        outs.append((o, l))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    check(w, *outs[0])


def test_staged_equals_one_shot_odd_group():
    """Row blocks that end mid-token (G = 7): the in-kernel plan and the staged planner agree bitwise."""
    w = W.make_random(15, 5, 700, 28, 4, 128, "bf16", max_q=200)
    t = pa.to_device(w)
    o1, l1 = run_gpu(w)
    o2, l2 = _staged(w, t)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _staged(w, t, ws=None):
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    ws = pa.alloc_workspace(desc) if ws is None else ws
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    pa.plan(desc, t["seq_lens"], t["query_start_loc"], ws)
    pa.attention_planned(desc, t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                         t["query_start_loc"], out, lse, ws)
    pa.merge_planned(desc, t["seq_lens"], t["query_start_loc"], out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def test_workspace_reused_across_batches():
    """One workspace serves a sequence of different batches, single-launch and staged calls mixed:
    the arrival counters the single launch relies on are left zero by every call."""
    batches = [W.make_random(61, 9, 900, 32, 8, 128, "bf16", max_q=1),
               W.make_random(62, 5, 700, 8, 1, 128, "bf16", max_q=300),
               W.make_random(63, 12, 400, 32, 8, 128, "bf16", max_q=5),
               W.make_config(2)]
    dev = [pa.to_device(w) for w in batches]
    descs = [pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale) for w, t in zip(batches, dev)]
    big = max(range(len(batches)), key=lambda i: pa.workspace_size(descs[i]))
    ws = pa.alloc_workspace(descs[big])
    for rep in range(2):
        for i, (w, t) in enumerate(zip(batches, dev)):
            ref_o, ref_l = _staged(w, t)  # fresh workspace
            if (i + rep) % 2:
                o, l = _staged(w, t, ws)
            else:
                o, l = pa.attention(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    t["query_start_loc"], w.scale, workspace=ws)
                torch.cuda.synchronize()
            assert torch.equal(o, ref_o) and torch.equal(l, ref_l), (rep, i, w.name)


@pytest.mark.parametrize("B", [2500, 600, 257])
def test_many_sequences_single_launch(B):
    """Batches the in-kernel planner covers with several sequences per thread: one pass of 1024
    sequences (600, 257: one more than one per thread) and several passes (2500)."""
    w = W.make_random(64, B, 90, 8, 2, 64, "bf16", max_q=4)
    t = pa.to_device(w)
    o, l = run_gpu(w)
    so, sl = _staged(w, t)
    assert torch.equal(o, so) and torch.equal(l, sl)
    check(w, o, l)


@pytest.mark.parametrize("maxq", [1, 4, 6])
def test_streamed_short_decode_units(maxq):
    """Many short key-split units back to back in each workgroup (bf16, D = 128): units of one
    to seven chunks, so some waves have no chunk of a unit, consecutive units of one sequence and
    of the next, and (max_q = 6) units of one and of two row tiles interleaved."""
    w = W.make_random(65, 300, 200, 32, 8, 128, "bf16", max_q=maxq)
    t = pa.to_device(w)
    o, l = run_gpu(w)
    o2, l2 = run_gpu(w)
    assert torch.equal(o, o2) and torch.equal(l, l2)
    so, sl = _staged(w, t)
    assert torch.equal(o, so) and torch.equal(l, sl)
    check(w, o, l)


# ---------------------------------------------------------------------------
# integer / indexing outputs (bit-exact)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f32", 64)])
def test_gather_kv_bit_exact(dt, D):
    w = W.make_random(31, 4, 200, 8, 2, D, dt, max_q=2)
    t = pa.to_device(w)
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    for s in range(w.num_seqs):
        n = int(w.seq_lens[s])
        for which, pool, key in ((0, t["k_pool"], "k"), (1, t["v_pool"], "v")):
            nk = min(n + 3, w.max_pages_per_seq * 16)
            g = pa.gather_kv(desc, which, pool, t["block_table"], t["seq_lens"], s, nk)
            ref = oracle.gather(w.k_pool if key == "k" else w.v_pool, w.block_table, w.seq_lens, s, key)
            got = g.cpu()
            got = got.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else got.numpy()
            assert got[:, :n].tobytes() == np.ascontiguousarray(ref).tobytes()
            assert not np.any(got[:, n:].view(np.uint8))  # keys past the end are zero bits


def cpu_plan(w, grid):
    """The plan's units re-derived on the CPU from the stated rules (sequence, kv head, row block order;
    key-split units for q_len*G <= 32 rows, else 64-row blocks; a unit costs start + chunks * weight
    (weight 4 for both kinds; start 48 for a key-split unit of more than 16 rows, else 32) and its
    chunk i starts at cost0 + start + i * weight; the cost axis
    is cut into min(g, key-split cost // 4 + row-split cost // 32) equal grains, one per workgroup, where
    g is the grid, halved -- one workgroup per CU -- for a batch without row-split work)."""
    BLOCK, W_ROW = 64, 4
    G = w.num_q_heads // w.num_kv_heads
    units, cost, row_cost = [], 0, 0
    for s in range(w.num_seqs):
        n, qn = int(w.seq_lens[s]), int(w.q_lens()[s])
        if qn == 0:
            continue
        rows = qn * G
        split = rows <= 32
        nb = 1 if split else -(-rows // BLOCK)
        for g in range(w.num_kv_heads):
            for rb in range(nb):
                r0 = 0 if split else rb * BLOCK
                nr = rows if split else min(BLOCK, rows - r0)
                nk = n if split else n - qn + (r0 + nr - 1) // G + 1
                nch = -(-nk // 32)
                wgt = 4 if split else W_ROW
                start = 48 if split and nr > 16 else 32
                units.append(dict(seq=s, kv_head=g, row0=r0, n_rows=nr, n_keys=nk, n_chunks=nch,
                                  kind=0 if split else 1, cost_weight=wgt, cost0=cost))
                cost += start + nch * wgt
                row_cost += 0 if split else start + nch * wgt
    g = grid // 2 if row_cost == 0 and grid % 16 == 0 else grid
    S = max(1, min(g, (cost - row_cost) // 4 + row_cost // (8 * W_ROW)))
    bounds = [k * cost // S for k in range(S + 1)]
    for u in units:
        start = 48 if u["kind"] == 0 and u["n_rows"] > 16 else 32
        owners = [bisect.bisect_right(bounds, u["cost0"] + start + i * u["cost_weight"]) - 1
                  for i in range(u["n_chunks"])]
        assert sorted(set(owners)) == list(range(owners[0], owners[-1] + 1))  # contiguous pieces, no gaps
        u["first_slot"], u["n_pieces"] = owners[0], owners[-1] - owners[0] + 1
    return units, cost, S


@pytest.mark.parametrize("c", [2, 3, 4])
def test_plan_matches_cpu_rederivation(c):
    w = W.make_config(c)
    t = pa.to_device(w)
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    ws = pa.alloc_workspace(desc)
    pa.plan(desc, t["seq_lens"], t["query_start_loc"], ws)
    hdr, units = pa.plan_read(desc, t["seq_lens"], t["query_start_loc"], ws)
    ref, cost, S = cpu_plan(w, hdr["grid"])
    assert hdr["total_cost"] == cost and hdr["n_slots"] == S and hdr["n_units"] == len(ref)
    assert 1 <= S <= hdr["grid"]
    assert units == ref  # bit-exact, field by field
    # every (sequence, kv head, window row) exactly once
    G = w.num_q_heads // w.num_kv_heads
    seen = {(u["seq"], u["kv_head"], r) for u in units for r in range(u["row0"], u["row0"] + u["n_rows"])}
    assert len(seen) == sum(u["n_rows"] for u in units) == int((w.q_lens() * G).sum()) * w.num_kv_heads


def test_validate_reports_bad_content():
    w = W.make_random(41, 5, 100, 8, 2, 64, "bf16", max_q=3)
    t = pa.to_device(w)
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    ws = pa.alloc_workspace(desc)
    assert pa.validate(desc, t["block_table"], t["seq_lens"], t["query_start_loc"], ws) == 0
    bad = t["block_table"].clone()
    bad[1, 0] = w.num_pages
    assert pa.validate(desc, bad, t["seq_lens"], t["query_start_loc"], ws) == 6
    sl = t["seq_lens"].clone()
    sl[2] = 0 if int(w.q_lens()[2]) > 0 else -1
    assert pa.validate(desc, t["block_table"], sl, t["query_start_loc"], ws) == 6


def test_workspace_too_small_is_rejected():
    """A workspace one byte short of pa_workspace_size, or misaligned, is refused on the host before any
    launch; pa_workspace_bytes agrees with pa_workspace_size."""
    import ctypes
    w = W.make_random(42, 5, 400, 32, 8, 128, "bf16", max_q=3)
    t = pa.to_device(w)
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    need = pa.workspace_size(desc)
    assert pa.workspace_bytes(desc) == need > 0
    ws = pa.alloc_workspace(desc)
    L = pa.lib()
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)

    def call(ptr, nbytes):
        return L.pa_attention(ctypes.byref(desc), vp(t["q"].data_ptr()), vp(t["k_pool"].data_ptr()),
                              vp(t["v_pool"].data_ptr()), vp(t["block_table"].data_ptr()), vp(t["seq_lens"].data_ptr()),
                              vp(t["query_start_loc"].data_ptr()), vp(out.data_ptr()), vp(lse.data_ptr()), vp(ptr),
                              nbytes, stream)

    assert call(ws.data_ptr(), need - 1) == 4  # PA_ERR_WORKSPACE_TOO_SMALL
    assert pa.status_str(4).startswith("PA_ERR_WORKSPACE_TOO_SMALL")
    assert call(ws.data_ptr() + 16, need) == 2  # not 256-byte aligned
    assert call(ws.data_ptr(), need) == 0
    torch.cuda.synchronize()
    check(w, out, lse)
    bad = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    bad.head_dim = 96
    assert pa.workspace_bytes(bad) == 0


def test_side_stream_with_binding_allocations():
    """A call on a stream other than torch's current one, with the binding allocating out, lse and the
    workspace: they are allocated and the counters zeroed on that stream, so the launch (with split
    units to merge) sees initialised counters."""
    w = W.make_config(2)
    t = pa.to_device(w)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = []
    for _ in range(3):
        o, l = pa.attention(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                            t["query_start_loc"], w.scale, stream=side)
        outs.append((o, l))
    side.synchronize()
    ref = oracle.attention_workload(w)
    for o, l in outs:
        check(w, o, l, ref=ref)


def test_validate_max_seq_len():
    w = W.make_random(43, 4, 300, 8, 2, 64, "bf16", max_q=2)
    t = pa.to_device(w)
    top = int(w.seq_lens.max())
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale, max_seq_len=top)
    ws = pa.alloc_workspace(desc)
    assert pa.validate(desc, t["block_table"], t["seq_lens"], t["query_start_loc"], ws) == 0
    desc.max_seq_len = top - 1
    assert pa.validate(desc, t["block_table"], t["seq_lens"], t["query_start_loc"], ws) == 6


def test_merge_op_against_oracle_merge():
    rng = np.random.default_rng(5)
    for D in (64, 128):
        P_, rows = 5, 77
        o = rng.standard_normal((P_, rows, D)).astype(np.float32)
        l = (rng.standard_normal((P_, rows)) * 3).astype(np.float32)
        l[1, :10] = -np.inf
        ro, rl = oracle.merge(o.astype(np.float64), l.astype(np.float64))
        go, gl = pa.merge(torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda())
        torch.cuda.synchronize()
        assert np.abs(go.cpu().numpy() - ro).max() <= 1e-5
        assert np.abs(gl.cpu().numpy() - rl).max() <= 1e-5


# ---------------------------------------------------------------------------
# softmax numerics: extreme score gaps, negative scale
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dt,D,maxq", [("bf16", 128, 1), ("bf16", 128, 70), ("f32", 64, 5)])
def test_peaked_rows_select_the_dominant_key(dt, D, maxq):
    """One key per sequence scores ~500 (natural log units) above the rest: every row that can
    see it must return that key's V row; any row-inconsistent running maximum would overflow."""
    w = W.make_random(61, 6, 400, 8, 2, D, dt, max_q=maxq)
    k = W.bf16_bits_to_f32(w.k_pool) if dt == "bf16" else w.k_pool.copy()
    qf = W.bf16_bits_to_f32(w.q) if dt == "bf16" else w.q.copy()
    rng = np.random.default_rng(3)
    peak = []
    for s in range(w.num_seqs):
        n, q0, q1 = int(w.seq_lens[s]), int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
        j = int(rng.integers(0, max(1, n - (q1 - q0) + 1)))  # visible to every row of the window
        pg, slot = int(w.block_table[s, j // 16]), j % 16
        for g in range(w.num_kv_heads):
            heads = slice(g * 4, g * 4 + 4)
            direction = qf[q0:q1, heads].sum(axis=(0, 1)) if q1 > q0 else np.ones(D, np.float32)
            k[pg, g, slot, :] = (np.sign(direction) * 8.0).astype(np.float32)
        peak.append((s, j))
    k_pool = W.f32_to_bf16_bits(k) if dt == "bf16" else k
    import oracle_pins as P
    w2 = P._replace(w, k_pool=k_pool)
    out, lse = run_gpu(w2)
    check(w2, out, lse)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


RISING_CASES = [
    # name, dtype, D, workload builder
    ("decode-bf16", "bf16", 128, lambda: W.make_random(62, 24, 900, 8, 2, 128, "bf16", max_q=1)),
    ("prefill-bf16", "bf16", 128, lambda: W.make_random(63, 5, 1200, 8, 2, 128, "bf16", max_q=400)),
    ("prefill-f32", "f32", 64, lambda: W.make_random(64, 5, 700, 8, 2, 64, "f32", max_q=300)),
    ("tall-bf16", "bf16", 128, lambda: W.build("tall-rising", 65, [6000, 3000, 700, 1500], [6000, 2500, 1, 5],
                                                8, 1, 128, "bf16")),
]


def _rising(w, dt, D, seed):
    """Per (sequence, kv head) a random sign pattern u: key j = u * c_j with c_j = (j mod 256 + 1) / 32
    (exact in bf16), query rows of even heads |q| * u and of odd heads -|q| * u.  Even heads' scores
    then climb by sum|q| per 32 keys (more than 2^8 in base 2 at D = 64 and 128) along each 256-key
    tooth, odd heads' fall."""
    k = W.bf16_bits_to_f32(w.k_pool) if dt == "bf16" else w.k_pool.copy()
    qf = W.bf16_bits_to_f32(w.q) if dt == "bf16" else w.q.copy()
    G = w.num_q_heads // w.num_kv_heads
    rng = np.random.default_rng(seed)
    c = ((np.arange(256) + 1) / 32.0).astype(np.float32)
    for s in range(w.num_seqs):
        n, q0, q1 = int(w.seq_lens[s]), int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
        for g in range(w.num_kv_heads):
            u = np.where(rng.random(D) < 0.5, -1.0, 1.0).astype(np.float32)
            for h in range(g * G, g * G + G):
                qf[q0:q1, h, :] = np.abs(qf[q0:q1, h, :]) * (u if h % 2 == 0 else -u)
            for j in range(n):
                k[int(w.block_table[s, j // 16]), g, j % 16, :] = u * c[j % 256]
    import oracle_pins as P
    if dt == "bf16":
        return P._replace(w, k_pool=W.f32_to_bf16_bits(k), q=W.f32_to_bf16_bits(qf))
    return P._replace(w, k_pool=k, q=qf)


@pytest.mark.parametrize("case", RISING_CASES, ids=[c[0] for c in RISING_CASES])
def test_rising_scores_move_the_maximum_every_chunk(case):
    """Scores that climb by more than 2^8 (base 2) per 32-key chunk for half the heads: each chunk
    moves those rows' running maxima (the rare rescale path, with the chunk's scores re-based against
    the new maximum), while the other heads see falling scores and keep theirs.  Log-sum-exps reach
    ~50-70 natural-log units."""
    name, dt, D, make = case
    w = _rising(make(), dt, D, 7)
    if name.startswith("tall"):
        assert int(w.q_lens().sum()) * w.num_q_heads >= 64 * 1024
    ref_o, ref_l = oracle.attention_workload(w)
    assert ref_l.max() > 40.0  # the scores do climb far past the lazy threshold
    out, lse = run_gpu(w)
    tol = None
    if dt == "f32":
        # fp32 exponents near 100 (base 2) carry an absolute rounding error of a few ulp(100) = a few
        # 7.6e-6 each, i.e. a relative error of ~2e-5 in the weights and up to ~5e-5 on outputs of
        # |v| <= 4.5: above the 1e-5 bound that holds for moderate scores
        tol = (5e-5, 1e-5)
    check(w, out, lse, ref=(ref_o, ref_l), tol=tol)


@pytest.mark.parametrize("scale", [0.0, 1e-39, -3e-40])
def test_zero_scale_gives_uniform_weights(scale):
    """scale = 0: every score is 0, so each row returns the mean of its visible V rows and
    lse = ln(visible keys).  Rows with masked keys in their last chunk (n = 17, ...) must not pick up
    a NaN from a masked key meeting the zero factor.  Subnormal scales (whose base-2 factor fp32
    flushes to zero) give the same to fp32 precision."""
    n = [17, 1, 300, 45, 64]
    q = [1, 1, 40, 3, 64]
    for dt, D in (("bf16", 128), ("f32", 64)):
        import oracle_pins as P
        w = P._replace(W.build(f"scale0-{dt}", 72, n, q, 8, 2, D, dt, num_pages=40), scale=scale)
        out, lse = run_gpu(w)
        check(w, out, lse)
        ql = w.q_lens()
        for s_ in range(w.num_seqs):
            for i in range(int(ql[s_])):
                r = int(w.query_start_loc[s_]) + i
                p = int(w.seq_lens[s_]) - int(ql[s_]) + i
                assert abs(float(lse[r, 0]) - math.log(p + 1)) <= 1e-5


def test_negative_scale():
    w = W.make_random(71, 5, 300, 8, 2, 128, "bf16", max_q=40)
    import oracle_pins as P
    w2 = P._replace(w, scale=-0.07)
    out, lse = run_gpu(w2)
    check(w2, out, lse)
