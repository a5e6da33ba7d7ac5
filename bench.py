"""Benchmark of paged-KV GQA attention on one MI355X.

A step is one full pass of the path over one batch: one pa_attention call, a
single persistent kernel launch that plans its own grain, computes it and merges
the key-split rows it completes (with --staged: pa_plan + pa_attention_planned +
pa_merge_planned, the same result in three launches).
Inputs are resident in HBM before the timed region.  The K/V pools are held in
several copies and step i reads copy i % n_copies, so that every step's K/V
were last touched more than 1 GiB of traffic earlier (the 256 MB MALL cannot
serve them); no flush kernel runs inside the timed region.

Default workload: the largest configuration, long-context reasoning decode
(256 sequences, one query token each, context lognormal with median 8192 clipped
to [1024, 32768], 64 query / 8 KV heads, head dim 128, bf16, 16-slot pages, 1%
of keys scaled by 4); its 13 GB of K/V pools fit one GPU's HBM.  --config 1-4
select the other workloads.
`value` is algorithmic bytes (every valid K/V row once per KV head, Q, out,
LSE, block-table entries) divided by the wall time per step over K steps issued
back to back.  The roofline's kernel duration is the span of two HIP events on
the launch stream bracketing those K launches, divided by K.  A second pass over
the same K steps records events around each launch for the spread (and for the
staged path's attention kernel); its event packets add a few microseconds per
launch, so it gives neither `value` nor the single launch's mean.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6  # dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
FP32_PEAK_TFLOPS = 157.3
METRIC = "decode KV-read HBM GB/s (% of peak) + prefill/verify TFLOP/s, 1 MI355X"
KERNEL_SOURCES = ["paged_kv_cache_gqa_amd/csrc/pa_kernels.hip", "paged_kv_cache_gqa_amd/csrc/pa_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_kernel_hbm_traffic.json")

TILE_DESCRIPTION = dict(batch=2, q_heads=32, kv_heads=8, head_dim=128, context="2048 prior + 2048 new",
                        queries_per_seq="2048")
DESCRIPTIONS = {
    1: dict(batch=4, q_heads=8, kv_heads=2, head_dim=64, context="{17,64,100,256}", queries_per_seq="1"),
    2: dict(batch=64, q_heads=32, kv_heads=8, head_dim=128, context="uniform[512,4096]", queries_per_seq="1"),
    3: dict(batch=132, q_heads=8, kv_heads=1, head_dim=128,
            context="4 x (prior uniform[0,2048] + 512 new) + 128 x uniform[1024,8192]",
            queries_per_seq="512 (4 prefill chunks) / 1 (128 decodes)"),
    4: dict(batch=32, q_heads=32, kv_heads=8, head_dim=128, context="prior uniform[2048,16384] + 5",
            queries_per_seq="5"),
    5: dict(batch=256, q_heads=64, kv_heads=8, head_dim=128, context="lognormal(median 8192, sigma 1) in [1024,32768]",
            queries_per_seq="1"),
}


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the attention kernel from the committed counter runs,
    or None when the counters were taken on other kernel sources, another kernel or another workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload)
    if not entry or entry.get("kernel_sha") != kernel_hash() or entry.get("kernel") != kernel:
        return None
    return entry.get("hbm_bytes_per_launch")


CALIBRATION_BYTES = 512 << 20  # the plain device copy that --copy-calibration runs, CALIBRATION_COPIES times
CALIBRATION_COPIES = 3


def record_traffic(workload: str, fetch_csv: str, write_csv: str, kernel: str) -> dict:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of a
    `--copy-calibration` bench run into HBM bytes per attention launch and store them in the traffic
    record under `workload`.  Each counter is scaled by (known copy bytes) / (what it reads for the
    calibration copy: the copy dispatches that moved 512 MiB)."""
    import csv

    def per_dispatch(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        target_rows = [r for r in rows if f"pa::{kernel}<" in r["Kernel_Name"]]
        target = [float(r["Counter_Value"]) for r in target_rows]
        last = max(int(r["Dispatch_Id"]) for r in target_rows)
        # the calibration copies: the largest copies dispatched after the last attention launch
        after = sorted(float(r["Counter_Value"]) for r in rows
                       if "copyBuffer" in r["Kernel_Name"] and int(r["Dispatch_Id"]) > last)
        calib_runs = after[-CALIBRATION_COPIES:]
        factor = CALIBRATION_BYTES / 1024 / statistics.fmean(calib_runs)
        return statistics.fmean(target) * 1024 * factor, factor, len(target)

    fetch, f_fac, n_f = per_dispatch(fetch_csv, "FETCH_SIZE")
    write, w_fac, n_w = per_dispatch(write_csv, "WRITE_SIZE")
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec.setdefault("workloads", {})[workload] = {
        "kernel": kernel, "kernel_sha": kernel_hash(), "hbm_bytes_per_launch": round(fetch + write),
        "fetch_bytes": round(fetch), "write_bytes": round(write),
        "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4), "dispatches": [n_f, n_w]}
    rec["method"] = ("rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE, separate runs, mean KiB per dispatch of "
                     "the attention kernel, each scaled by 512 MiB / (the counter's reading for a 512 MiB "
                     "device copy in the same run)")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    return rec["workloads"][workload]


def cpu_baseline(w, alg_bytes: int, min_seconds: float = 10.0, min_runs: int = 3, max_runs: int = 1000):
    """The oracle (plain fp64 C, OpenMP) on the host cores: the whole batch, repeated until at least
    `min_seconds` of CPU work (and `min_runs` runs) are timed."""
    import oracle
    oracle.attention_workload(w)  # warm (and build) once, untimed
    times = []
    t_start = time.perf_counter()
    while len(times) < max_runs and (len(times) < min_runs or time.perf_counter() - t_start < min_seconds):
        t0 = time.perf_counter()
        oracle.attention_workload(w)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": round(alg_bytes / t / 1e9, 4), "unit": "GB/s", "cores": oracle.max_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"the whole batch (all sequences, all heads) run {len(times)} times "
                      f"({sum(times):.1f} s in all), median {t:.3f} s per batch; fp64 two-pass softmax"}


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def bench_append(args, w) -> int:
    """Time pa_append_kv: the K/V rows of every new token of the batch written into their pages.
    Algorithmic bytes: the new rows read and written once (K and V), plus one block-table entry
    per touched page."""
    import numpy as np
    import torch

    import paged_kv_cache_gqa_amd as pa
    from paged_kv_cache_gqa_amd import binding as B
    import ctypes

    t = pa.to_device(w)
    T, Hkv, D = w.num_q_tokens, w.num_kv_heads, w.head_dim
    g = torch.Generator(device="cuda").manual_seed(1000 + args.config)
    dt = t["k_pool"].dtype
    k_new = torch.randn((T, Hkv, D), generator=g, device="cuda").to(dt)
    v_new = torch.randn((T, Hkv, D), generator=g, device="cuda").to(dt)
    ql = w.q_lens()
    first = (w.seq_lens - ql) // 16
    last = (w.seq_lens - 1) // 16
    pages = int(np.sum(np.where(ql > 0, last - first + 1, 0)))
    alg_bytes = 2 * 2 * T * Hkv * D * k_new.element_size() + 4 * pages
    stream = torch.cuda.current_stream()
    desc = B.PaDesc(num_seqs=w.num_seqs, num_q_tokens=T, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D,
                    page_size=16, num_pages=w.num_pages, max_pages_per_seq=w.max_pages_per_seq, max_seq_len=0,
                    dtype=B._DTYPES[dt], scale=1.0)
    vp = ctypes.c_void_p
    cargs = (ctypes.byref(desc), vp(k_new.data_ptr()), vp(v_new.data_ptr()), vp(t["block_table"].data_ptr()),
             vp(t["seq_lens"].data_ptr()), vp(t["query_start_loc"].data_ptr()), vp(t["k_pool"].data_ptr()),
             vp(t["v_pool"].data_ptr()), vp(stream.cuda_stream))
    L = B.lib()
    for _ in range(args.warmup):
        L.pa_append_kv(*cargs)
    torch.cuda.synchronize()
    # timed region: K launches back to back, bracketed by two HIP events on the launch stream
    bracket = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t0 = time.perf_counter()
    bracket[0].record(stream)
    for _ in range(args.steps):
        if L.pa_append_kv(*cargs):
            raise RuntimeError("append launch failed")
    bracket[1].record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    kmean = bracket[0].elapsed_time(bracket[1]) / args.steps
    # spread: a second pass with HIP events around each launch (their packets lengthen each launch)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in events:
        a.record(stream)
        rc = L.pa_append_kv(*cargs)
        b.record(stream)
        if rc:
            raise RuntimeError(f"launch failed: {B.status_string(rc)}")
    torch.cuda.synchronize()
    ks = [a.elapsed_time(b) for a, b in events]
    name = w.name
    line = {
        "metric": "paged KV append GB/s (new K/V rows read + written, block-table entries), 1 MI355X",
        "value": round(alg_bytes / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded; shapes of the named configuration)",
        "config": {"workload": f"{name} (configuration {args.config}) new tokens", "new_tokens": T, "kv_heads": Hkv,
                   "head_dim": D, "pages_touched": pages, "algorithmic_bytes": alg_bytes},
        "roofline": {"bound": "hbm", "achieved": round(alg_bytes / (kmean * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(alg_bytes / (kmean * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
                     "traffic": None, "kernel": "pa::append_kv_kernel", "kernel_ms_mean": round(kmean, 5),
                     "kernel_ms_source": "two events bracketing the timed region, divided by the steps",
                     "kernel_ms_p10_p90_events_each": [round(float(np.percentile(ks, 10)), 5),
                                                       round(float(np.percentile(ks, 90)), 5)]},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_prefix(args) -> int:
    """Shared-prefix attention on the system-prompt decode batch: the cascade (prefix pass, suffix
    pass, merge) against plain pa_attention on the same batch.  value = distinct K/V bytes (the
    shared prefix once per group) plus Q, out, LSE and block-table entries, over the step time."""
    import ctypes

    import numpy as np
    import torch

    import paged_kv_cache_gqa_amd as pa
    from paged_kv_cache_gqa_amd import binding as B
    from paged_kv_cache_gqa_amd import workloads as W

    w = W.make_shared_prefix_config()
    t = pa.to_device(w)
    gs = torch.from_numpy(w.meta["group_start"].astype(np.int32)).cuda()
    pl = torch.from_numpy(w.meta["prefix_len"].astype(np.int32)).cuda()
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    ws = pa.shared_prefix_workspace(desc, int(pl.shape[0]))
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    vp = ctypes.c_void_p
    L = B.lib()
    dref = ctypes.byref(desc)
    base = (dref, vp(t["q"].data_ptr()), vp(t["k_pool"].data_ptr()), vp(t["v_pool"].data_ptr()),
            vp(t["block_table"].data_ptr()), vp(t["seq_lens"].data_ptr()), vp(t["query_start_loc"].data_ptr()))
    tail = (vp(out.data_ptr()), vp(lse.data_ptr()), vp(ws.data_ptr()), ws.numel(), vp(stream.cuda_stream))
    calls = {"shared_prefix": lambda: L.pa_attention_shared_prefix(*base, int(pl.shape[0]), vp(gs.data_ptr()),
                                                                    vp(pl.data_ptr()), *tail),
             "plain": lambda: L.pa_attention(*base, *tail)}
    ms = {}
    for name, fn in calls.items():
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            if fn():
                raise RuntimeError(f"{name} launch failed")
        torch.cuda.synchronize()
        ms[name] = (time.perf_counter() - t0) * 1e3 / args.steps
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    uniq = W.shared_prefix_unique_bytes(w)
    line = {
        "metric": "shared-prefix attention GB/s (distinct K/V pages read once) , 1 MI355X",
        "value": round(uniq / (ms["shared_prefix"] * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms["shared_prefix"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": {"workload": f"{w.name}: 8 groups x 16 decode sequences, 4096-token shared prefix, suffix "
                               "256..1024, 32/8 heads, head dim 128", "distinct_bytes": uniq,
                   "plain_algorithmic_bytes": w.algorithmic_bytes()},
        "plain_attention_ms_per_step": round(ms["plain"], 5),
        "speedup_vs_plain": round(ms["plain"] / ms["shared_prefix"], 3),
        "frac_of_hbm_peak": round(uniq / (ms["shared_prefix"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_read(args) -> int:
    """The device's plain streaming-read rate (pa_read_stream over an 8 GiB buffer, or --read-bytes):
    the practical ceiling that the memory-bound attention paths are measured against, beside the
    8 TB/s peak; at a configuration's byte count, what a plain read of that many bytes takes."""
    import torch

    import paged_kv_cache_gqa_amd as pa

    quantum = 16 * 4096  # pa_read_stream reads a multiple of 16 bytes per workgroup
    nbytes = -(-args.read_bytes // quantum) * quantum
    # below 2 GiB, passes rotate over several buffers (2 GiB in all), so that no pass is served from
    # the previous one's lines in the 256 MB memory-attached last-level cache
    n_buf = max(1, -(-(2 << 30) // nbytes))
    g = torch.Generator(device="cuda").manual_seed(1008)
    bufs = [torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=g)
            for _ in range(n_buf)]
    stream = torch.cuda.current_stream()
    rates = {}
    for grid in (256, 512, 1024, 2048, 4096):
        sink = torch.empty((grid,), dtype=torch.int32, device="cuda")
        for i in range(max(n_buf, args.warmup // 4)):
            pa.read_stream(bufs[i % n_buf], grid, sink)
        torch.cuda.synchronize()
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        ev[0].record(stream)
        for i in range(args.steps):
            pa.read_stream(bufs[i % n_buf], grid, sink)
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        rates[grid] = (nbytes / (ms * 1e-3) / 1e9, ms)
    best = max(rates, key=lambda k: rates[k][0])
    gbs, ms = rates[best]
    line = {
        "metric": "plain streaming read GB/s (% of HBM peak), 1 MI355X",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u32", "data": "synthetic (seeded random words)",
        "config": {"workload": f"one pass over a {nbytes}-byte device buffer ({n_buf} rotated), 16-byte loads, "
                               "one contiguous slice per workgroup of 256 threads", "bytes": nbytes, "grid": best},
        "by_grid_gbs": {str(k): round(v[0], 1) for k, v in rates.items()},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 5), "traffic": None, "kernel": "pa::read_stream_kernel",
                     "kernel_ms_mean": round(ms, 5),
                     "kernel_ms_source": "two events bracketing the timed launches, divided by the steps"},
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--read-bytes", type=int, default=8 << 30,
                    help="--op read only: bytes per pass (rounded up to 64 KiB; default 8 GiB)")
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="workload (default 5: long-context decode, the largest that runs on one GPU)")
    ap.add_argument("--part", default="all", choices=["all", "prefill", "decode"],
                    help="configuration 3 only: time its prefill chunks or its decode rows alone")
    ap.add_argument("--op", default="attention", choices=["attention", "append", "tree", "fp8", "prefix", "tile", "tile-fp8", "read"],
                    help="attention (default): the attention call; append: the paged KV append of the batch's new "
                         "tokens (pa_append_kv); tree: attention with each window a random draft-token tree "
                         "(pa_attention_tree); fp8: attention over the batch's K/V quantized to FP8 E4M3 pages with "
                         "per-(page, kv head) scales (pa_attention_fp8kv); prefix: shared-prefix attention "
                         "(pa_attention_shared_prefix) on the system-prompt decode batch (8 groups x 16 sequences, "
                         "4096-token shared prefix), --config ignored; tile: pa_attention on a long chunked prefill "
                         "(2 x 2048-token windows on 2048 tokens of context, 32/8 heads, head dim 128), the prefill "
                         "tile's steady state, reported as MFMA TFLOP/s, --config ignored; tile-fp8: the same tile over FP8 "
                         "E4M3 pages (pa_attention_fp8kv); read: the device's plain "
                         "streaming-read rate (pa_read_stream over 8 GiB), the practical ceiling for the decode "
                         "paths, --config ignored")
    ap.add_argument("--staged", action="store_true",
                    help="time pa_plan + pa_attention_planned + pa_merge_planned instead of the single launch")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for HBM counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store the HBM bytes per launch from two rocprofv3 counter CSVs of this workload "
                         "and exit (no GPU use)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "the attention call shards by KV head with no exchange, so N GPUs run N independent copies.",
              file=sys.stderr)
        return 2

    if args.record_traffic:
        from paged_kv_cache_gqa_amd import workloads as W
        name = W.LONG_PREFILL_NAME + ("-fp8kv" if args.op == "tile-fp8" else "") if args.op.startswith("tile") else \
            W.CONFIG_NAMES[args.config] + ("" if args.part == "all" else f"-{args.part}-part") + \
            {"tree": "-tree", "fp8": "-fp8kv"}.get(args.op, "")
        kernel = "attention_kernel" if args.staged else "attention_fused_kernel"
        print(json.dumps(record_traffic(name, *args.record_traffic, kernel=kernel)))
        return 0

    import numpy as np
    import torch

    import paged_kv_cache_gqa_amd as pa
    from paged_kv_cache_gqa_amd import binding as B
    from paged_kv_cache_gqa_amd import workloads as W

    torch.cuda.set_device(0)
    if args.op == "prefix":
        return bench_prefix(args)
    if args.op == "read":
        return bench_read(args)
    tile = args.op in ("tile", "tile-fp8")
    w = W.make_long_prefill() if tile else W.make_config(args.config)
    if args.part != "all" and not tile:
        ql = w.q_lens()
        keep = np.nonzero(ql > 1 if args.part == "prefill" else ql == 1)[0]
        w = W.subset(w, keep)
        w.name = f"{W.CONFIG_NAMES[args.config]}-{args.part}-part"
    if args.op == "append":
        return bench_append(args, w)
    if args.op in ("fp8", "tile-fp8"):
        w = W.to_fp8(w)
    alg_bytes = w.algorithmic_bytes()
    alg_flops = w.algorithmic_flops()
    t = pa.to_device(w)
    kv_bytes = t["k_pool"].numel() * t["k_pool"].element_size() * 2
    n_copies = max(1, min(8, int(np.ceil(3 * 256e6 / kv_bytes)) + 1)) if kv_bytes < 2e9 else 1
    pools = [(t["k_pool"], t["v_pool"])] + [(t["k_pool"].clone(), t["v_pool"].clone()) for _ in range(n_copies - 1)]
    desc = pa.make_desc(t["q"], t["k_pool"], t["block_table"], t["seq_lens"], w.scale)
    ws = pa.alloc_workspace(desc)
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    # pre-marshalled arguments
    L = B.lib()
    import ctypes
    dref = ctypes.byref(desc)
    vp = ctypes.c_void_p
    sp = vp(stream.cuda_stream)
    wsn = ws.numel()
    plan_args = (dref, vp(t["seq_lens"].data_ptr()), vp(t["query_start_loc"].data_ptr()), vp(ws.data_ptr()), wsn, sp)
    tree = args.op == "tree"
    if tree:
        masks, _ = W.random_trees(w.q_lens(), 1000 + args.config)
        tm = torch.from_numpy(masks.view(np.int64)).cuda()
    fp8 = args.op in ("fp8", "tile-fp8")
    mask_arg = (vp(tm.data_ptr()),) if tree else ()
    scale_args = (vp(t["k_scale"].data_ptr()), vp(t["v_scale"].data_ptr())) if fp8 else ()
    attn_args = [(dref, vp(t["q"].data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()), *scale_args,
                  vp(t["block_table"].data_ptr()), vp(t["seq_lens"].data_ptr()), vp(t["query_start_loc"].data_ptr()),
                  *mask_arg, vp(out.data_ptr()), vp(lse.data_ptr()), vp(ws.data_ptr()), wsn, sp) for k, v in pools]
    attention_call = L.pa_attention_tree if tree else L.pa_attention_fp8kv if fp8 else L.pa_attention
    merge_args = (dref, vp(t["seq_lens"].data_ptr()), vp(t["query_start_loc"].data_ptr()), vp(out.data_ptr()),
                  vp(lse.data_ptr()), vp(ws.data_ptr()), wsn, sp)

    def step(i, ev=None):
        if args.staged:
            rc = L.pa_plan(*plan_args)
            if ev is not None:
                ev[0].record(stream)
            rc |= L.pa_attention_planned(*attn_args[i % n_copies])
            if ev is not None:
                ev[1].record(stream)
            rc |= L.pa_merge_planned(*merge_args)
        else:
            if ev is not None:
                ev[0].record(stream)
            rc = attention_call(*attn_args[i % n_copies])
            if ev is not None:
                ev[1].record(stream)
        if rc:
            raise RuntimeError(f"launch failed: {B.status_string(rc)}")

    print(f"[bench] {w.name}: B={w.num_seqs} T_q={w.num_q_tokens} pages={w.num_pages} copies={n_copies} "
          f"alg_bytes={alg_bytes / 1e6:.1f} MB alg_flops={alg_flops / 1e9:.2f} GF", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps back to back, as a caller issues them, bracketed by two HIP events on
    # the launch stream.  With one launch per step, the events' span over K is the kernel's average
    # launch duration (including the gap to the next launch, ~1 us).
    bracket = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bracket[0].record(stream)
    for i in range(args.steps):
        step(i)
    bracket[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    bracket_ms = bracket[0].elapsed_time(bracket[1]) / args.steps
    # Spread of single launches: the same K steps again with HIP events around each attention launch
    # (the staged path's attention kernel is timed this way too).  The event packets add a few
    # microseconds per launch, so this pass gives neither `value` nor, for one launch per step, the mean.
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    te0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    ms_per_step_events = (time.perf_counter() - te0) * 1e3 / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in events]
    attn_mean = statistics.fmean(attn_ms) if args.staged else bracket_ms

    if args.copy_calibration:  # a plain copy of known size, for scaling the HBM counters
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(CALIBRATION_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()

    # correctness spot check of the timed result (outputs are the same for every pool copy)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()

    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (attn_mean * 1e-3) / 1e9
    tflops = alg_flops / (ms_per_step * 1e-3) / 1e12
    compute_dtype = "bf16" if w.dtype in ("bf16", "fp8") else w.dtype  # FP8 pages run through bf16 MFMAs
    peak_tf = BF16_PEAK_TFLOPS if compute_dtype == "bf16" else FP32_PEAK_TFLOPS
    kernel = "attention_kernel" if args.staged else "attention_fused_kernel"
    if (tree or fp8) and args.staged:
        raise SystemExit("--op tree / fp8 run the single launch only")
    desc_cfg = TILE_DESCRIPTION if tile else DESCRIPTIONS[args.config]
    config = {"workload": w.name if tile else f"{w.name} (configuration {args.config})", **desc_cfg,
              "part": args.part, "path": "staged (3 launches)" if args.staged else "single launch",
              "windows": "random draft-token trees (per-row ancestor masks)" if tree else "causal",
              "kv_pages": "FP8 E4M3, per-(page, kv head) fp32 scales" if fp8 else w.dtype,
              "page_size": 16, "seed": 1007 if tile else 1000 + args.config, "kv_pool_copies": n_copies,
              "algorithmic_bytes": alg_bytes, "algorithmic_flops": alg_flops}
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": compute_dtype, "data": "synthetic (seeded; shapes of the named configuration)",
        "config": config,
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "tflops": round(tflops, 3), "frac_of_mfma_peak": round(tflops / peak_tf, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w.name + ("-tree" if tree else ""), kernel),
                     "kernel": f"pa::{kernel}", "kernel_ms_mean": round(attn_mean, 5),
                     "kernel_ms_source": ("events around each attention launch (second pass)" if args.staged
                                          else "two events bracketing the timed region, divided by the steps"),
                     "kernel_ms_p10_p90_events_each": [round(float(np.percentile(attn_ms, 10)), 5),
                                                       round(float(np.percentile(attn_ms, 90)), 5)],
                     "per_launch": "algorithmic bytes of the whole batch (one launch covers the batch)",
                     "events_pass_ms_per_step": round(ms_per_step_events, 5)},
    }
    if tile:  # an MFMA-bound workload: TFLOP/s against the dense bf16 peak
        k_tf = alg_flops / (attn_mean * 1e-3) / 1e12
        line.update({"metric": ("prefill tile over FP8 pages, MFMA TFLOP/s (bf16 MFMAs, % of dense bf16 peak), "
                               "1 MI355X" if fp8 else "prefill tile MFMA TFLOP/s (bf16, % of dense peak), 1 MI355X"),
                     "value": round(tflops, 2), "unit": "TFLOP/s"})
        line["roofline"].update({"bound": "mfma", "achieved": round(k_tf, 2), "peak": BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(k_tf / BF16_PEAK_TFLOPS, 4),
                                 "per_launch": "algorithmic flops of the whole batch (one launch covers the batch)"})
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, alg_bytes)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
