"""CPU tests of the C ABI: the built library loads, exports every entry point
include/pa.h declares, and rejects bad descriptors on the host (no GPU call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


@pytest.fixture(scope="module")
def pa():
    from paged_kv_cache_gqa_amd import binding, build
    if build.is_stale():
        build.build()
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("pa_attention", "pa_attention_tree", "pa_attention_fp8kv", "pa_attention_shared_prefix", "pa_workspace_size", "pa_workspace_init", "pa_append_kv", "pa_plan", "pa_attention_planned", "pa_merge_planned",
              "pa_merge", "pa_gather_kv", "pa_validate", "pa_check_desc", "pa_status_string", "pa_abi_version",
              "pa_plan_read", "pa_workspace_bytes", "pa_status_str"):
        assert n in names


def test_library_exports_every_declared_symbol(pa):
    lib = ctypes.CDLL(pa.library_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_abi_version_and_status_strings(pa):
    assert pa.abi_version() == 2
    for st in range(7):
        assert pa.status_string(st).startswith("PA_")
        assert pa.status_str(st) == pa.status_string(st)
    assert "unknown" in pa.status_string(99)


def test_struct_sizes_match_header(pa):
    assert ctypes.sizeof(pa.PaDesc) == 44
    assert ctypes.sizeof(pa.PlanUnit) == 48
    assert ctypes.sizeof(pa.PlanHeader) == 32


def good_desc(pa, **kw):
    d = dict(num_seqs=4, num_q_tokens=4, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16, num_pages=64,
             max_pages_per_seq=16, max_seq_len=0, dtype=0, scale=0.125)
    d.update(kw)
    return pa.PaDesc(**d)


@pytest.mark.parametrize("field,value,status", [
    ("num_seqs", -1, 2), ("num_q_tokens", -3, 2), ("num_q_heads", 0, 2), ("num_kv_heads", 0, 2),
    ("num_kv_heads", 3, 2), ("num_pages", 0, 2), ("max_pages_per_seq", 0, 2), ("head_dim", 96, 3),
    ("head_dim", 256, 3), ("page_size", 32, 3), ("dtype", 2, 3), ("scale", float("nan"), 2),
    ("scale", float("inf"), 2), ("max_pages_per_seq", 1 << 27, 2), ("max_seq_len", -1, 2),
    ("max_seq_len", 16 * 16 + 1, 2),
])
def test_check_desc_rejects(pa, field, value, status):
    assert pa.check_desc(good_desc(pa)) == 0
    assert pa.check_desc(good_desc(pa, **{field: value})) == status


def test_check_desc_accepts_supported_shapes(pa):
    for D in (64, 128):
        for dt in (0, 1):
            for hq, hkv in ((8, 2), (32, 8), (8, 1), (64, 8), (4, 4)):
                assert pa.check_desc(good_desc(pa, head_dim=D, dtype=dt, num_q_heads=hq, num_kv_heads=hkv)) == 0


def test_null_pointers_rejected_without_touching_the_device(pa):
    L = pa.lib()
    d = good_desc(pa)
    # a NULL descriptor is caught before any HIP call
    assert L.pa_check_desc(None) == 1
    assert L.pa_workspace_bytes(None) == 0  # errors read as size 0
    assert L.pa_workspace_bytes(ctypes.byref(good_desc(pa, head_dim=96))) == 0
    assert pa.check_desc(good_desc(pa, max_seq_len=16 * 16)) == 0
    assert pa.check_desc(good_desc(pa, scale=0.0)) == 0
    assert L.pa_attention(None, None, None, None, None, None, None, None, None, None, 0, None) == 1
    assert L.pa_merge(0, 4, 64, None, None, 0, None, None, None) == 2  # n_parts < 1
    assert L.pa_merge(1, 4, 96, None, None, 0, None, None, None) == 3  # head_dim
    assert L.pa_merge(1, 0, 64, None, None, 0, None, None, None) == 0  # nothing to do
    assert L.pa_merge(1, 4, 64, None, None, 0, None, None, None) == 1
    # T_q == 0: pa_attention enqueues nothing and succeeds
    assert L.pa_attention(ctypes.byref(good_desc(pa, num_q_tokens=0)), None, None, None, None, None, None, None,
                          None, None, 0, None) == 0
    # bad descriptor wins over missing pointers
    assert L.pa_attention(ctypes.byref(good_desc(pa, head_dim=80)), None, None, None, None, None, None, None,
                          None, None, 0, None) == 3
    assert L.pa_gather_kv(ctypes.byref(d), 2, None, None, None, 0, 4, None, None) == 2
    assert L.pa_gather_kv(ctypes.byref(d), 0, None, None, None, 7, 4, None, None) == 2  # seq out of range
    # streaming-read diagnostic: sizes are checked before any HIP call
    buf, sink = ctypes.c_void_p(16), ctypes.c_void_p(16)
    assert L.pa_read_stream(None, 1024, 4, sink, None) == 1
    assert L.pa_read_stream(buf, 1024, 0, sink, None) == 2
    assert L.pa_read_stream(buf, 1024, 65536, sink, None) == 2
    assert L.pa_read_stream(buf, 1000, 4, sink, None) == 2  # not a multiple of 16 * grid
    assert L.pa_read_stream(buf, 0, 1, sink, None) == 2
