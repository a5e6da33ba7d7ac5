"""ctypes binding of the C ABI in ``include/pa.h`` (argument marshalling only).

Every function has the name of its C entry point without the ``pa_`` prefix.
torch supplies device memory and the current stream; all arithmetic runs in
the gfx950 kernels of ``libpa_mi355x.so``.  There is no fallback: if the
library is missing or a call fails, a ``PagedAttentionError`` is raised.

Streams: every call takes ``stream=`` (a ``torch.cuda.Stream``; default: torch's
current stream).  Whatever the binding allocates for a call (out, lse, a
workspace and its counter initialisation, contiguous copies of inputs) is
allocated and initialised with that stream current, so torch's caching
allocator orders its reuse after the call's kernels on that stream.

torch is imported before the library is opened so that the library binds to
the HIP runtime torch already loaded (one runtime per process).
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

from .build import LIB_PATH

PAGE_SIZE = 16
ABI_VERSION = 2
PA_F32, PA_BF16 = 0, 1
_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}


class PagedAttentionError(RuntimeError):
    def __init__(self, call: str, status: int, text: str):
        super().__init__(f"{call}: {text} (status {status})")
        self.status = status


class PaDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_tokens", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class PlanUnit(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int32), ("kv_head", ctypes.c_int32), ("row0", ctypes.c_int32),
                ("n_rows", ctypes.c_int32), ("n_keys", ctypes.c_int32), ("n_chunks", ctypes.c_int32),
                ("kind", ctypes.c_int32), ("cost_weight", ctypes.c_int32), ("cost0", ctypes.c_int64),
                ("first_slot", ctypes.c_int32), ("n_pieces", ctypes.c_int32)]


class PlanHeader(ctypes.Structure):
    _fields_ = [("n_units", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("total_cost", ctypes.c_int64), ("reserved", ctypes.c_int64)]


_lib = None


def library_path() -> str:
    return LIB_PATH


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise PagedAttentionError("load", -1, f"{LIB_PATH} is missing; run paged_kv_cache_gqa_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        dp = ctypes.POINTER(PaDesc)
        L.pa_abi_version.restype = ctypes.c_int
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_status_string.argtypes = [ctypes.c_int]
        L.pa_status_str.restype = ctypes.c_char_p
        L.pa_status_str.argtypes = [ctypes.c_int]
        L.pa_workspace_bytes.restype = sz
        L.pa_workspace_bytes.argtypes = [dp]
        L.pa_check_desc.argtypes = [dp]
        L.pa_workspace_size.argtypes = [dp, ctypes.POINTER(sz)]
        L.pa_workspace_init.argtypes = [dp, vp, sz, vp]
        L.pa_attention.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pa_plan.argtypes = [dp, vp, vp, vp, sz, vp]
        L.pa_attention_planned.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pa_merge_planned.argtypes = [dp, vp, vp, vp, vp, vp, sz, vp]
        L.pa_plan_read.argtypes = [dp, vp, vp, vp, sz, ctypes.POINTER(PlanHeader), ctypes.POINTER(PlanUnit), i32,
                                   vp]
        L.pa_gather_kv.argtypes = [dp, i32, vp, vp, vp, i32, i32, vp, vp]
        L.pa_merge.argtypes = [i32, i64, i32, vp, vp, i32, vp, vp, vp]
        L.pa_validate.argtypes = [dp, vp, vp, vp, vp, sz, vp]
        L.pa_append_kv.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.pa_attention_tree.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pa_attention_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.pa_attention_fp8kv.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pa_shared_prefix_workspace_size.argtypes = [dp, i32, ctypes.POINTER(sz)]
        L.pa_attention_shared_prefix.argtypes = [dp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.pa_read_stream.argtypes = [vp, sz, i32, vp, vp]
        for name in ("pa_check_desc", "pa_workspace_size", "pa_workspace_init", "pa_attention", "pa_plan", "pa_attention_planned",
                     "pa_merge_planned", "pa_plan_read", "pa_gather_kv", "pa_merge", "pa_validate", "pa_append_kv", "pa_attention_tree",
                     "pa_attention_fp8kv", "pa_shared_prefix_workspace_size", "pa_attention_shared_prefix",
                     "pa_attention_noalloc", "pa_read_stream"):
            getattr(L, name).restype = ctypes.c_int
        if L.pa_abi_version() != ABI_VERSION:
            raise PagedAttentionError("load", -1, "ABI version mismatch")
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pa_status_string(int(status)).decode()


def status_str(status: int) -> str:
    return lib().pa_status_str(int(status)).decode()


def abi_version() -> int:
    return int(lib().pa_abi_version())


def _check(call: str, status: int) -> None:
    if status != 0:
        raise PagedAttentionError(call, status, status_string(status))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context in which the call's temporaries are allocated: `stream` made current (torch's
    allocator then ties them to it), or nothing when the call runs on the current stream."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def make_desc(q, k_pool, block_table, seq_lens, scale: float, max_seq_len: int = 0) -> PaDesc:
    """Descriptor from tensor shapes (host values only; nothing is read from the device).
    max_seq_len: a known bound on seq_lens, or 0 for none (the block-table width bounds them)."""
    T, Hq, D = q.shape
    NP, Hkv, ps, D2 = k_pool.shape
    if ps != PAGE_SIZE or D2 != D:
        raise ValueError(f"k_pool must be [NP][Hkv][16][{D}], got {tuple(k_pool.shape)}")
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return PaDesc(num_seqs=seq_lens.shape[0], num_q_tokens=T, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                  page_size=PAGE_SIZE, num_pages=NP, max_pages_per_seq=block_table.shape[1],
                  max_seq_len=int(max_seq_len), dtype=_DTYPES[q.dtype], scale=float(scale))


def check_desc(desc: PaDesc) -> int:
    return int(lib().pa_check_desc(ctypes.byref(desc)))


def workspace_size(desc: PaDesc) -> int:
    n = ctypes.c_size_t(0)
    _check("pa_workspace_size", lib().pa_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def workspace_bytes(desc: PaDesc) -> int:
    """pa_workspace_bytes: the workspace size, or 0 for a descriptor pa_workspace_size rejects."""
    return int(lib().pa_workspace_bytes(ctypes.byref(desc)))


def workspace_init(desc: PaDesc, workspace, stream=None) -> None:
    """Zero the workspace's arrival counters (pa_workspace_init)."""
    _check("pa_workspace_init", lib().pa_workspace_init(ctypes.byref(desc), _ptr(workspace), workspace.numel(),
                                                        _stream(stream)))


def alloc_workspace(desc: PaDesc, device=None, stream=None) -> torch.Tensor:
    """A 256-byte-aligned uint8 device buffer of workspace_size(desc) bytes (torch's allocator aligns),
    allocated on `stream` and initialised there with pa_workspace_init."""
    with _on(stream):
        ws = torch.empty(max(workspace_size(desc), 256), dtype=torch.uint8, device=device or "cuda")
        workspace_init(desc, ws, stream)
    return ws


def _check_inputs(q, k_pool, v_pool, block_table, seq_lens, query_start_loc):
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("block_table", block_table),
                    ("seq_lens", seq_lens), ("query_start_loc", query_start_loc)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens), ("query_start_loc", query_start_loc)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise TypeError("q, k_pool and v_pool must share a dtype")
    NP, Hkv, ps, D = k_pool.shape
    if tuple(v_pool.shape) != (NP, Hkv, D, ps):
        raise ValueError(f"v_pool must be [NP][Hkv][D][16] = {(NP, Hkv, D, ps)}, got {tuple(v_pool.shape)}")
    if query_start_loc.shape[0] != seq_lens.shape[0] + 1 or block_table.shape[0] != seq_lens.shape[0]:
        raise ValueError("seq_lens [B], query_start_loc [B+1] and block_table [B][*] disagree")


def _outputs(desc: PaDesc, q, out, lse, workspace, stream):
    """out, lse and workspace of an attention call: the caller's, or allocated (and the workspace's
    counters zeroed) with the call's stream current."""
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(desc, q.device, stream)
    return out, lse, workspace


def attention(q, k_pool, v_pool, block_table, seq_lens, query_start_loc, scale: float, out=None, lse=None,
              workspace=None, stream=None):
    """Paged causal GQA attention (pa_attention).  Returns (out [T_q][Hq][D], lse [T_q][Hq] float32)."""
    _check_inputs(q, k_pool, v_pool, block_table, seq_lens, query_start_loc)
    desc = make_desc(q, k_pool, block_table, seq_lens, scale)
    out, lse, workspace = _outputs(desc, q, out, lse, workspace, stream)
    _check("pa_attention", lib().pa_attention(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                              _ptr(block_table), _ptr(seq_lens), _ptr(query_start_loc), _ptr(out),
                                              _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def attention_noalloc(q, k_pool, v_pool, block_table, seq_lens, query_start_loc, scale: float, out, lse,
                      stream=None):
    """pa_attention_noalloc: pa_attention with the library's static scratch instead of a workspace.
    out [T_q][Hq][D] (q's dtype) and lse [T_q][Hq] float32 are the caller's; nothing is allocated."""
    _check_inputs(q, k_pool, v_pool, block_table, seq_lens, query_start_loc)
    if out.shape != q.shape or out.dtype != q.dtype or lse.shape != q.shape[:2] or lse.dtype != torch.float32:
        raise ValueError("out must match q and lse be float32 [T_q][Hq]")
    if not out.is_contiguous() or not lse.is_contiguous():
        raise ValueError("out and lse must be contiguous")
    desc = make_desc(q, k_pool, block_table, seq_lens, scale)
    _check("pa_attention_noalloc",
           lib().pa_attention_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                      _ptr(seq_lens), _ptr(query_start_loc), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def attention_tree(q, k_pool, v_pool, block_table, seq_lens, query_start_loc, tree_mask, scale: float, out=None,
                   lse=None, workspace=None, stream=None):
    """pa_attention_tree: verify windows as draft-token trees.  tree_mask: [T_q] int64 device tensor holding
    each row's uint64 mask bits.  Returns (out, lse)."""
    _check_inputs(q, k_pool, v_pool, block_table, seq_lens, query_start_loc)
    if (not tree_mask.is_cuda or tree_mask.dtype not in (torch.int64, torch.uint64) or tree_mask.shape != q.shape[:1]
            or not tree_mask.is_contiguous()):
        raise ValueError("tree_mask must be a contiguous [T_q] int64 / uint64 device tensor")
    desc = make_desc(q, k_pool, block_table, seq_lens, scale)
    out, lse, workspace = _outputs(desc, q, out, lse, workspace, stream)
    _check("pa_attention_tree",
           lib().pa_attention_tree(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                   _ptr(seq_lens), _ptr(query_start_loc), _ptr(tree_mask), _ptr(out),
                                   _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def attention_fp8kv(q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, query_start_loc, scale: float,
                    out=None, lse=None, workspace=None, stream=None):
    """pa_attention_fp8kv: K/V pools of FP8 E4M3 codes (uint8) with [NP][Hkv] float32 scales; q and out bf16.
    Returns (out, lse)."""
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("k_scale", k_scale), ("v_scale", v_scale),
                    ("block_table", block_table), ("seq_lens", seq_lens), ("query_start_loc", query_start_loc)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dtype != torch.bfloat16 or k_pool.dtype != torch.uint8 or v_pool.dtype != torch.uint8:
        raise TypeError("q must be bf16 and the pools uint8 FP8 E4M3 codes")
    if k_scale.dtype != torch.float32 or k_scale.shape != k_pool.shape[:2] or v_scale.shape != k_scale.shape:
        raise ValueError("k_scale / v_scale must be float32 [NP][Hkv]")
    T, Hq, D = q.shape
    NP, Hkv = k_pool.shape[:2]
    desc = PaDesc(num_seqs=seq_lens.shape[0], num_q_tokens=T, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                  page_size=PAGE_SIZE, num_pages=NP, max_pages_per_seq=block_table.shape[1], max_seq_len=0,
                  dtype=PA_BF16, scale=float(scale))
    out, lse, workspace = _outputs(desc, q, out, lse, workspace, stream)
    _check("pa_attention_fp8kv",
           lib().pa_attention_fp8kv(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                    _ptr(v_scale), _ptr(block_table), _ptr(seq_lens), _ptr(query_start_loc),
                                    _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def shared_prefix_workspace(desc: PaDesc, num_groups: int, device=None, stream=None) -> torch.Tensor:
    """Workspace for pa_attention_shared_prefix (arrival counters initialised on `stream`)."""
    n = ctypes.c_size_t(0)
    _check("pa_shared_prefix_workspace_size",
           lib().pa_shared_prefix_workspace_size(ctypes.byref(desc), int(num_groups), ctypes.byref(n)))
    with _on(stream):
        ws = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=device or "cuda")
        workspace_init(desc, ws, stream)
    return ws


def attention_shared_prefix(q, k_pool, v_pool, block_table, seq_lens, query_start_loc, group_start, prefix_len,
                            scale: float, out=None, lse=None, workspace=None, stream=None):
    """pa_attention_shared_prefix: groups of sequences (group_start [G+1], prefix_len [G], int32 device
    tensors) whose first prefix_len keys are shared pages.  Returns (out, lse)."""
    _check_inputs(q, k_pool, v_pool, block_table, seq_lens, query_start_loc)
    for name, t in (("group_start", group_start), ("prefix_len", prefix_len)):
        if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    G = prefix_len.shape[0]
    if group_start.shape != (G + 1,):
        raise ValueError("group_start must hold num_groups + 1 entries")
    desc = make_desc(q, k_pool, block_table, seq_lens, scale)
    if workspace is None:
        workspace = shared_prefix_workspace(desc, G, q.device, stream)
    out, lse, workspace = _outputs(desc, q, out, lse, workspace, stream)
    _check("pa_attention_shared_prefix",
           lib().pa_attention_shared_prefix(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                            _ptr(seq_lens), _ptr(query_start_loc), int(G), _ptr(group_start),
                                            _ptr(prefix_len), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                            _stream(stream)))
    return out, lse


def plan(desc: PaDesc, seq_lens, query_start_loc, workspace, stream=None) -> None:
    _check("pa_plan", lib().pa_plan(ctypes.byref(desc), _ptr(seq_lens), _ptr(query_start_loc), _ptr(workspace),
                                    workspace.numel(), _stream(stream)))


def attention_planned(desc: PaDesc, q, k_pool, v_pool, block_table, seq_lens, query_start_loc, out, lse, workspace,
                      stream=None) -> None:
    _check("pa_attention_planned",
           lib().pa_attention_planned(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                      _ptr(seq_lens), _ptr(query_start_loc), _ptr(out), _ptr(lse), _ptr(workspace),
                                      workspace.numel(), _stream(stream)))


def merge_planned(desc: PaDesc, seq_lens, query_start_loc, out, lse, workspace, stream=None) -> None:
    _check("pa_merge_planned", lib().pa_merge_planned(ctypes.byref(desc), _ptr(seq_lens), _ptr(query_start_loc),
                                                      _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                                      _stream(stream)))


def plan_read(desc: PaDesc, seq_lens, query_start_loc, workspace, max_units: int = 1 << 20, stream=None):
    """(header dict, list of unit dicts) of the plan in `workspace` (synchronizes)."""
    hdr = PlanHeader()
    units = (PlanUnit * max(1, max_units))()
    _check("pa_plan_read", lib().pa_plan_read(ctypes.byref(desc), _ptr(seq_lens), _ptr(query_start_loc),
                                              _ptr(workspace), workspace.numel(), ctypes.byref(hdr), units,
                                              max_units, _stream(stream)))
    h = {f: getattr(hdr, f) for f, _ in PlanHeader._fields_}
    n = min(h["n_units"], max_units)
    us = [{f: getattr(units[i], f) for f, _ in PlanUnit._fields_} for i in range(n)]
    return h, us


def gather_kv(desc: PaDesc, which: int, pool, block_table, seq_lens, seq: int, n_keys: int, stream=None):
    """Dense [Hkv][n_keys][D] copy of one sequence's K (which=0) or V (which=1) rows."""
    with _on(stream):
        dense = torch.empty((desc.num_kv_heads, n_keys, desc.head_dim), dtype=pool.dtype, device=pool.device)
    _check("pa_gather_kv", lib().pa_gather_kv(ctypes.byref(desc), int(which), _ptr(pool), _ptr(block_table),
                                              _ptr(seq_lens), int(seq), int(n_keys), _ptr(dense), _stream(stream)))
    return dense


def append_kv(k_new, v_new, k_pool, v_pool, block_table, seq_lens, query_start_loc, stream=None) -> None:
    """Paged KV append (pa_append_kv): write k_new / v_new [T_q][Hkv][D] into the pools at each
    sequence's last q_len positions."""
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_pool", k_pool), ("v_pool", v_pool),
                    ("block_table", block_table), ("seq_lens", seq_lens), ("query_start_loc", query_start_loc)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    T, Hkv, D = k_new.shape
    if v_new.shape != k_new.shape or k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
        raise ValueError("k_new / v_new must be [T_q][Hkv][D] in the pools' dtype")
    desc = PaDesc(num_seqs=seq_lens.shape[0], num_q_tokens=T, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D,
                  page_size=PAGE_SIZE, num_pages=k_pool.shape[0], max_pages_per_seq=block_table.shape[1],
                  max_seq_len=0, dtype=_DTYPES[k_pool.dtype], scale=1.0)
    _check("pa_append_kv", lib().pa_append_kv(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(block_table),
                                              _ptr(seq_lens), _ptr(query_start_loc), _ptr(k_pool), _ptr(v_pool),
                                              _stream(stream)))


def merge(o_parts, lse_parts, out_dtype=torch.float32, stream=None):
    """Log-sum-exp merge (pa_merge) of o_parts [P][rows][D] f32 and lse_parts [P][rows] f32."""
    P, rows, D = o_parts.shape
    with _on(stream):
        o_parts = o_parts.contiguous()
        lse_parts = lse_parts.contiguous()
        out = torch.empty((rows, D), dtype=out_dtype, device=o_parts.device)
        lse = torch.empty((rows,), dtype=torch.float32, device=o_parts.device)
    _check("pa_merge", lib().pa_merge(P, rows, D, _ptr(o_parts), _ptr(lse_parts),
                                      _DTYPES[out_dtype], _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def validate(desc: PaDesc, block_table, seq_lens, query_start_loc, workspace, stream=None) -> int:
    """pa_validate status (0 = OK, 6 = invalid content); synchronizes."""
    st = lib().pa_validate(ctypes.byref(desc), _ptr(block_table), _ptr(seq_lens), _ptr(query_start_loc),
                           _ptr(workspace), workspace.numel(), _stream(stream))
    if st not in (0, 6):
        _check("pa_validate", st)
    return int(st)


def read_stream(buf, grid: int, sink=None, stream=None):
    """pa_read_stream over the bytes of the contiguous device tensor `buf`; returns the [grid] uint32
    sink of per-workgroup XOR words (as int32)."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    with _on(stream):
        if sink is None:
            sink = torch.empty((grid,), dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check("pa_read_stream", lib().pa_read_stream(_ptr(buf), nbytes, grid, _ptr(sink), _stream(stream)))
    return sink


def to_device(w, device="cuda"):
    """Device tensors of a ``workloads.Workload`` (bf16 bit patterns are reinterpreted, not converted)."""
    import numpy as np

    def arr(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    extra = {}
    if "k_scale" in w.meta:  # FP8 pages
        extra = {"k_scale": arr(w.meta["k_scale"]), "v_scale": arr(w.meta["v_scale"])}
    return {**extra, "q": arr(w.q), "k_pool": arr(w.k_pool), "v_pool": arr(w.v_pool),
            "block_table": torch.from_numpy(np.ascontiguousarray(w.block_table, dtype=np.int32)).to(device),
            "seq_lens": torch.from_numpy(np.ascontiguousarray(w.seq_lens, dtype=np.int32)).to(device),
            "query_start_loc": torch.from_numpy(np.ascontiguousarray(w.query_start_loc, dtype=np.int32)).to(device)}
