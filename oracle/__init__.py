"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle for paged-KV GQA attention.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg use this
package.  It shares no code with the GPU library (``paged_kv_cache_gqa_amd``)
and imports nothing from it.  The arithmetic lives in ``pa_oracle.c`` (plain
C, double precision); this module builds it with gcc and marshals numpy
arrays through ctypes.

Every function here has at least one independent pin in
``tests/test_oracle.py`` (brute force on tiny inputs, closed forms, page-layout
invariants, reduction to ``torch.nn.functional.scaled_dot_product_attention``
in float64, hand-derived golden cases under ``tests/golden/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")

F32, BF16 = 0, 1
_ERRORS = {1: "bad argument", 2: "bad batch content (q_len > seq_len, page id out of range, ...)",
           3: "out of memory"}

_lib = None


def build(force: bool = True, src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile pa_oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                    "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def open_library(path: str):
    """ctypes handle on a compiled oracle (the default one, or a test's variant)."""
    lib = ctypes.CDLL(path)
    vp, ip = ctypes.c_void_p, ctypes.c_int
    lib.oracle_attention.argtypes = [ip, ip, ip, ip, ip, ip, ip, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_double, vp, vp, ip]
    lib.oracle_attention.restype = ip
    lib.oracle_gather.argtypes = [ip, ip, ip, ip, ip, ip, vp, vp, vp, ip, vp]
    lib.oracle_gather.restype = ip
    lib.oracle_merge.argtypes = [ip, ctypes.c_int64, ip, vp, vp, vp, vp]
    lib.oracle_merge.restype = ip
    lib.oracle_append.argtypes = [ip, ip, ip, ip, ip, ip, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_append.restype = ip
    lib.oracle_attention_tree.argtypes = [ip, ip, ip, ip, ip, ip, ip, vp, vp, vp, vp, vp, vp, vp,
                                          ctypes.c_double, vp, vp]
    lib.oracle_attention_tree.restype = ip
    lib.oracle_fp8_decode.argtypes = [ip]
    lib.oracle_fp8_decode.restype = ctypes.c_double
    lib.oracle_attention_fp8.argtypes = [ip, ip, ip, ip, ip, ip, vp, vp, vp, vp, vp, vp, vp, vp,
                                         ctypes.c_double, vp, vp, ip]
    lib.oracle_attention_fp8.restype = ip
    lib.oracle_max_threads.restype = ip
    return lib


def _load(lib=None):
    global _lib
    if lib is not None:
        return lib
    if _lib is None:
        build(force=False)
        _lib = open_library(LIB_PATH)
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int) -> None:
    if rc != 0:
        raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle takes float32 or bf16 bits (uint16), got {a.dtype}")


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def attention(q, k_pool, v_pool, block_table, seq_lens, query_start_loc, scale: float,
              num_kv_heads: int | None = None, threads: int = 0, lib=None):
    """fp64 paged causal GQA attention.  Returns (out [T_q][Hq][D] f64, lse [T_q][Hq] f64).

    q: [T_q][Hq][D]; k_pool: [NP][Hkv][16][D]; v_pool: [NP][Hkv][D][16];
    both float32 or bf16 bits (uint16), the same for all three.
    """
    lib = _load(lib)
    q = np.ascontiguousarray(q)
    k_pool = np.ascontiguousarray(k_pool)
    v_pool = np.ascontiguousarray(v_pool)
    dt = _dtype_code(q)
    assert _dtype_code(k_pool) == dt and _dtype_code(v_pool) == dt
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    T, Hq, D = q.shape
    NP, Hkv = k_pool.shape[0], k_pool.shape[1]
    if num_kv_heads is not None:
        assert num_kv_heads == Hkv
    assert k_pool.shape == (NP, Hkv, 16, D) and v_pool.shape == (NP, Hkv, D, 16)
    B = sl.shape[0]
    assert qsl.shape == (B + 1,) and int(qsl[-1]) == T
    assert bt.ndim == 2 and bt.shape[0] == B
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.zeros((T, Hq), dtype=np.float64)
    _check(lib.oracle_attention(B, Hq, Hkv, D, dt, NP, bt.shape[1], _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                _ptr(bt), _ptr(sl), _ptr(qsl), float(scale), _ptr(out), _ptr(lse), int(threads)))
    return out, lse


def attention_workload(w, threads: int = 0, lib=None):
    """``attention`` on a ``paged_kv_cache_gqa_amd.workloads.Workload``-like object."""
    return attention(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, w.query_start_loc, w.scale,
                     threads=threads, lib=lib)


def gather(pool, block_table, seq_lens, seq: int, which: str, lib=None):
    """Dense [Hkv][n][D] copy of one sequence's K (which='k') or V (which='v') rows."""
    lib = _load(lib)
    pool = np.ascontiguousarray(pool)
    dt = _dtype_code(pool)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    NP, Hkv = pool.shape[0], pool.shape[1]
    D = pool.shape[3] if which == "k" else pool.shape[2]
    n = int(sl[seq])
    dense = np.zeros((Hkv, n, D), dtype=pool.dtype)
    _check(lib.oracle_gather(0 if which == "k" else 1, dt, Hkv, D, NP, bt.shape[1], _ptr(pool), _ptr(bt),
                             _ptr(sl), int(seq), _ptr(dense)))
    return dense


def merge(o_parts, lse_parts, lib=None):
    """Combine results over disjoint key sets: o_parts [P][rows][D], lse_parts [P][rows]."""
    lib = _load(lib)
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    P, rows, D = o_parts.shape
    assert lse_parts.shape == (P, rows)
    o = np.zeros((rows, D), dtype=np.float64)
    lse = np.zeros(rows, dtype=np.float64)
    _check(lib.oracle_merge(P, rows, D, _ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse)))
    return o, lse


def append(k_new, v_new, k_pool, v_pool, block_table, seq_lens, query_start_loc, lib=None):
    """Paged KV append: copies of k_pool / v_pool with the new tokens' rows written in.

    k_new, v_new: [T_q][Hkv][D]; token i of sequence s goes to position seq_lens[s] - q_s + i."""
    lib = _load(lib)
    k_new = np.ascontiguousarray(k_new)
    v_new = np.ascontiguousarray(v_new)
    k_out = np.array(k_pool, copy=True, order="C")
    v_out = np.array(v_pool, copy=True, order="C")
    dt = _dtype_code(k_out)
    assert _dtype_code(v_out) == dt and _dtype_code(k_new) == dt and _dtype_code(v_new) == dt
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    NP, Hkv, _, D = k_out.shape
    B = sl.shape[0]
    assert k_new.shape == (int(qsl[-1]), Hkv, D) and v_new.shape == k_new.shape
    _check(lib.oracle_append(B, Hkv, D, dt, NP, bt.shape[1], _ptr(bt), _ptr(sl), _ptr(qsl), _ptr(k_new),
                             _ptr(v_new), _ptr(k_out), _ptr(v_out)))
    return k_out, v_out


def attention_tree(q, k_pool, v_pool, block_table, seq_lens, query_start_loc, tree_mask, scale: float, lib=None):
    """fp64 attention with tree-structured verify windows: tree_mask [T_q] uint64, bit k of row r's
    mask lets it see window token k (windows of at most 64 tokens; longer windows are causal)."""
    lib = _load(lib)
    q = np.ascontiguousarray(q)
    k_pool = np.ascontiguousarray(k_pool)
    v_pool = np.ascontiguousarray(v_pool)
    dt = _dtype_code(q)
    assert _dtype_code(k_pool) == dt and _dtype_code(v_pool) == dt
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    tm = np.ascontiguousarray(tree_mask, dtype=np.uint64)
    T, Hq, D = q.shape
    NP, Hkv = k_pool.shape[0], k_pool.shape[1]
    B = sl.shape[0]
    assert tm.shape == (T,) and qsl.shape == (B + 1,) and int(qsl[-1]) == T
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.zeros((T, Hq), dtype=np.float64)
    _check(lib.oracle_attention_tree(B, Hq, Hkv, D, dt, NP, bt.shape[1], _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                     _ptr(bt), _ptr(sl), _ptr(qsl), _ptr(tm), float(scale), _ptr(out), _ptr(lse)))
    return out, lse


def fp8_decode(code: int, lib=None) -> float:
    """Value of one OCP FP8 E4M3 code (0..255)."""
    return float(_load(lib).oracle_fp8_decode(int(code)))


def attention_fp8(q, k_codes, v_codes, k_scale, v_scale, block_table, seq_lens, query_start_loc, scale: float,
                  threads: int = 0, lib=None):
    """fp64 attention over FP8 E4M3 pages with per-(page, kv head) scales.
    q: [T_q][Hq][D] bf16 bits; k_codes [NP][Hkv][16][D], v_codes [NP][Hkv][D][16] uint8;
    k_scale, v_scale [NP][Hkv] float32."""
    lib = _load(lib)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kc = np.ascontiguousarray(k_codes, dtype=np.uint8)
    vc = np.ascontiguousarray(v_codes, dtype=np.uint8)
    ks = np.ascontiguousarray(k_scale, dtype=np.float32)
    vs = np.ascontiguousarray(v_scale, dtype=np.float32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    T, Hq, D = q.shape
    NP, Hkv = kc.shape[0], kc.shape[1]
    assert kc.shape == (NP, Hkv, 16, D) and vc.shape == (NP, Hkv, D, 16) and ks.shape == vs.shape == (NP, Hkv)
    B = sl.shape[0]
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.zeros((T, Hq), dtype=np.float64)
    _check(lib.oracle_attention_fp8(B, Hq, Hkv, D, NP, bt.shape[1], _ptr(q), _ptr(kc), _ptr(vc), _ptr(ks), _ptr(vs),
                                    _ptr(bt), _ptr(sl), _ptr(qsl), float(scale), _ptr(out), _ptr(lse), int(threads)))
    return out, lse
