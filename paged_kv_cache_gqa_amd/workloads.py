"""Seeded synthetic inputs for paged-KV GQA attention.

This module only draws and lays out inputs: sequence lengths, the physical page
placement, the block table and the Q / K-pool / V-pool values.  It holds none
of the attention arithmetic, and it imports neither the oracle nor the HIP
binding, so both sides of every parity test are fed from here.

Layouts (the library's ABI; see ``include/pa.h``):

* ``q``            ``[T_q][Hq][D]``      T_q = query_start_loc[B]
* ``k_pool``       ``[NP][Hkv][16][D]``  one page = 16 token slots, D contiguous
* ``v_pool``       ``[NP][Hkv][D][16]``  same pages, stored transposed (slots contiguous)
* ``block_table``  ``[B][max_pages]``    int32 physical page ids, -1 padding
* ``seq_lens``     ``[B]``               keys per sequence, new tokens included
* ``query_start_loc`` ``[B+1]``          prefix sum of per-sequence query counts

bf16 tensors are carried as ``uint16`` bit patterns (round-to-nearest-even from
float32 draws); float32 tensors as ``float32``.

Random streams: lengths, the page permutation and the config-5 key-outlier
mask come from ``default_rng(seed)`` in that order; Q from
``default_rng([seed, 1])``; the K pool and the V pool are drawn in chunks of
``POOL_CHUNK_PAGES`` pages, chunk ``j`` from ``default_rng([seed, 2, j])`` (K)
and ``default_rng([seed, 3, j])`` (V).  Chunk streams are independent, so large
pools are drawn on several threads with the same result as one thread.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 16
POOL_CHUNK_PAGES = 1024


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    dtype: str  # "f32" | "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    seq_lens: np.ndarray  # int32 [B]
    query_start_loc: np.ndarray  # int32 [B+1]
    block_table: np.ndarray  # int32 [B][max_pages]
    q: np.ndarray  # [T_q][Hq][D]   uint16 (bf16 bits) or float32
    k_pool: np.ndarray  # [NP][Hkv][16][D]
    v_pool: np.ndarray  # [NP][Hkv][D][16]
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_q_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def elem_bytes(self) -> int:
        """Bytes of one Q / output element (bf16 for FP8-KV batches)."""
        return 2 if self.dtype in ("bf16", "fp8") else 4

    @property
    def kv_elem_bytes(self) -> int:
        """Bytes of one K / V pool element."""
        return 1 if self.dtype == "fp8" else self.elem_bytes

    def q_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int64)

    def algorithmic_bytes(self) -> int:
        """Bytes the path must move at least once: every valid K and V row once per
        KV head, Q in, output out, LSE out, and the block-table entries used (FP8 pages: also
        the K and V scale of every used (page, kv head))."""
        n = self.seq_lens.astype(np.int64)
        eb = self.elem_bytes
        hkv, hq, d = self.num_kv_heads, self.num_q_heads, self.head_dim
        tq = self.num_q_tokens
        kv = int(n.sum()) * hkv * d * self.kv_elem_bytes * 2
        pages = int(((n + PAGE_SIZE - 1) // PAGE_SIZE).sum())
        scales = 2 * 4 * pages * hkv if self.dtype == "fp8" else 0
        return kv + 2 * tq * hq * d * eb + 4 * tq * hq + 4 * pages + scales

    def algorithmic_flops(self) -> int:
        """4*D flops (QK^T and PV) per (query row, query head, visible key)."""
        n = self.seq_lens.astype(np.int64)
        ql = self.q_lens()
        # row i of a window of q keys over n keys sees n - q + i + 1 keys
        visible = (ql * (n - ql) + ql * (ql + 1) // 2).sum()
        return int(4 * self.head_dim * self.num_q_heads * visible)


def _draw_normal_bits(seed_parts, n: int, dtype: str) -> np.ndarray:
    x = np.random.default_rng(seed_parts).standard_normal(n, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _draw_pool(seed: int, tag: int, num_pages: int, page_elems: int, dtype: str,
               threads: int | None = None) -> np.ndarray:
    """Fill a whole pool page-chunk by page-chunk from independent streams."""
    out = np.empty(num_pages * page_elems, dtype=np.uint16 if dtype == "bf16" else np.float32)
    nchunks = (num_pages + POOL_CHUNK_PAGES - 1) // POOL_CHUNK_PAGES

    def fill(j: int) -> None:
        p0 = j * POOL_CHUNK_PAGES
        p1 = min(num_pages, p0 + POOL_CHUNK_PAGES)
        out[p0 * page_elems:p1 * page_elems] = _draw_normal_bits([seed, tag, j], (p1 - p0) * page_elems, dtype)

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if nchunks == 1 or threads <= 1:
        for j in range(nchunks):
            fill(j)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def pages_for(n) -> np.ndarray:
    return (np.asarray(n, dtype=np.int64) + PAGE_SIZE - 1) // PAGE_SIZE


def build(name: str, seed: int, seq_lens, q_lens, num_q_heads: int, num_kv_heads: int,
          head_dim: int, dtype: str, scale: float | None = None, num_pages: int | None = None,
          rng: np.random.Generator | None = None, key_outlier_frac: float = 0.0,
          max_pages_per_seq: int | None = None, threads: int | None = None) -> Workload:
    """Lay out a batch: random page placement, block table, then Q, K pool, V pool.

    ``rng`` is the main stream, already advanced past the length draws; it draws
    the page permutation (and the key-outlier mask when ``key_outlier_frac`` > 0).
    ``num_pages`` defaults to ceil(1.1 * pages used).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    assert seq_lens.shape == q_lens.shape
    assert np.all(q_lens >= 0) and np.all(q_lens <= seq_lens)
    if rng is None:
        rng = np.random.default_rng(seed)
    npg = pages_for(seq_lens)
    used = int(npg.sum())
    if num_pages is None:
        num_pages = int(math.ceil(1.1 * used))
    assert num_pages >= used
    max_pages = int(npg.max()) if len(npg) else 0
    if max_pages_per_seq is not None:
        assert max_pages_per_seq >= max_pages
        max_pages = max_pages_per_seq
    max_pages = max(max_pages, 1)
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((len(seq_lens), max_pages), -1, dtype=np.int32)
    cursor = 0
    for s, p in enumerate(npg):
        bt[s, :p] = perm[cursor:cursor + p]
        cursor += int(p)
    qsl = np.zeros(len(seq_lens) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_lens)
    tq = int(qsl[-1])
    d = head_dim
    q = _draw_normal_bits([seed, 1], tq * num_q_heads * d, dtype).reshape(tq, num_q_heads, d)
    page_elems = num_kv_heads * PAGE_SIZE * d
    k = _draw_pool(seed, 2, num_pages, page_elems, dtype, threads).reshape(num_pages, num_kv_heads, PAGE_SIZE, d)
    v = _draw_pool(seed, 3, num_pages, page_elems, dtype, threads).reshape(num_pages, num_kv_heads, d, PAGE_SIZE)
    meta = {"seed": seed, "pages_used": used}
    if key_outlier_frac > 0.0:
        mask = rng.random((num_pages, num_kv_heads, PAGE_SIZE)) < key_outlier_frac
        meta["key_outliers"] = int(mask.sum())
        _scale_rows_by_4(k, mask, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Workload(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=d, scale=float(scale), seq_lens=seq_lens.astype(np.int32),
                    query_start_loc=qsl, block_table=bt, q=q, k_pool=k, v_pool=v, meta=meta)


def _scale_rows_by_4(k: np.ndarray, mask: np.ndarray, dtype: str) -> None:
    """Multiply the selected (page, head, slot) key rows by 4 (exact in bf16 and fp32)."""
    idx = np.nonzero(mask)
    if dtype == "bf16":
        k[idx] = f32_to_bf16_bits(bf16_bits_to_f32(k[idx]) * np.float32(4.0))
    else:
        k[idx] = k[idx] * np.float32(4.0)


# ---------------------------------------------------------------------------
# The five benchmark configurations (seed 1000 + c).
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny-decode-f32",
    2: "llama3-8b-decode-bf16",
    3: "mixed-prefill-decode-bf16",
    4: "spec-verify-bf16",
    5: "long-context-decode-bf16",
}


def config_lengths(c: int):
    """Sequence and query lengths of configuration ``c`` plus the advanced main stream."""
    rng = np.random.default_rng(1000 + c)
    if c == 1:
        n = np.array([17, 64, 100, 256], dtype=np.int64)
        ql = np.ones(4, dtype=np.int64)
    elif c == 2:
        n = rng.integers(512, 4096, 64, endpoint=True)
        ql = np.ones(64, dtype=np.int64)
    elif c == 3:
        prior = rng.integers(0, 2048, 4, endpoint=True)
        dec = rng.integers(1024, 8192, 128, endpoint=True)
        n = np.concatenate([prior + 512, dec])
        ql = np.concatenate([np.full(4, 512), np.ones(128)]).astype(np.int64)
    elif c == 4:
        prior = rng.integers(2048, 16384, 32, endpoint=True)
        n = prior + 5
        ql = np.full(32, 5, dtype=np.int64)
    elif c == 5:
        n = np.clip(np.rint(np.exp(rng.normal(math.log(8192.0), 1.0, 256))), 1024, 32768).astype(np.int64)
        ql = np.ones(256, dtype=np.int64)
    else:
        raise ValueError(f"no configuration {c}")
    return n, ql, rng


def make_config(c: int, threads: int | None = None) -> Workload:
    """Build configuration ``c`` (1..5) with its seed 1000 + c."""
    n, ql, rng = config_lengths(c)
    name = CONFIG_NAMES[c]
    if c == 1:
        return build(name, 1001, n, ql, 8, 2, 64, "f32", scale=1.0 / 8.0, num_pages=64, rng=rng, threads=threads)
    if c == 2:
        return build(name, 1002, n, ql, 32, 8, 128, "bf16", rng=rng, threads=threads)
    if c == 3:
        return build(name, 1003, n, ql, 8, 1, 128, "bf16", rng=rng, threads=threads)
    if c == 4:
        return build(name, 1004, n, ql, 32, 8, 128, "bf16", rng=rng, threads=threads)
    return build(name, 1005, n, ql, 64, 8, 128, "bf16", rng=rng, key_outlier_frac=0.01, threads=threads)


def make_random(seed: int, num_seqs: int, max_len: int, num_q_heads: int, num_kv_heads: int,
                head_dim: int, dtype: str, max_q: int = 1, slack_pages: int = 3, **kw) -> Workload:
    """A small random batch: lengths uniform in [1, max_len], query counts in [0, min(n, max_q)]."""
    rng = np.random.default_rng(seed)
    n = rng.integers(1, max_len, num_seqs, endpoint=True)
    ql = np.minimum(n, rng.integers(0, max_q, num_seqs, endpoint=True))
    used = int(pages_for(n).sum())
    return build(f"random-{seed}", seed, n, ql, num_q_heads, num_kv_heads, head_dim, dtype,
                 num_pages=used + slack_pages, rng=rng, **kw)


def make_interleaved_mixed(seed: int, dtype: str) -> Workload:
    """Prefill windows (2..300 tokens over a prior context of 0..900 keys) and decode / verify
    sequences (1..6 tokens over 1..3000 keys) in a shuffled batch order, with a random kv-head count
    (1, 2, 8), GQA group (1, 4, 8) and head dim (64, 128)."""
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 4, 8]))
    d = int(rng.choice([64, 128]))
    n_pre, n_dec = int(rng.integers(1, 5)), int(rng.integers(5, 120))
    prior = rng.integers(0, 900, n_pre, endpoint=True)
    q_pre = rng.integers(2, 300, n_pre, endpoint=True)
    n_d = rng.integers(1, 3000, n_dec, endpoint=True)
    q_d = np.minimum(n_d, rng.integers(1, 6, n_dec, endpoint=True))
    n, ql = np.concatenate([prior + q_pre, n_d]), np.concatenate([q_pre, q_d])
    perm = rng.permutation(len(n))
    return build(f"interleaved-{seed}", seed, n[perm], ql[perm], g * hkv, hkv, d, dtype, rng=rng)


def subset(w: Workload, seqs) -> Workload:
    """The same pools with only the listed sequences (block-table rows and queries)."""
    seqs = np.asarray(seqs, dtype=np.int64)
    ql = w.q_lens()[seqs]
    qsl = np.zeros(len(seqs) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(ql)
    rows = np.concatenate([np.arange(w.query_start_loc[s], w.query_start_loc[s + 1]) for s in seqs]) \
        if len(seqs) else np.zeros(0, dtype=np.int64)
    return Workload(name=w.name + "-subset", dtype=w.dtype, num_q_heads=w.num_q_heads,
                    num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, scale=w.scale,
                    seq_lens=w.seq_lens[seqs].copy(), query_start_loc=qsl,
                    block_table=np.ascontiguousarray(w.block_table[seqs]), q=np.ascontiguousarray(w.q[rows]),
                    k_pool=w.k_pool, v_pool=w.v_pool, meta=dict(w.meta, subset=seqs.tolist()))


def causal_masks(q_lens) -> np.ndarray:
    """Tree masks that encode the plain causal rule: row i of a window sees window tokens 0..i."""
    rows = []
    for q in np.asarray(q_lens):
        for i in range(int(q)):
            rows.append((1 << (i + 1)) - 1 if i < 63 else (1 << 64) - 1)
    return np.array(rows, dtype=np.uint64)


def random_trees(q_lens, seed: int):
    """A random draft tree per window (token 0 is the root, token k > 0 has a parent in [0, k)) and
    the per-row masks: bit k of row i's mask is set iff window token k is i or an ancestor of i.
    Windows longer than 64 tokens get causal masks.  Returns (masks uint64 [T_q], parents list)."""
    rng = np.random.default_rng([seed, 7])
    masks, parents = [], []
    for q in np.asarray(q_lens):
        q = int(q)
        par = [-1] + [int(rng.integers(0, k)) for k in range(1, q)]
        parents.append(par)
        for i in range(q):
            if q > 64:
                masks.append((1 << (i + 1)) - 1 if i < 63 else (1 << 64) - 1)
                continue
            m, k = 0, i
            while k >= 0:
                m |= 1 << k
                k = par[k]
            masks.append(m)
    return np.array(masks, dtype=np.uint64), parents


FP8_MAX = 448.0  # largest finite OCP FP8 E4M3 value


def _quantize_pool(pool: np.ndarray, chunk_pages: int = 4096):
    """Per-(page, kv head) FP8 E4M3 codes and scales of a pool [NP][Hkv][...]: scale = amax / 448
    over the block (1 for an all-zero block), code = E4M3 rounding of x / scale (torch's
    float8_e4m3fn conversion: round to nearest, ties to even)."""
    import torch
    NP, Hkv = pool.shape[:2]
    codes = np.empty(pool.shape, dtype=np.uint8)
    scales = np.empty((NP, Hkv), dtype=np.float32)
    for p0 in range(0, NP, chunk_pages):
        p1 = min(NP, p0 + chunk_pages)
        x = pool[p0:p1]
        x = bf16_bits_to_f32(x) if x.dtype == np.uint16 else x.astype(np.float32)
        amax = np.abs(x).reshape(p1 - p0, Hkv, -1).max(axis=2)
        sc = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
        y = x / sc.reshape(p1 - p0, Hkv, *([1] * (x.ndim - 2)))
        codes[p0:p1] = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        scales[p0:p1] = sc
    return codes, scales


def to_fp8(w: Workload) -> Workload:
    """The same batch with FP8 E4M3 K/V pages (per-(page, kv head) scales in meta["k_scale"] and
    meta["v_scale"]) and bf16 queries."""
    kc, ks = _quantize_pool(w.k_pool)
    vc, vs = _quantize_pool(w.v_pool)
    q = w.q if w.q.dtype == np.uint16 else f32_to_bf16_bits(w.q)
    meta = dict(w.meta, k_scale=ks, v_scale=vs)
    return Workload(name=w.name + "-fp8kv", dtype="fp8", num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                    head_dim=w.head_dim, scale=w.scale, seq_lens=w.seq_lens, query_start_loc=w.query_start_loc,
                    block_table=w.block_table, q=q, k_pool=kc, v_pool=vc, meta=meta)


def make_shared_prefix(seed: int, group_sizes, prefix_lens, suffix_max: int, max_q: int, num_q_heads: int,
                       num_kv_heads: int, head_dim: int, dtype: str, suffix_min: int = 1, slack_pages: int = 3,
                       name: str | None = None) -> Workload:
    """Groups of sequences that share their first prefix_lens[g] keys (a multiple of 16) as the same
    physical pages, then a private suffix of suffix_min..suffix_max keys holding the query window
    (0..max_q tokens, never longer than the suffix).  meta["group_start"] ([G+1], CSR over the
    sequences) and meta["prefix_len"] ([G]) describe the groups."""
    rng = np.random.default_rng(seed)
    group_sizes = [int(g) for g in group_sizes]
    prefix_lens = [int(p) for p in prefix_lens]
    assert len(group_sizes) == len(prefix_lens) and all(p % PAGE_SIZE == 0 for p in prefix_lens)
    suf, ql = [], []
    for m in group_sizes:
        for _ in range(m):
            u = int(rng.integers(suffix_min, suffix_max, endpoint=True))
            suf.append(u)
            ql.append(min(u, int(rng.integers(0, max_q, endpoint=True))))
    used = sum(p // PAGE_SIZE for p in prefix_lens) + sum((u + PAGE_SIZE - 1) // PAGE_SIZE for u in suf)
    num_pages = used + slack_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    lens, rows = [], []
    cursor, s = 0, 0
    for m, P in zip(group_sizes, prefix_lens):
        shared = perm[cursor:cursor + P // PAGE_SIZE]
        cursor += P // PAGE_SIZE
        for _ in range(m):
            own = perm[cursor:cursor + (suf[s] + PAGE_SIZE - 1) // PAGE_SIZE]
            cursor += len(own)
            rows.append(np.concatenate([shared, own]))
            lens.append(P + suf[s])
            s += 1
    max_pages = max(len(r) for r in rows)
    bt = np.full((len(rows), max_pages), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = r
    qsl = np.zeros(len(rows) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(ql)
    d = head_dim
    q = _draw_normal_bits([seed, 1], int(qsl[-1]) * num_q_heads * d, dtype).reshape(int(qsl[-1]), num_q_heads, d)
    page_elems = num_kv_heads * PAGE_SIZE * d
    k = _draw_pool(seed, 2, num_pages, page_elems, dtype).reshape(num_pages, num_kv_heads, PAGE_SIZE, d)
    v = _draw_pool(seed, 3, num_pages, page_elems, dtype).reshape(num_pages, num_kv_heads, d, PAGE_SIZE)
    gs = np.zeros(len(group_sizes) + 1, dtype=np.int32)
    gs[1:] = np.cumsum(group_sizes)
    meta = {"seed": seed, "pages_used": used, "group_start": gs, "prefix_len": np.array(prefix_lens, dtype=np.int32)}
    return Workload(name=name or f"shared-prefix-{seed}", dtype=dtype, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=d, scale=1.0 / math.sqrt(d),
                    seq_lens=np.array(lens, dtype=np.int32), query_start_loc=qsl, block_table=bt, q=q, k_pool=k,
                    v_pool=v, meta=meta)


def shared_prefix_unique_bytes(w: Workload) -> int:
    """Bytes a shared-prefix batch must move at least once: every distinct (page, kv head) row of
    K and V that some sequence reads (the shared prefix once per group), Q, out, LSE and the
    block-table entries of the prefix pass and of every sequence's suffix."""
    gs, pl = w.meta["group_start"], w.meta["prefix_len"]
    n = w.seq_lens.astype(np.int64)
    hkv, hq, d, eb = w.num_kv_heads, w.num_q_heads, w.head_dim, w.elem_bytes
    keys = int(pl.astype(np.int64).sum()) + int(sum(n[gs[g]:gs[g + 1]].sum() - (gs[g + 1] - gs[g]) * pl[g]
                                                   for g in range(len(pl))))
    tq = w.num_q_tokens
    pages = int((pl // PAGE_SIZE).sum()) + int(sum(((n[gs[g]:gs[g + 1]] - pl[g] + PAGE_SIZE - 1) // PAGE_SIZE).sum()
                                                  for g in range(len(pl))))
    return keys * hkv * d * w.kv_elem_bytes * 2 + 2 * tq * hq * d * eb + 4 * tq * hq + 4 * pages


SHARED_PREFIX_NAME = "shared-prefix-decode-bf16"


def make_shared_prefix_config(seed: int = 1006) -> Workload:
    """System-prompt decode: 8 groups of 16 sequences sharing a 4096-token prefix, private suffixes of
    256..1024 tokens, one query token each; Llama-3-8B attention shape (32 / 8 heads, head dim 128)."""
    return make_shared_prefix(seed, [16] * 8, [4096] * 8, 1024, 1, 32, 8, 128, "bf16", suffix_min=256,
                              name=SHARED_PREFIX_NAME)


LONG_PREFILL_NAME = "long-prefill-bf16"


def make_long_prefill(seed: int = 1007) -> Workload:
    """Long chunked prefill for the prefill tile's steady state: 2 sequences, each a 2048-token
    window on 2048 tokens of prior context (4096 keys), Llama-3-8B attention shape (32 query / 8 KV
    heads, head dim 128), bf16, values N(0, 1), pages in a seeded permutation of a pool with 10%
    slack."""
    return build(LONG_PREFILL_NAME, seed, [4096, 4096], [2048, 2048], 32, 8, 128, "bf16")

