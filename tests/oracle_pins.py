"""Independent pins for the fp64 oracle (imported by test_oracle.py).

Each ``pin_*`` function checks the oracle (the default build, or a variant
library passed as ``lib``) against something that is not the oracle itself:

* brute force: pure-Python ``math.fsum`` attention over K/V rows gathered by
  a Python page walk, on tiny random batches;
* closed forms: a single key, equal scores, two keys, the causal staircase
  (q = 0 and V_j = j), strictly dominant last key;
* hand-derived cases in ``tests/golden/worked_examples.json``;
* invariants: physical page permutation, NaN poison outside valid slots, GQA
  equals MHA with repeated K/V heads, merge of key splits;
* reduction to ``torch.nn.functional.scaled_dot_product_attention`` (float64,
  explicit bottom-right causal mask) and ``torch.logsumexp``.

Each raises AssertionError on a mismatch.  They are functions (not tests) so
that the mutation test can run all of them against an oracle with a planted
mistake and demand that at least one fails.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from paged_kv_cache_gqa_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")
PS = 16


# ---------------------------------------------------------------------------
# helpers (no attention arithmetic beyond the brute-force statement itself)
# ---------------------------------------------------------------------------

def widen(a: np.ndarray) -> np.ndarray:
    """float64 values of a float32 or bf16-bits array."""
    if a.dtype == np.uint16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def narrow(x, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return W.f32_to_bf16_bits(x) if dtype == "bf16" else x


def dense_kv(w, s: int):
    """K and V of sequence s as float64 [Hkv][n][D], by a Python page walk."""
    n = int(w.seq_lens[s])
    k = widen(w.k_pool)
    v = widen(w.v_pool)
    Hkv, D = w.num_kv_heads, w.head_dim
    K = np.zeros((Hkv, n, D))
    V = np.zeros((Hkv, n, D))
    for j in range(n):
        pg = int(w.block_table[s, j // PS])
        t = j % PS
        for g in range(Hkv):
            K[g, j, :] = k[pg, g, t, :]
            V[g, j, :] = v[pg, g, :, t]
    return K, V


def brute_force(w):
    """Pure-Python attention (math.fsum sums, math.exp weights)."""
    T, Hq, D = w.num_q_tokens, w.num_q_heads, w.head_dim
    G = Hq // w.num_kv_heads
    q = widen(w.q)
    out = np.zeros((T, Hq, D))
    lse = np.zeros((T, Hq))
    for s in range(w.num_seqs):
        K, V = dense_kv(w, s)
        n = int(w.seq_lens[s])
        q0, q1 = int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
        for i, r in enumerate(range(q0, q1)):
            last = n - (q1 - q0) + i
            for h in range(Hq):
                g = h // G
                x = [w.scale * math.fsum(float(a) * float(b) for a, b in zip(q[r, h], K[g, j]))
                     for j in range(last + 1)]
                m = max(x)
                e = [math.exp(xj - m) for xj in x]
                tot = math.fsum(e)
                for d in range(D):
                    out[r, h, d] = math.fsum(e[j] * V[g, j, d] for j in range(last + 1)) / tot
                lse[r, h] = m + math.log(tot)
    return out, lse


def run(w, lib=None):
    return oracle.attention_workload(w, lib=lib)


def poison_unused(w):
    """Copy of w whose pool slots outside every sequence's valid keys hold NaN."""
    k = w.k_pool.copy()
    v = w.v_pool.copy()
    valid = np.zeros((w.num_pages, PS), dtype=bool)
    for s in range(w.num_seqs):
        n = int(w.seq_lens[s])
        for j in range(n):
            valid[int(w.block_table[s, j // PS]), j % PS] = True
    nan = W.f32_to_bf16_bits(np.float32(np.nan)) if w.dtype == "bf16" else np.float32(np.nan)
    for pg in range(w.num_pages):
        for t in range(PS):
            if not valid[pg, t]:
                k[pg, :, t, :] = nan
                v[pg, :, :, t] = nan
    return _replace(w, k_pool=k, v_pool=v)


def permute_pages(w, seed: int):
    """Same logical cache with physical pages renumbered by a random permutation."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(w.num_pages)  # old page id -> new page id
    k = np.empty_like(w.k_pool)
    v = np.empty_like(w.v_pool)
    k[perm] = w.k_pool
    v[perm] = w.v_pool
    bt = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    return _replace(w, k_pool=k, v_pool=v, block_table=bt)


def _replace(w, **kw):
    d = dict(name=w.name, dtype=w.dtype, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
             head_dim=w.head_dim, scale=w.scale, seq_lens=w.seq_lens, query_start_loc=w.query_start_loc,
             block_table=w.block_table, q=w.q, k_pool=w.k_pool, v_pool=w.v_pool, meta=dict(w.meta))
    d.update(kw)
    return W.Workload(**d)


def from_logical(dtype, Hq, Hkv, D, scale, num_pages, seqs):
    """Build a batch from logical rows.  seqs: list of dicts with 'page_ids', 'keys', 'values'
    ([key][kv_head][d] arrays) and 'queries' ([token][q_head][d]).  Unlisted slots hold NaN."""
    nan = np.float32(np.nan)
    kf = np.full((num_pages, Hkv, PS, D), nan, dtype=np.float32)
    vf = np.full((num_pages, Hkv, D, PS), nan, dtype=np.float32)
    max_pages = max(len(sq["page_ids"]) for sq in seqs)
    bt = np.full((len(seqs), max_pages), -1, dtype=np.int32)
    lens, qs = [], []
    for s, sq in enumerate(seqs):
        keys = np.asarray(sq["keys"], dtype=np.float64)
        vals = np.asarray(sq["values"], dtype=np.float64)
        n = keys.shape[0]
        bt[s, :len(sq["page_ids"])] = sq["page_ids"]
        for j in range(n):
            pg = sq["page_ids"][j // PS]
            kf[pg, :, j % PS, :] = keys[j]
            vf[pg, :, :, j % PS] = vals[j]
        lens.append(n)
        qs.append(np.asarray(sq["queries"], dtype=np.float32).reshape(-1, Hq, D))
    q = np.concatenate(qs, axis=0)
    qsl = np.zeros(len(seqs) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum([x.shape[0] for x in qs])
    return W.Workload(name="logical", dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                      scale=float(scale), seq_lens=np.asarray(lens, dtype=np.int32), query_start_loc=qsl,
                      block_table=bt, q=narrow(q, dtype), k_pool=narrow(kf, dtype), v_pool=narrow(vf, dtype))


def tiny_batches():
    """Random tiny batches: ragged lengths, windows of several rows, GQA, both dtypes."""
    out = []
    for seed, (B, maxlen, Hq, Hkv, D, dt, maxq) in enumerate([
            (3, 40, 4, 2, 8, "f32", 6), (2, 35, 4, 1, 4, "bf16", 35), (3, 20, 2, 2, 8, "f32", 1),
            (2, 33, 6, 3, 4, "bf16", 4)]):
        out.append(W.make_random(100 + seed, B, maxlen, Hq, Hkv, D, dt, max_q=maxq))
    return out


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_brute_force(lib=None):
    for w in tiny_batches():
        o, l = run(w, lib)
        bo, bl = brute_force(w)
        assert np.max(np.abs(o - bo)) <= 1e-12, (w.name, np.max(np.abs(o - bo)))
        assert np.max(np.abs(l - bl)) <= 1e-12, (w.name, np.max(np.abs(l - bl)))


def pin_golden(lib=None):
    doc = json.load(open(GOLDEN))
    for case in doc["cases"]:
        Hq, Hkv, D = case["num_q_heads"], case["num_kv_heads"], case["head_dim"]
        seqs = []
        for sq in case["sequences"]:
            keys = np.asarray(sq["keys"], dtype=np.float64)
            vals = np.asarray(sq["values"], dtype=np.float64)
            if not sq.get("per_head"):
                keys = np.repeat(keys[:, None, :], Hkv, axis=1)
                vals = np.repeat(vals[:, None, :], Hkv, axis=1)
            seqs.append(dict(sq, keys=keys, values=vals))
        exp_out = [np.asarray(x, dtype=np.float64) for x in
                   [[[float(v) for v in h] for h in tok] for tok in case["out"]]]
        exp_lse = np.asarray([[float(v) for v in tok] for tok in case["lse"]], dtype=np.float64)
        for dt in case["dtype"]:
            w = from_logical(dt, Hq, Hkv, D, case["scale"], case["num_pages"], seqs)
            o, l = run(w, lib)
            assert np.max(np.abs(o - np.asarray(exp_out))) <= 1e-12, (case["name"], dt)
            assert np.max(np.abs(l - exp_lse)) <= 1e-12, (case["name"], dt)


def pin_closed_forms(lib=None):
    rng = np.random.default_rng(7)
    D, Hq, Hkv = 8, 4, 2
    # (i) one key: out = V_0, lse = scale * q.k_0
    for dt in ("f32", "bf16"):
        k = rng.standard_normal((1, Hkv, D))
        v = rng.standard_normal((1, Hkv, D))
        q = rng.standard_normal((1, Hq, D))
        w = from_logical(dt, Hq, Hkv, D, 0.3, 2, [dict(page_ids=[1], keys=k, values=v, queries=q)])
        o, l = run(w, lib)
        kk, vv, qq = widen(w.k_pool)[1, :, 0, :], widen(w.v_pool)[1, :, :, 0], widen(w.q)[0]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            assert np.array_equal(o[0, h], vv[g]), "single key must return V_0 exactly"
            assert abs(l[0, h] - 0.3 * math.fsum(qq[h] * kk[g])) <= 1e-12
    # (ii) equal scores (q = 0): out = mean of visible V rows, lse = ln(#visible); over 3 pages
    n, win = 37, 5
    k = rng.standard_normal((n, Hkv, D))
    v = rng.standard_normal((n, Hkv, D))
    q = np.zeros((win, Hq, D))
    w = from_logical("f32", Hq, Hkv, D, 1.0, 4, [dict(page_ids=[3, 0, 2], keys=k, values=v, queries=q)])
    o, l = run(w, lib)
    vv = v.astype(np.float32).astype(np.float64)
    for i in range(win):
        last = n - win + i
        for h in range(Hq):
            g = h // (Hq // Hkv)
            assert np.max(np.abs(o[i, h] - vv[:last + 1, g].mean(axis=0))) <= 1e-12
            assert abs(l[i, h] - math.log(last + 1)) <= 1e-12
    # (iii) two keys: weights sigmoid(x0 - x1), sigmoid(x1 - x0)
    k = rng.standard_normal((2, 1, D))
    v = rng.standard_normal((2, 1, D))
    q = rng.standard_normal((1, 1, D))
    w = from_logical("f32", 1, 1, D, 0.7, 1, [dict(page_ids=[0], keys=k, values=v, queries=q)])
    o, l = run(w, lib)
    kk, vv, qq = widen(w.k_pool)[0, 0, :2, :], widen(w.v_pool)[0, 0, :, :2].T, widen(w.q)[0, 0]
    x0, x1 = 0.7 * math.fsum(qq * kk[0]), 0.7 * math.fsum(qq * kk[1])
    a = 1.0 / (1.0 + math.exp(x1 - x0))
    assert np.max(np.abs(o[0, 0] - (a * vv[0] + (1 - a) * vv[1]))) <= 1e-12
    assert abs(l[0, 0] - (max(x0, x1) + math.log1p(math.exp(-abs(x0 - x1))))) <= 1e-12
    # (iv) causal staircase: q = 0, V_j = j -> row i of a window over prior P: out = (P+i)/2
    P, win = 21, 12
    n = P + win
    k = rng.standard_normal((n, 1, 4))
    v = np.repeat(np.arange(n, dtype=np.float64)[:, None, None], 4, axis=2)
    for dt in ("f32", "bf16"):
        w = from_logical(dt, 2, 1, 4, 0.25, 3, [dict(page_ids=[2, 1, 0], keys=k, values=v,
                                                     queries=np.zeros((win, 2, 4)))])
        o, l = run(w, lib)
        for i in range(win):
            assert np.max(np.abs(o[i] - (P + i) / 2.0)) <= 1e-12, ("staircase", dt, i)
            assert np.max(np.abs(l[i] - math.log(P + i + 1))) <= 1e-12
    # (v) strictly increasing, widely spaced scores: out = V of the last visible key
    n, win = 20, 4
    k = np.zeros((n, 1, 2))
    k[:, 0, 0] = 50.0 * np.arange(n)
    v = rng.standard_normal((n, 1, 2))
    w = from_logical("f32", 1, 1, 2, 1.0, 2, [dict(page_ids=[1, 0], keys=k, values=v,
                                                   queries=np.tile([[[1.0, 0.0]]], (win, 1, 1)))])
    o, l = run(w, lib)
    vv = v.astype(np.float32).astype(np.float64)
    for i in range(win):
        last = n - win + i
        assert np.max(np.abs(o[i, 0] - vv[last, 0])) <= 1e-12
        assert abs(l[i, 0] - 50.0 * last) <= 1e-9


def pin_invariants(lib=None):
    for w in tiny_batches()[:2] + [W.make_config(1)]:
        o, l = run(w, lib)
        o2, l2 = run(permute_pages(w, 5), lib)
        assert np.array_equal(o, o2) and np.array_equal(l, l2), "page permutation changed the result"
        o3, l3 = run(poison_unused(w), lib)
        assert np.array_equal(o, o3) and np.array_equal(l, l3), "unused slots leaked into the result"
    # GQA == MHA with each K/V head repeated G times
    w = W.make_random(301, 3, 30, 6, 2, 8, "f32", max_q=5)
    G = 3
    mha = _replace(w, num_kv_heads=6, k_pool=np.repeat(w.k_pool, G, axis=1),
                   v_pool=np.repeat(w.v_pool, G, axis=1))
    o, l = run(w, lib)
    o2, l2 = run(mha, lib)
    assert np.array_equal(o, o2) and np.array_equal(l, l2), "GQA differs from MHA with repeated K/V"


def pin_merge_of_splits(lib=None):
    """Attention over keys [0, a) and [a, n) merged == attention over [0, n), for every a."""
    rng = np.random.default_rng(11)
    n, D, Hq, Hkv = 37, 8, 4, 2
    k = rng.standard_normal((n, Hkv, D))
    v = rng.standard_normal((n, Hkv, D))
    q = rng.standard_normal((1, Hq, D))
    full = from_logical("f32", Hq, Hkv, D, 0.4, 3, [dict(page_ids=[0, 1, 2], keys=k, values=v, queries=q)])
    o, l = run(full, lib)
    for a in range(1, n):
        left = from_logical("f32", Hq, Hkv, D, 0.4, 3, [dict(page_ids=[2, 0, 1][:(a + 15) // 16], keys=k[:a],
                                                            values=v[:a], queries=q)])
        right = from_logical("f32", Hq, Hkv, D, 0.4, 3, [dict(page_ids=[1, 2, 0][:(n - a + 15) // 16],
                                                             keys=k[a:], values=v[a:], queries=q)])
        o1, l1 = run(left, lib)
        o2, l2 = run(right, lib)
        om, lm = oracle.merge(np.stack([o1.reshape(Hq, D), o2.reshape(Hq, D)]), np.stack([l1[0], l2[0]]), lib=lib)
        assert np.max(np.abs(om - o.reshape(Hq, D))) <= 1e-12, a
        assert np.max(np.abs(lm - l[0])) <= 1e-12, a
    # a part that saw no key (lse = -inf) contributes nothing
    om, lm = oracle.merge(np.stack([o.reshape(Hq, D), np.full((Hq, D), 123.0)]),
                          np.stack([l[0], np.full(Hq, -np.inf)]), lib=lib)
    assert np.max(np.abs(om - o.reshape(Hq, D))) <= 1e-15 and np.max(np.abs(lm - l[0])) <= 1e-15
    # closed form: parts with lse ln 1 and ln 3 weigh 1/4 and 3/4
    om, lm = oracle.merge(np.array([[[4.0]], [[8.0]]]), np.array([[0.0], [math.log(3.0)]]), lib=lib)
    assert abs(om[0, 0] - 7.0) <= 1e-14 and abs(lm[0] - math.log(4.0)) <= 1e-14


def pin_sdpa(lib=None):
    """fp64 torch scaled_dot_product_attention with an explicit bottom-right causal mask."""
    import torch
    for seed, (B, maxlen, Hq, Hkv, D, dt, maxq) in enumerate([
            (3, 300, 8, 2, 64, "f32", 40), (2, 200, 4, 4, 128, "bf16", 200), (4, 90, 8, 1, 64, "bf16", 3)]):
        w = W.make_random(200 + seed, B, maxlen, Hq, Hkv, D, dt, max_q=maxq)
        o, l = run(w, lib)
        G = Hq // Hkv
        q = torch.from_numpy(widen(w.q))
        for s in range(w.num_seqs):
            q0, q1 = int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
            if q1 == q0:
                continue
            n = int(w.seq_lens[s])
            K, V = dense_kv(w, s)
            Kt = torch.from_numpy(K).repeat_interleave(G, dim=0)  # [Hq][n][D]
            Vt = torch.from_numpy(V).repeat_interleave(G, dim=0)
            Q = q[q0:q1].transpose(0, 1).contiguous()  # [Hq][win][D]
            win = q1 - q0
            mask = torch.arange(n)[None, :] <= (n - win + torch.arange(win))[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(Q[None], Kt[None], Vt[None],
                                                                   attn_mask=mask[None, None], scale=w.scale)[0]
            scores = (Q @ Kt.transpose(1, 2).contiguous()) * w.scale
            ref_lse = torch.logsumexp(scores.masked_fill(~mask[None], -math.inf), dim=-1)  # [Hq][win]
            assert np.max(np.abs(o[q0:q1] - ref.transpose(0, 1).numpy())) <= 1e-12, (seed, s)
            assert np.max(np.abs(l[q0:q1] - ref_lse.transpose(0, 1).numpy())) <= 1e-12, (seed, s)


def pin_gather(lib=None):
    for w in tiny_batches()[:2]:
        for s in range(w.num_seqs):
            n = int(w.seq_lens[s])
            pages = w.block_table[s, (np.arange(n) // PS)]
            slots = np.arange(n) % PS
            ek = w.k_pool[pages, :, slots, :].transpose(1, 0, 2)  # numpy fancy-index gather
            ev = w.v_pool[pages, :, :, slots].transpose(1, 0, 2)
            gk = oracle.gather(w.k_pool, w.block_table, w.seq_lens, s, "k", lib=lib)
            gv = oracle.gather(w.v_pool, w.block_table, w.seq_lens, s, "v", lib=lib)
            assert gk.tobytes() == np.ascontiguousarray(ek).tobytes()
            assert gv.tobytes() == np.ascontiguousarray(ev).tobytes()


def pin_append(lib=None):
    """Paged KV append, pinned without its own formula: (1) the pinned page-walk gather of every
    sequence returns its old context followed by exactly its new rows; (2) nothing else changes (the
    new values lie in [1000, 1001), which no pool value does, and exactly T_q * Hkv * D elements of
    each pool differ); (3) attention over the appended pools equals fp64 torch SDPA over the dense
    concatenation of the old context and the new rows."""
    import torch
    for seed, (B, maxlen, Hq, Hkv, D, dt, maxq) in enumerate([
            (4, 200, 8, 2, 64, "f32", 40), (5, 300, 4, 1, 128, "bf16", 70), (6, 60, 8, 8, 64, "bf16", 1)]):
        w = W.make_random(300 + seed, B, maxlen, Hq, Hkv, D, dt, max_q=maxq)
        T = w.num_q_tokens
        rng = np.random.default_rng(400 + seed)
        k_new = narrow(1000.0 + rng.random((T, Hkv, D)), dt)
        v_new = narrow(1000.0 + rng.random((T, Hkv, D)), dt)
        k2, v2 = oracle.append(k_new, v_new, w.k_pool, w.v_pool, w.block_table, w.seq_lens, w.query_start_loc,
                               lib=lib)
        for old, new in ((w.k_pool, k2), (w.v_pool, v2)):
            changed = widen(old) != widen(new)
            assert int(changed.sum()) == T * Hkv * D, (seed, int(changed.sum()))
        q = torch.from_numpy(widen(w.q))
        G = Hq // Hkv
        after = _replace(w, k_pool=k2, v_pool=v2)
        o, l = run(after, lib)
        for s in range(w.num_seqs):
            n = int(w.seq_lens[s])
            q0, q1 = int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
            win = q1 - q0
            gk_old = oracle.gather(w.k_pool, w.block_table, w.seq_lens, s, "k", lib=lib)
            gv_old = oracle.gather(w.v_pool, w.block_table, w.seq_lens, s, "v", lib=lib)
            gk = oracle.gather(k2, w.block_table, w.seq_lens, s, "k", lib=lib)
            gv = oracle.gather(v2, w.block_table, w.seq_lens, s, "v", lib=lib)
            for g_old, g_new, rows in ((gk_old, gk, k_new), (gv_old, gv, v_new)):
                assert g_new[:, :n - win].tobytes() == g_old[:, :n - win].tobytes(), seed
                assert g_new[:, n - win:].tobytes() == np.ascontiguousarray(rows[q0:q1].transpose(1, 0, 2)).tobytes()
            if win == 0:
                continue
            K = np.concatenate([widen(gk_old[:, :n - win]), widen(k_new[q0:q1]).transpose(1, 0, 2)], axis=1)
            V = np.concatenate([widen(gv_old[:, :n - win]), widen(v_new[q0:q1]).transpose(1, 0, 2)], axis=1)
            Kt = torch.from_numpy(K).repeat_interleave(G, dim=0)
            Vt = torch.from_numpy(V).repeat_interleave(G, dim=0)
            Q = q[q0:q1].transpose(0, 1).contiguous()
            mask = torch.arange(n)[None, :] <= (n - win + torch.arange(win))[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(Q[None], Kt[None], Vt[None],
                                                                   attn_mask=mask[None, None], scale=w.scale)[0]
            assert np.max(np.abs(o[q0:q1] - ref.transpose(0, 1).numpy())) <= 1e-9, (seed, s)


def pin_tree(lib=None):
    """Tree-structured verify windows.  (1) causal masks give exactly the plain attention; (2) with
    random draft trees, every row equals fp64 torch SDPA of that one query over the sequence's
    context followed by the K/V of its ancestor path (built from the parent pointers, not from the
    masks); (3) windows longer than 64 tokens ignore their masks; (4) a row that sees no key gives
    out = 0 and lse = -inf."""
    import torch
    for seed, (B, maxlen, Hq, Hkv, D, dt, maxq) in enumerate([
            (4, 120, 8, 2, 64, "f32", 12), (3, 90, 4, 1, 64, "bf16", 20), (5, 60, 8, 8, 64, "bf16", 6)]):
        w = W.make_random(500 + seed, B, maxlen, Hq, Hkv, D, dt, max_q=maxq)
        args = (w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, w.query_start_loc)
        o_ref, l_ref = run(w, lib)
        o, l = oracle.attention_tree(*args, W.causal_masks(w.q_lens()), w.scale, lib=lib)
        assert np.max(np.abs(o - o_ref)) <= 1e-13 and np.max(np.abs(l - l_ref)) <= 1e-13, seed
        masks, parents = W.random_trees(w.q_lens(), 600 + seed)
        o, l = oracle.attention_tree(*args, masks, w.scale, lib=lib)
        q = widen(w.q)
        G = Hq // Hkv
        for s in range(w.num_seqs):
            n = int(w.seq_lens[s])
            q0, q1 = int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
            win = q1 - q0
            K, V = dense_kv(w, s)
            for i in range(win):
                path, k = [], i
                while k >= 0:
                    path.append(n - win + k)
                    k = parents[s][k]
                keys = list(range(n - win)) + sorted(path)
                Kp = torch.from_numpy(K[:, keys]).repeat_interleave(G, dim=0)
                Vp = torch.from_numpy(V[:, keys]).repeat_interleave(G, dim=0)
                Q = torch.from_numpy(q[q0 + i])[:, None, :]  # [Hq][1][D]
                ref = torch.nn.functional.scaled_dot_product_attention(Q[None], Kp[None], Vp[None], scale=w.scale)[0]
                ref_l = torch.logsumexp((Q @ Kp.transpose(1, 2).contiguous())[:, 0] * w.scale, dim=-1)
                assert np.max(np.abs(o[q0 + i] - ref[:, 0].numpy())) <= 1e-12, (seed, s, i)
                assert np.max(np.abs(l[q0 + i] - ref_l.numpy())) <= 1e-12, (seed, s, i)
    # (3) a 70-token window over 150 keys and a 20-token window: the long window ignores its masks
    rng = np.random.default_rng(510)
    lw = from_logical("f32", 4, 2, 16, 0.25, 20, [
        dict(page_ids=[3, 7, 1, 12, 0, 9, 15, 4, 11, 18], keys=rng.standard_normal((150, 2, 16)),
             values=rng.standard_normal((150, 2, 16)), queries=rng.standard_normal((70, 4, 16))),
        dict(page_ids=[5, 2], keys=rng.standard_normal((30, 2, 16)), values=rng.standard_normal((30, 2, 16)),
             queries=rng.standard_normal((20, 4, 16)))])
    masks, _ = W.random_trees(lw.q_lens(), 7)
    masks[:70] = rng.integers(0, 2**63, size=70, dtype=np.int64).astype(np.uint64)  # garbage: ignored
    causal = W.causal_masks(lw.q_lens())
    o_ref, l_ref = oracle.attention_tree(lw.q, lw.k_pool, lw.v_pool, lw.block_table, lw.seq_lens,
                                         lw.query_start_loc, causal, lw.scale, lib=lib)
    o, l = oracle.attention_tree(lw.q, lw.k_pool, lw.v_pool, lw.block_table, lw.seq_lens, lw.query_start_loc,
                                 masks, lw.scale, lib=lib)
    assert np.max(np.abs(o[:70] - o_ref[:70])) <= 1e-13 and np.max(np.abs(l[:70] - l_ref[:70])) <= 1e-13
    assert np.max(np.abs(o[70:] - o_ref[70:])) > 1e-6  # the short window's tree does change its rows
    # (4) no context and a row whose mask hides even itself
    ew = from_logical("f32", 4, 2, 8, 0.3, 4, [
        dict(page_ids=[2], keys=rng.standard_normal((3, 2, 8)), values=rng.standard_normal((3, 2, 8)),
             queries=rng.standard_normal((3, 4, 8)))])
    o, l = oracle.attention_tree(ew.q, ew.k_pool, ew.v_pool, ew.block_table, ew.seq_lens, ew.query_start_loc,
                                 np.array([1, 0, 7], dtype=np.uint64), ew.scale, lib=lib)
    assert np.all(o[1] == 0.0) and np.all(np.isneginf(l[1])) and np.all(np.isfinite(l[[0, 2]]))


def _fp8_values(codes):
    """float64 values of E4M3 codes by torch's float8_e4m3fn (a library decode, not the oracle's)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def pin_fp8(lib=None):
    """FP8 E4M3 pages.  (1) the oracle's decode of all 256 codes equals torch's float8_e4m3fn
    (NaN codes included); (2) with power-of-two scales the dequantized pools are exact in float32
    and attention over the FP8 pages equals the (pinned) float32 attention over them; (3) with
    arbitrary scales it equals fp64 torch SDPA over K/V dequantized by torch and gathered by a
    Python page walk."""
    import torch
    dec = np.array([oracle.fp8_decode(c, lib=lib) for c in range(256)])
    ref = _fp8_values(np.arange(256))
    assert np.array_equal(np.isnan(dec), np.isnan(ref)) and np.array_equal(dec[~np.isnan(dec)], ref[~np.isnan(ref)])
    for seed, (B, maxlen, Hq, Hkv, D, maxq) in enumerate([(4, 150, 8, 2, 64, 5), (3, 90, 4, 1, 64, 30),
                                                          (3, 70, 8, 8, 128, 1)]):
        w8 = W.to_fp8(W.make_random(700 + seed, B, maxlen, Hq, Hkv, D, "bf16", max_q=maxq))
        ks, vs = w8.meta["k_scale"], w8.meta["v_scale"]
        p2 = lambda x: np.exp2(np.round(np.log2(x))).astype(np.float32)  # noqa: E731
        ks2, vs2 = p2(ks), p2(vs)
        args = (w8.block_table, w8.seq_lens, w8.query_start_loc, w8.scale)
        o8, l8 = oracle.attention_fp8(w8.q, w8.k_pool, w8.v_pool, ks2, vs2, *args, lib=lib)
        kf = (_fp8_values(w8.k_pool) * ks2[:, :, None, None]).astype(np.float32)
        vf = (_fp8_values(w8.v_pool) * vs2[:, :, None, None]).astype(np.float32)
        assert np.array_equal(kf[np.isfinite(kf)].astype(np.float64),
                              (_fp8_values(w8.k_pool) * ks2[:, :, None, None])[np.isfinite(kf)])  # exact in f32
        qf = W.bf16_bits_to_f32(w8.q)
        o32, l32 = oracle.attention(qf, kf, vf, *args, lib=lib)
        assert np.max(np.abs(o8 - o32)) <= 1e-13 and np.max(np.abs(l8 - l32)) <= 1e-13, seed
        o8, l8 = oracle.attention_fp8(w8.q, w8.k_pool, w8.v_pool, ks, vs, *args, lib=lib)
        K64 = _fp8_values(w8.k_pool) * ks.astype(np.float64)[:, :, None, None]
        V64 = _fp8_values(w8.v_pool) * vs.astype(np.float64)[:, :, None, None]
        G = Hq // Hkv
        q = torch.from_numpy(qf.astype(np.float64))
        for s in range(w8.num_seqs):
            n = int(w8.seq_lens[s])
            q0, q1 = int(w8.query_start_loc[s]), int(w8.query_start_loc[s + 1])
            if q1 == q0:
                continue
            win = q1 - q0
            pages = w8.block_table[s, np.arange(n) // PS]
            slots = np.arange(n) % PS
            K = K64[pages, :, slots, :].transpose(1, 0, 2)  # [Hkv][n][D]
            V = V64[pages, :, :, slots].transpose(1, 0, 2)
            Kt = torch.from_numpy(np.ascontiguousarray(K)).repeat_interleave(G, dim=0)
            Vt = torch.from_numpy(np.ascontiguousarray(V)).repeat_interleave(G, dim=0)
            Q = q[q0:q1].transpose(0, 1).contiguous()
            mask = torch.arange(n)[None, :] <= (n - win + torch.arange(win))[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(Q[None], Kt[None], Vt[None],
                                                                   attn_mask=mask[None, None], scale=w8.scale)[0]
            assert np.max(np.abs(o8[q0:q1] - ref.transpose(0, 1).numpy())) <= 1e-12, (seed, s)


ALL_PINS = [pin_brute_force, pin_golden, pin_closed_forms, pin_invariants, pin_merge_of_splits,
            pin_sdpa, pin_gather, pin_append, pin_tree, pin_fp8]
