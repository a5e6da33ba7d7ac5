"""CPU tests: the fp64 oracle against its independent pins, and a mutation check
showing that each plausible mistake planted in the oracle's C source fails at
least one pin."""
import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle
import oracle_pins as P
from paged_kv_cache_gqa_amd import workloads as W


def test_oracle_brute_force():
    P.pin_brute_force()


def test_oracle_golden_worked_examples():
    P.pin_golden()


def test_oracle_closed_forms():
    P.pin_closed_forms()


def test_oracle_invariants():
    P.pin_invariants()


def test_oracle_merge_of_key_splits():
    P.pin_merge_of_splits()


def test_oracle_matches_torch_sdpa_fp64():
    P.pin_sdpa()


def test_oracle_append():
    P.pin_append()


def test_oracle_tree_masks():
    P.pin_tree()


def test_oracle_fp8_pages():
    P.pin_fp8()


def test_oracle_gather_page_walk():
    P.pin_gather()


def test_oracle_rejects_bad_content():
    w = W.make_random(5, 2, 30, 2, 1, 4, "f32", max_q=2)
    bad = w.block_table.copy()
    bad[0, 0] = w.num_pages  # page id out of range
    with pytest.raises(ValueError):
        oracle.attention(w.q, w.k_pool, w.v_pool, bad, w.seq_lens, w.query_start_loc, w.scale)
    qsl = w.query_start_loc.copy()
    sl = w.seq_lens.copy()
    sl[0] = int(qsl[1] - qsl[0]) - 1  # q_len > seq_len
    if qsl[1] > qsl[0]:
        with pytest.raises(ValueError):
            oracle.attention(w.q, w.k_pool, w.v_pool, w.block_table, sl, qsl, w.scale)


def test_oracle_empty_and_zero_query_sequences():
    # sequences with q_len = 0 produce no rows; an empty batch is legal
    w = W.build("zq", 9, [5, 40, 17], [0, 3, 0], 4, 2, 8, "f32", num_pages=8)
    o, l = oracle.attention_workload(w)
    assert o.shape == (3, 4, 8) and np.all(np.isfinite(o))
    e = W.build("empty", 9, [], [], 4, 2, 8, "f32", num_pages=1)
    o, l = oracle.attention_workload(e)
    assert o.shape == (0, 4, 8)


def test_generator_check_values():
    """Sequence-length draws of the five configurations (seed 1000 + c)."""
    expect = {2: 141622, 3: 600906, 4: 269344, 5: 2869412}
    for c, total in expect.items():
        n, ql, _ = W.config_lengths(c)
        assert int(n.sum()) == total
    n, _, _ = W.config_lengths(3)
    assert (n[:4] - 512).tolist() == [608, 384, 1194, 525]
    assert W.config_lengths(1)[0].tolist() == [17, 64, 100, 256]


def test_generator_deterministic_and_thread_independent():
    a = W.make_config(1)
    b = W.make_config(1)
    assert a.k_pool.tobytes() == b.k_pool.tobytes() and a.q.tobytes() == b.q.tobytes()
    x = W._draw_pool(7, 2, 2500, 64, "bf16", threads=1)
    y = W._draw_pool(7, 2, 2500, 64, "bf16", threads=4)
    assert x.tobytes() == y.tobytes()


# Planted mistakes: (description, text in pa_oracle.c, replacement).  All stay in bounds.
MUTATIONS = [
    ("causal limit off by one", "const int p = n - qn + i;", "const int p = n - qn + i - 1 + (i == 0);"),
    ("causal limit one too far", "const int p = n - qn + i;", "const int p = n - qn + i + (i + 1 < qn);"),
    ("GQA head map interleaved", "const int g = h / G;", "const int g = h % Hkv;"),
    ("V read with K's layout", "acc[d] += w * widen(v_pool, dtype, v_offset(pg, g, t, d, Hkv, D));",
     "acc[d] += w * widen(v_pool, dtype, k_offset(pg, g, t, d, Hkv, D));"),
    ("K read with V's layout", "widen(k_pool, dtype, k_offset(pg, g, t, d, Hkv, D));",
     "widen(k_pool, dtype, v_offset(pg, g, t, d, Hkv, D));"),
    ("slot order reversed", "const int t = j % ORACLE_PAGE;\n        double dot",
     "const int t = ORACLE_PAGE - 1 - j % ORACLE_PAGE;\n        double dot"),
    ("scale dropped", "x[j] = scale * dot;", "x[j] = dot;"),
    ("lse without the max", "lse[r * Hq + h] = m + log(l);", "lse[r * Hq + h] = log(l);"),
    ("no normalisation", "out[qoff + d] = acc[d] / l;", "out[qoff + d] = acc[d];"),
    ("softmax sign flipped", "const double w = exp(x[j] - m);", "const double w = exp(m - x[j]);"),
    ("query head taken as KV head", "widen(q, dtype, qoff + d)", "widen(q, dtype, (r * Hq + g) * (int64_t)D + d)"),
    ("merge weight w.r.t. the max", "v += exp(li - total) * o_parts", "v += exp(li - m) * o_parts"),
    ("append one position late", "const int p = n - q + i;", "const int p = n - q + i + (i + 1 < q);"),
    ("append V with K's layout", "memcpy((char*)v_pool + v_offset(pg, g, t, d, Hkv, D) * eb",
     "memcpy((char*)v_pool + k_offset(pg, g, t, d, Hkv, D) * eb"),
    ("append reads the wrong head", "const int64_t src = (r * Hkv + g) * D + d;",
     "const int64_t src = (r * Hkv + (Hkv - 1 - g)) * D + d;"),
    ("tree bit index off by one", "return (int)((mask >> (j - win0)) & 1u);", "return (int)((mask >> (j - win0 + 1)) & 1u);"),
    ("tree shows the first window token as context", "if (j < win0 || qn > 64) return 1;",
     "if (j <= win0 || qn > 64) return 1;"),
    ("tree always shows the row itself", "return (int)((mask >> (j - win0)) & 1u);",
     "return j == p ? 1 : (int)((mask >> (j - win0)) & 1u);"),
    ("tree masks applied to long windows", "if (j < win0 || qn > 64) return 1;", "if (j < win0) return 1;"),
    ("fp8 exponent bias off by one", "ldexp(1.0 + man / 8.0, ex - 7)", "ldexp(1.0 + man / 8.0, ex - 8)"),
    ("fp8 subnormals one binade low", "ldexp(man / 8.0, -6)", "ldexp(man / 8.0, -7)"),
    ("fp8 K scale of the wrong head", "const double ks = (double)k_scale[page * Hkv + kvh];",
     "const double ks = (double)k_scale[page * Hkv + (Hkv - 1 - kvh)];"),
    ("fp8 V scaled by the K scale", "const double vs = (double)v_scale[page * Hkv + kvh];",
     "const double vs = (double)k_scale[page * Hkv + kvh];"),
    ("page lookup off by one page", "const int64_t pg = bt[j / ORACLE_PAGE];\n        const int t = j % ORACLE_PAGE;\n        double",
     "const int64_t pg = bt[(j / ORACLE_PAGE + 1) % ((n + 15) / 16)];\n        const int t = j % ORACLE_PAGE;\n        double"),
]


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(desc, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        path = os.path.join(tmp, "mut.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.open_library(oracle.build(src=path, out=os.path.join(tmp, "libmut.so")))
        caught = []
        for pin in P.ALL_PINS:
            try:
                with np.errstate(all="ignore"):
                    pin(lib=lib)
            except (AssertionError, ValueError) as e:  # noqa: PERF203
                caught.append((pin.__name__, str(e)[:80]))
                break
        assert caught, f"no pin caught the planted mistake: {desc}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
