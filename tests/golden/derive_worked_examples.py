"""Write worked_examples.json: small attention cases whose results have closed forms.

The pages print no numerical example, so these cases are built by hand so that
the softmax weights are known exactly (scores 0, 1, 2 give weights
proportional to 1, e, e^2; equal scores give a plain mean).  Each expected
value is the closed form written in ``derivation``, evaluated here with the
``decimal`` module at 40 significant digits.  Nothing here calls the oracle or
the GPU library.

Definition followed (XY-Serve verdict page, "key_machinery": the attention
primitive is matmul, then softmax, then matmul; "core_discovery": K/V sit in a
PagedAttention-style block cache): for query row i of a window of q tokens over
n keys, keys 0..n-q+i are visible, out = sum_j softmax(scale*q.k_j) v_j and
lse = ln sum_j exp(scale*q.k_j).

Run:  python tests/golden/derive_worked_examples.py
"""
import json
import os
from decimal import Decimal, getcontext

getcontext().prec = 40
E = Decimal(1).exp()


def s(x: Decimal) -> str:
    return format(x, ".30e")


def ln(x: Decimal) -> Decimal:
    return x.ln()


cases = []

# A: one decode row over three keys; scores 0, 1, 2 (q = e0, k_j = j e0, scale 1).
den = 1 + E + E * E
cases.append({
    "name": "three-keys-weights-1-e-e2",
    "dtype": ["f32", "bf16"],
    "num_q_heads": 1, "num_kv_heads": 1, "head_dim": 2, "scale": 1.0,
    "num_pages": 2,
    "sequences": [{"page_ids": [1], "keys": [[0, 0], [1, 0], [2, 0]],
                   "values": [[1, 0], [0, 1], [1, 1]],
                   "queries": [[[1, 0]]]}],
    "derivation": "weights (1, e, e^2)/(1+e+e^2); out = ((1+e^2), (e+e^2))/(1+e+e^2); lse = ln(1+e+e^2)",
    "out": [[[s((1 + E * E) / den), s((E + E * E) / den)]]],
    "lse": [[s(ln(den))]],
})

# B: a causal window of 3 rows over 5 keys (prior context 2) with equal scores (q = 0).
#    Row i sees keys 0..2+i; V_j = (j, 2j) -> out = ((2+i)/2, 2+i), lse = ln(3+i).
cases.append({
    "name": "causal-window-equal-scores",
    "dtype": ["f32", "bf16"],
    "num_q_heads": 1, "num_kv_heads": 1, "head_dim": 2, "scale": 0.5,
    "num_pages": 3,
    "sequences": [{"page_ids": [2], "keys": [[1, -1], [2, 3], [-4, 5], [6, 7], [8, -9]],
                   "values": [[j, 2 * j] for j in range(5)],
                   "queries": [[[0, 0]], [[0, 0]], [[0, 0]]]}],
    "derivation": "q = 0 gives equal weights over keys 0..2+i: out = mean(V_0..V_{2+i}) = ((2+i)/2, 2+i); lse = ln(3+i)",
    "out": [[[s(Decimal(2 + i) / 2), s(Decimal(2 + i))]] for i in range(3)],
    "lse": [[s(ln(Decimal(3 + i)))] for i in range(3)],
})

# C: GQA, two query heads sharing one KV head, keys spanning two pages (18 keys, page ids 4 then 0).
#    Keys 0..16 are zero, key 17 = (1, 2); head 0 q = (1, 0) -> score of key 17 is 1, others 0;
#    head 1 q = (0, 1) -> score 2.  V_17 = (0, 1), other V rows = (1, 0).
#    head 0: weights 1 (x17) and e -> out = (17, e)/(17+e), lse = ln(17+e)
#    head 1: out = (17, e^2)/(17+e^2), lse = ln(17+e^2)
keys = [[0, 0]] * 17 + [[1, 2]]
vals = [[1, 0]] * 17 + [[0, 1]]
cases.append({
    "name": "gqa-two-heads-two-pages",
    "dtype": ["f32", "bf16"],
    "num_q_heads": 2, "num_kv_heads": 1, "head_dim": 2, "scale": 1.0,
    "num_pages": 5,
    "sequences": [{"page_ids": [4, 0], "keys": keys, "values": vals,
                   "queries": [[[1, 0], [0, 1]]]}],
    "derivation": "head 0: out = (17, e)/(17+e), lse = ln(17+e); head 1: out = (17, e^2)/(17+e^2), lse = ln(17+e^2)",
    "out": [[[s(Decimal(17) / (17 + E)), s(E / (17 + E))],
             [s(Decimal(17) / (17 + E * E)), s(E * E / (17 + E * E))]]],
    "lse": [[s(ln(17 + E)), s(ln(17 + E * E))]],
})

# D: two sequences in one batch, the second with two KV heads mapped to four query heads.
#    Sequence 0: one key, so out = V_0 and lse = scale * q.k_0 = 0.5 * (3*2 + 1*(-1)) = 2.5.
#    Sequence 1 (2 query heads per KV head): one query over 2 keys with scores 0 and 0
#    for KV head 0 (q = 0), and scores (0, 4) for KV head 1 -> weights 1, e^4 (scale 0.5, q.k = 8).
cases.append({
    "name": "batch-single-key-and-gqa-pairs",
    "dtype": ["f32", "bf16"],
    "num_q_heads": 4, "num_kv_heads": 2, "head_dim": 2, "scale": 0.5,
    "num_pages": 4,
    "sequences": [
        {"page_ids": [3], "keys": [[[2, -1], [2, -1]]], "values": [[[5, -7], [5, -7]]],
         "queries": [[[3, 1], [3, 1], [3, 1], [3, 1]]], "per_head": True},
        {"page_ids": [1], "keys": [[[1, 1], [0, 0]], [[1, 1], [4, 4]]],
         "values": [[[1, 2], [3, 4]], [[-1, -2], [-3, -4]]],
         "queries": [[[0, 0], [0, 0], [1, 1], [1, 1]]], "per_head": True},
    ],
    "derivation": "seq 0: a single key, so every head returns V_0 = (5, -7) with lse = 0.5*(3*2 + 1*(-1)) = 2.5; "
                  "seq 1, KV head 0 (query heads 0 and 1, q = 0): equal weights over V rows (1, 2) and (-1, -2) "
                  "give out = (0, 0), lse = ln 2; KV head 1 (query heads 2 and 3, q = (1, 1)): keys (0, 0) and "
                  "(4, 4) score 0 and 0.5*8 = 4, V rows (3, 4) and (-3, -4) give "
                  "out = (3 - 3e^4, 4 - 4e^4)/(1 + e^4), lse = ln(1 + e^4)",
    "out": [
        [[s(Decimal(5)), s(Decimal(-7))]] * 4,
        [[s(Decimal(0)), s(Decimal(0))], [s(Decimal(0)), s(Decimal(0))],
         [s((Decimal(3) + Decimal(-3) * E ** 4) / (1 + E ** 4)), s((Decimal(4) + Decimal(-4) * E ** 4) / (1 + E ** 4))],
         [s((Decimal(3) + Decimal(-3) * E ** 4) / (1 + E ** 4)), s((Decimal(4) + Decimal(-4) * E ** 4) / (1 + E ** 4))]],
    ],
    "lse": [[s(Decimal("2.5"))] * 4,
            [s(ln(Decimal(2))), s(ln(Decimal(2))), s(ln(1 + E ** 4)), s(ln(1 + E ** 4))]],
})
doc = {
    "about": "Hand-built paged attention cases with closed-form results (no printed example exists on "
             "the source pages). Keys/values are listed in logical order; 'page_ids' places them 16 per "
             "page. Unless 'per_head' is set, keys/values are [key][d] for the single KV head; with "
             "'per_head' they are [key][kv_head][d]. queries are [token][q_head][d]. Every page slot not "
             "listed is filled with NaN by the test. K pool layout [page][kv_head][slot][d]; V pool "
             "layout [page][kv_head][d][slot].",
    "source": "closed forms of softmax attention; definition per the XY-Serve verdict page "
              "(pith_extraction.key_machinery, core_discovery)",
    "cases": cases,
}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_examples.json")
with open(path, "w") as f:
    json.dump(doc, f, indent=1)
print("wrote", path)
