"""Write the hand-derived worked examples under tests/golden/.

The pages print no numeric worked example, so every fixture here is a small
case whose answer follows from the definition by hand: the expected values
are closed forms (stated in each fixture's "derivation") evaluated with
mpmath at 50 digits.  This script does not call the oracle or the HIP
library; it is re-run only when a fixture is added.

    python tests/golden/make_golden.py
"""
import json
import os

import mpmath

mpmath.mp.dps = 50
HERE = os.path.dirname(os.path.abspath(__file__))


def s(x):
    return mpmath.nstr(mpmath.mpf(x), 30)


def write(name, d):
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")


# 1. One cached token: weight 1, out = V[0], lse = the logit 0.5*(q.k).
write("single_token.json", {
    "citation": "tinyvolt 'Kernel visualization: Flash Decoding', combine kernel: "
                "out = unnormalised sum / l; with one token l = exp(0) = 1",
    "derivation": "q.k = 1*0.5 + 2*0.25 + (-1)*1 + 3*1 = 3; logit = 0.5*3 = 1.5; "
                  "out = V[0]; lse = 1.5",
    "B": 1, "Hq": 1, "Hkv": 1, "T": 1, "D": 4, "scale": 0.5,
    "q": [[[1, 2, -1, 3]]],
    "k": [[[[0.5, 0.25, 1, 1]]]],
    "v": [[[[1.5, -2.25, 0, 7]]]],
    "expected_out": [[[s(1.5), s(-2.25), s(0), s(7)]]],
    "expected_lse": [[s(1.5)]],
    "tol": 1e-15,
})

# 2. Two tokens with logits 0 and 1: weights 1/(1+e) and e/(1+e).
e = mpmath.e
write("two_tokens_logistic.json", {
    "citation": "zenaique explainer, interview answer (softmax of the logits); "
                "closed form of a two-way softmax",
    "derivation": "logits 0 and 1; w0 = 1/(1+e), w1 = e/(1+e); out = w0*V0 + w1*V1 "
                  "= [e/(1+e), 1/(1+e)]; lse = ln(1+e)",
    "B": 1, "Hq": 1, "Hkv": 1, "T": 2, "D": 2, "scale": 1.0,
    "q": [[[1, 0]]],
    "k": [[[[0, 5], [1, -3]]]],
    "v": [[[[0, 1], [1, 0]]]],
    "expected_out": [[[s(e / (1 + e)), s(1 / (1 + e))]]],
    "expected_lse": [[s(mpmath.log(1 + e))]],
    "tol": 1e-15,
})

# 3. Logits ln1, ln2, ln3: weights 1/6, 2/6, 3/6.
write("weights_one_two_three.json", {
    "citation": "tinyvolt walkthrough (p = exp(logit - max), one division by l at "
                "the end); weights proportional to exp(logit)",
    "derivation": "D = 1, q = 1, scale = 1, K = [0, ln 2, ln 3] -> weights 1:2:3; "
                  "V = [6, 0, 2] and [0, 3, 1] -> out = [(6+0+6)/6, (0+6+3)/6] = [2, 1.5]; "
                  "lse = ln 6",
    "B": 1, "Hq": 1, "Hkv": 1, "T": 3, "D": 2, "scale": 1.0,
    "q": [[[1, 0]]],
    "k": [[[[0, 9], [float(mpmath.log(2)), -4], [float(mpmath.log(3)), 2]]]],
    "v": [[[[6, 0], [0, 3], [2, 1]]]],
    "expected_out": [[[s(2), s(1.5)]]],
    "expected_lse": [[s(mpmath.log(6))]],
    "tol": 1e-15,
})

# 4. GQA: query heads 0,1 read kv head 0, heads 2,3 read kv head 1.
write("gqa_head_groups.json", {
    "citation": "zenaique explainer, 'What decode looks like' (Q has n_heads, K/V "
                "have n_kv_heads); consecutive query heads share a kv head",
    "derivation": "K = 0 so every weight is 1/2: out = mean of the two value rows of "
                  "the head's kv head: kv0 rows [1],[3] -> 2, kv1 rows [10],[30] -> 20; "
                  "lse = ln 2",
    "B": 1, "Hq": 4, "Hkv": 2, "T": 2, "D": 1, "scale": 1.0,
    "q": [[[1], [2], [3], [4]]],
    "k": [[[[0], [0]], [[0], [0]]]],
    "v": [[[[1], [3]], [[10], [30]]]],
    "expected_out": [[[s(2)], [s(2)], [s(20)], [s(20)]]],
    "expected_lse": [[s(mpmath.log(2))] * 4],
    "tol": 1e-15,
})

# 5. Paged: two pages of 2 tokens, table reversed, length 3 (ends inside a page).
write("paged_reversed_table.json", {
    "citation": "dupenodi guide, 'Walking through it' (paged / ragged KV layouts); "
                "token t lives in page page_table[t / P] at row t % P",
    "derivation": "q = 0 -> uniform weights over the 3 valid tokens; table [1, 0]: "
                  "t0 -> page 1 row 0 = 3, t1 -> page 1 row 1 = 4, t2 -> page 0 row 0 = 1; "
                  "out = (3+4+1)/3 = 8/3; lse = ln 3",
    "B": 1, "Hq": 1, "Hkv": 1, "T": 4, "D": 1, "scale": 1.0,
    "page_size": 2,
    "q": [[[0]]],
    "k": [[[[5], [6]]], [[[7], [8]]]],
    "v": [[[[1], [2]]], [[[3], [4]]]],
    "page_table": [[1, 0]],
    "seq_lens": [3],
    "expected_out": [[[s(mpmath.mpf(8) / 3)]]],
    "expected_lse": [[s(mpmath.log(3))]],
    "tol": 1e-15,
})

print("wrote fixtures to", HERE)
