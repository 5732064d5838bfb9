"""Writes hand_worked.json: tiny attention cases whose outputs are closed forms.

The pages print no numeric worked example, so these cases are derived by hand
from the definition (scores, row max, exp, normalise, P V; LSE = ln of the
normaliser of the scaled scores).  The expected values below are those closed
forms evaluated with Python's math module; nothing here runs the oracle or the
GPU path.  Run: ``python tests/golden/make_hand_worked.py``.
"""
import json
import math
import os

e = math.e
CASES = [
    {
        "name": "two_by_two",
        "cite": "Scaled-dot-product attention definition: 'standard attention' equation block of "
                "the 'FlashAttention 1-4 explained' post; compute chain of section 1.1 of the "
                "FlashAttention V4 explainer.",
        "derivation": "scale=1. S = Q K^T: row 0 = [1, 0]; row 1 = [0, 0]. Non-causal: "
                      "P0 = [e, 1]/(e+1), P1 = [1/2, 1/2]. O0 = [2e/(e+1), 4/(e+1)], O1 = [1, 2]. "
                      "LSE0 = ln(e+1), LSE1 = ln 2. Causal: row 0 sees key 0 only, so O0 = V0 = "
                      "[2, 0] and LSE0 = S00 = 1; row 1 is unchanged.",
        "d": 2, "scale": 1.0,
        "q": [[1, 0], [0, 1]], "k": [[1, 0], [0, 0]], "v": [[2, 0], [0, 4]],
        "noncausal": {"o": [[2 * e / (e + 1), 4 / (e + 1)], [1.0, 2.0]],
                      "lse": [math.log(e + 1), math.log(2)]},
        "causal": {"o": [[2.0, 0.0], [1.0, 2.0]], "lse": [1.0, math.log(2)]},
    },
    {
        "name": "three_keys_one_dim",
        "cite": "Same definition; an explicit scale of 0.5 replaces 1/sqrt(d) so that the scores "
                "are small integers.",
        "derivation": "d=1, scale=0.5, every query is 2 and the keys are [0, 1, 2], so every score "
                      "row is [0, 1, 2]. Non-causal: P = [1, e, e^2]/(1+e+e^2); with V = [1, 2, 3], "
                      "O = (1+2e+3e^2)/(1+e+e^2) and LSE = ln(1+e+e^2). Causal: row 0 sees [0]: "
                      "O = 1, LSE = 0; row 1 sees [0, 1]: O = (1+2e)/(1+e), LSE = ln(1+e); row 2 "
                      "is the full row.",
        "d": 1, "scale": 0.5,
        "q": [[2], [2], [2]], "k": [[0], [1], [2]], "v": [[1], [2], [3]],
        "noncausal": {"o": [[(1 + 2 * e + 3 * e * e) / (1 + e + e * e)]] * 3,
                      "lse": [math.log(1 + e + e * e)] * 3},
        "causal": {"o": [[1.0], [(1 + 2 * e) / (1 + e)], [(1 + 2 * e + 3 * e * e) / (1 + e + e * e)]],
                   "lse": [0.0, math.log(1 + e), math.log(1 + e + e * e)]},
    },
    {
        "name": "dominant_key",
        "cite": "Same definition; subtracting the row max (step 2 of the section 1.1 compute chain) "
                "keeps exp finite when one score dominates.",
        "derivation": "d=1, scale=1, every query is 64 and the keys are [-64, 64, 0], so the scores "
                      "are [-4096, 4096, 0]. exp(-8192) and exp(-4096) underflow to 0 in double, so "
                      "P = [0, 1, 0] exactly: O = V1 = 5 and LSE = 4096. Causal row 0 sees only "
                      "key 0: O = 3, LSE = -4096. Without the max subtraction exp overflows.",
        "d": 1, "scale": 1.0,
        "q": [[64], [64], [64]], "k": [[-64], [64], [0]], "v": [[3], [5], [7]],
        "noncausal": {"o": [[5.0], [5.0], [5.0]], "lse": [4096.0, 4096.0, 4096.0]},
        "causal": {"o": [[3.0], [5.0], [5.0]], "lse": [-4096.0, 4096.0, 4096.0]},
    },
]

if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_worked.json")
    with open(out, "w") as f:
        json.dump({"source": "hand-worked closed forms; the pages print no numeric worked example",
                   "cases": CASES}, f, indent=1)
    print("wrote", out)
