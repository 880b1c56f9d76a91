"""Writes four_token_case.json: a 4-token attention case with hand-derived
closed-form outputs.

The case is built so that every input is exact in bfloat16 and the logits
are small integers:  N = 4 tokens, one image, one head, scale = 1/8,
Q[i][0] = i, K[l][0] = 8 l, V[l][0] = l, V[l][1] = 1, all other entries 0.
Then S[i][l] = (1/8) * i * 8 l = i l, so row i of the softmax is
P[i][l] = e^(i l) / sum_k e^(i k), and
    O[i][0] = sum_l l e^(i l) / sum_l e^(i l),  O[i][1] = 1,  O[i][d >= 2] = 0.

The values below are these closed forms evaluated with Python's decimal
module at 40 significant digits.  This script uses neither the oracle nor
the GPU library: it is an independent evaluation of the definition of
softmax attention on a case small enough to do by hand.
"""
import json
import os
from decimal import Decimal, getcontext

getcontext().prec = 40


def row(i):
    e = [Decimal(i * l).exp() for l in range(4)]
    z = sum(e)
    p = [x / z for x in e]
    o0 = sum(Decimal(l) * p[l] for l in range(4))
    return p, o0


def main():
    rows = [row(i) for i in range(4)]
    case = {
        "what": "4-token softmax attention with closed-form outputs",
        "derivation": __doc__,
        "N": 4, "B": 1, "H": 1, "scale": 0.125,
        "q_col0": [0, 1, 2, 3],
        "k_col0": [0, 8, 16, 24],
        "v_col0": [0, 1, 2, 3],
        "v_col1": [1, 1, 1, 1],
        "expected_o_col0": [float(r[1]) for r in rows],
        "expected_o_col1": [1.0, 1.0, 1.0, 1.0],
        "expected_p": [[float(x) for x in r[0]] for r in rows],
    }
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "four_token_case.json")
    with open(out, "w") as f:
        json.dump(case, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
