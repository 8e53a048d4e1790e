"""Writes tests/golden/tiny_bruteforce.json from the 50-digit brute force.

The FlashAttention-4 pages print no worked numeric example, so the stored
values are not the pages'; they are produced here by oracle/brute.py only
(no GPU code, no C oracle) from bf16-exact inputs drawn with a fixed seed.
Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import brute  # noqa: E402


def bf16_grid(rng, shape):
    x = rng.standard_normal(shape)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def main():
    rng = np.random.default_rng(2024)
    cases = []
    for causal in (False, True):
        B, S, H, D = 1, 5, 2, 3
        q, k, v = (bf16_grid(rng, (B, S, H, D)) for _ in range(3))
        o, lse = brute.attention(q, k, v, 0.5, causal)
        cases.append({"B": B, "S": S, "H": H, "D": D, "scale": 0.5, "causal": causal,
                      "q": q.tolist(), "k": k.tolist(), "v": v.tolist(),
                      "o": o.tolist(), "lse": lse.tolist()})
    doc = {"source": "oracle/brute.py at %d digits (exp without max subtraction); "
                     "inputs are bf16-exact values from numpy seed 2024" % brute.DIGITS,
           "cases": cases}
    with open(os.path.join(HERE, "tiny_bruteforce.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
