"""Write tests/golden/core_exact.json: exact-rational outputs of the core recurrence.

Calls only oracle.exact (fractions.Fraction; no rounding).  Run from the repo root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, os.path.dirname(HERE))

from oracle.exact import core_exact  # noqa: E402
from test_oracle_exact import rand_case  # noqa: E402  (input recipe only)


def main():
    cases = []
    for K, T, seed in [(2, 3, 11), (3, 4, 12), (4, 5, 13)]:
        alpha, beta, kn, qn, v, scale, S0 = rand_case(seed, K, T)
        out, S = core_exact(alpha, beta, kn, qn, v, scale, S0)
        s = lambda m: [[str(x) for x in r] for r in m]
        cases.append({"K": K, "T": T, "seed": seed, "alpha": s(alpha), "beta": [str(b) for b in beta],
                      "kn": s(kn), "qn": s(qn), "v": s(v), "scale": str(scale), "S0": s(S0),
                      "out": s(out), "S": s(S)})
    with open(os.path.join(HERE, "core_exact.json"), "w") as f:
        json.dump(cases, f, indent=1)


if __name__ == "__main__":
    main()
