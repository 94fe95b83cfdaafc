"""Write the exact-rational golden fixtures of tests/golden/.

Calls only ``oracle.brute`` (exact rational arithmetic); the fixture holds the
inputs and the exact outputs of the KDA recurrence as fraction strings.  The
recurrence is the matrix form of the miniKimiK3 card's Kimi Delta Attention
bullet ("Architecture" section).  Run from the repository root:

    python tests/golden/make_golden.py
"""

import json
import os
import sys
from fractions import Fraction

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.brute import brute_force  # noqa: E402


def fr(x):
    return str(Fraction(x))


def case_worked():
    """A hand-sized worked example: d_k = d_v = 2, three tokens.

    Token 0 writes v_0 under the unit key e_1 (beta = 1: exact replacement),
    token 1 decays channel 2 by 1/2 and writes with a (3/5, 4/5) unit key at
    beta = 1/2, token 2 decays both channels and writes with key e_2.
    """
    q = [[1, 0], [Fraction(3, 5), Fraction(4, 5)], [0, 1]]
    k = [[1, 0], [Fraction(3, 5), Fraction(4, 5)], [0, 1]]
    v = [[2, -1], [1, 1], [Fraction(1, 2), 3]]
    alpha = [[1, 1], [1, Fraction(1, 2)], [Fraction(3, 4), Fraction(1, 4)]]
    beta = [1, Fraction(1, 2), Fraction(3, 4)]
    S0 = [[Fraction(1, 2), 0], [0, -1]]
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)


def case_random(seed, T=5, dk=3, dv=2):
    import random
    r = random.Random(seed)
    F = lambda lo, hi, den: Fraction(r.randint(lo, hi), den)
    return dict(
        q=[[F(-4, 4, 4) for _ in range(dk)] for _ in range(T)],
        k=[[F(-5, 5, 5) for _ in range(dk)] for _ in range(T)],
        v=[[F(-6, 6, 3) for _ in range(dv)] for _ in range(T)],
        alpha=[[F(1, 8, 8) for _ in range(dk)] for _ in range(T)],
        beta=[F(0, 4, 4) for _ in range(T)],
        S0=[[F(-3, 3, 2) for _ in range(dv)] for _ in range(dk)],
    )


def dump(case, path, note):
    o, states = brute_force(case["q"], case["k"], case["v"], case["alpha"], case["beta"], case["S0"])
    enc = lambda m: [[fr(x) for x in row] for row in m]
    out = dict(
        note=note,
        q=enc(case["q"]), k=enc(case["k"]), v=enc(case["v"]), alpha=enc(case["alpha"]),
        beta=[fr(b) for b in case["beta"]], S0=enc(case["S0"]),
        o=enc(o), S_final=enc(states[-1]),
    )
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    here = os.path.dirname(os.path.abspath(__file__))
    dump(case_worked(), os.path.join(here, "worked_d2_t3.json"),
         "exact KDA recurrence, hand-sized worked example (matrix form of the miniKimiK3 KDA bullet)")
    dump(case_random(20260), os.path.join(here, "rational_d3_t5.json"),
         "exact KDA recurrence on random rationals (matrix form of the miniKimiK3 KDA bullet)")
    print("wrote golden fixtures")
