"""Pin the oracle's core recurrence against exact rational arithmetic.

The core (decay, delta-rule write, inclusive read-out; FlashKDA article index,
"Delta Attention Algorithm: linear-time recurrence") is evaluated by
``oracle.exact.core_exact`` with ``fractions.Fraction`` -- no rounding at all --
on tiny K = V in {2, 3, 4} with rational unit keys and queries, and compared
with the C oracle's fp64 result.  A stored fixture (tests/golden, written by
tests/golden/make_golden.py, which calls only oracle/) guards the exact values.
"""
import json
import os
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.exact import core_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "core_exact.json")

# rational unit vectors (Pythagorean tuples), before sign flips and permutations
UNIT = {
    2: [(Fraction(3, 5), Fraction(4, 5)), (Fraction(5, 13), Fraction(12, 13)),
        (Fraction(8, 17), Fraction(15, 17)), (Fraction(1), Fraction(0))],
    3: [(Fraction(1, 3), Fraction(2, 3), Fraction(2, 3)), (Fraction(2, 7), Fraction(3, 7), Fraction(6, 7)),
        (Fraction(1), Fraction(0), Fraction(0)), (Fraction(4, 9), Fraction(4, 9), Fraction(7, 9))],
    4: [(Fraction(1, 2),) * 4, (Fraction(1, 3), Fraction(2, 3), Fraction(2, 3), Fraction(0)),
        (Fraction(2, 7), Fraction(3, 7), Fraction(6, 7), Fraction(0)), (Fraction(0), Fraction(1), Fraction(0), Fraction(0))],
}


def rand_unit(rng, K):
    base = list(rng.choice(UNIT[K]))
    rng.shuffle(base)
    return [x * rng.choice([1, -1]) for x in base]


def rand_case(seed, K, T):
    rng = random.Random(seed)
    alpha = [[Fraction(rng.randint(1, 8), 8) for _ in range(K)] for _ in range(T)]
    beta = [Fraction(rng.randint(0, 4), 4) for _ in range(T)]
    kn = [rand_unit(rng, K) for _ in range(T)]
    qn = [rand_unit(rng, K) for _ in range(T)]
    v = [[Fraction(rng.randint(-6, 6), 2) for _ in range(K)] for _ in range(T)]
    S0 = [[Fraction(rng.randint(-4, 4), 4) for _ in range(K)] for _ in range(K)]
    scale = Fraction(1, 2)
    return alpha, beta, kn, qn, v, scale, S0


def as_np(m):
    return np.array([[float(x) for x in row] for row in m], dtype=np.float64)


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("seed", range(6))
def test_core_matches_exact_rational(K, seed):
    T = 1 + seed % 6
    alpha, beta, kn, qn, v, scale, S0 = rand_case(1000 * K + seed, K, T)
    out_x, S_x = core_exact(alpha, beta, kn, qn, v, scale, S0)
    out, S = oracle.core(as_np(alpha), np.array([float(b) for b in beta]), as_np(kn), as_np(qn),
                         as_np(v), float(scale), as_np(S0))
    ox, sx = as_np(out_x), as_np(S_x)
    assert np.abs(out - ox).max() <= 1e-13 * max(1.0, np.abs(ox).max())
    assert np.abs(S - sx).max() <= 1e-13 * max(1.0, np.abs(sx).max())


def test_exact_core_hand_example():
    """One token, K = V = 2, worked by hand: alpha = (1/2, 1), beta = 1, k^ = (3/5, 4/5),
    q^ = (1, 0), v = (1, 2), S0 = I, scale = 1.
    decay: S = diag(1/2, 1); S k^ = (3/10, 4/5); r = v - S k^ = (7/10, 6/5);
    S += r k^T = [[1/2 + 21/50, 28/50], [18/25, 1 + 24/25]]; out = S q^ = (23/25, 18/25)."""
    out, S = core_exact([[Fraction(1, 2), 1]], [1], [[Fraction(3, 5), Fraction(4, 5)]], [[1, 0]],
                        [[1, 2]], 1, [[1, 0], [0, 1]])
    assert out == [[Fraction(23, 25), Fraction(18, 25)]]
    assert S == [[Fraction(23, 25), Fraction(14, 25)], [Fraction(18, 25), Fraction(49, 25)]]
    o2, S2 = oracle.core(np.array([[0.5, 1.0]]), np.array([1.0]), np.array([[0.6, 0.8]]),
                         np.array([[1.0, 0.0]]), np.array([[1.0, 2.0]]), 1.0, np.eye(2))
    assert np.allclose(o2, [[23 / 25, 18 / 25]], rtol=0, atol=1e-15)
    assert np.allclose(S2, [[23 / 25, 14 / 25], [18 / 25, 49 / 25]], rtol=0, atol=1e-15)


def test_golden_fixture():
    with open(GOLDEN) as f:
        cases = json.load(f)
    assert len(cases) >= 3
    for c in cases:
        F = lambda m: [[Fraction(x) for x in row] for row in m]
        alpha, kn, qn, v, S0 = F(c["alpha"]), F(c["kn"]), F(c["qn"]), F(c["v"]), F(c["S0"])
        beta = [Fraction(x) for x in c["beta"]]
        scale = Fraction(c["scale"])
        # the fixture is reproducible from oracle.exact ...
        out_x, S_x = core_exact(alpha, beta, kn, qn, v, scale, S0)
        assert [[str(x) for x in r] for r in out_x] == c["out"]
        assert [[str(x) for x in r] for r in S_x] == c["S"]
        # ... and the fp64 oracle reproduces it
        out, S = oracle.core(as_np(alpha), np.array([float(b) for b in beta]), as_np(kn), as_np(qn),
                             as_np(v), float(scale), as_np(S0))
        assert np.abs(out - as_np(F(c["out"]))).max() <= 1e-13
        assert np.abs(S - as_np(F(c["S"]))).max() <= 1e-13
