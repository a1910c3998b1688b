"""Exact-rational brute force of the KDA core recurrence -- TEST INFRASTRUCTURE ONLY.

Steps 4-7 of the token recurrence (decay, delta-rule write, inclusive read-out),
evaluated with ``fractions.Fraction`` so that no rounding happens at all.  It
takes already-activated inputs (alpha, beta, unit keys/queries as rationals),
which is what the FlashKDA article index page calls the "linear-time
recurrence replacing quadratic softmax attention"; the per-token order
(decay first, then the write, then the read-out) is the reading stated in
``kda_ref.c``.
"""
from __future__ import annotations

from fractions import Fraction


def core_exact(alpha, beta, kn, qn, v, scale, S0):
    """alpha, kn, qn: T x K; beta: T; v: T x V; S0: V x K (nested lists of Fractions/ints).

    Returns (out T x V, S V x K) as nested lists of Fractions.
    """
    T = len(alpha)
    V = len(S0)
    K = len(S0[0]) if V else 0
    S = [[Fraction(x) for x in row] for row in S0]
    out = []
    scale = Fraction(scale)
    for t in range(T):
        for i in range(V):
            for c in range(K):
                S[i][c] = S[i][c] * Fraction(alpha[t][c])
        for i in range(V):
            pred = sum((S[i][c] * Fraction(kn[t][c]) for c in range(K)), Fraction(0))
            r = Fraction(v[t][i]) - pred
            for c in range(K):
                S[i][c] = S[i][c] + Fraction(beta[t]) * r * Fraction(kn[t][c])
        out.append([scale * sum((S[i][c] * Fraction(qn[t][c]) for c in range(K)), Fraction(0))
                    for i in range(V)])
    return out, S
