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


class Dual:
    """a + b eps with eps^2 = 0, over Fractions: exact forward-mode derivatives of a
    polynomial computation."""
    __slots__ = ("a", "b")

    def __init__(self, a, b=0):
        self.a = Fraction(a)
        self.b = Fraction(b)

    def _c(self, o):
        return o if isinstance(o, Dual) else Dual(o)

    def __add__(self, o):
        o = self._c(o)
        return Dual(self.a + o.a, self.b + o.b)

    __radd__ = __add__

    def __sub__(self, o):
        o = self._c(o)
        return Dual(self.a - o.a, self.b - o.b)

    def __rsub__(self, o):
        return self._c(o) - self

    def __mul__(self, o):
        o = self._c(o)
        return Dual(self.a * o.a, self.a * o.b + self.b * o.a)

    __rmul__ = __mul__


def core_exact_jvp(alpha, beta, kn, qn, v, scale, S0, tangents):
    """The core recurrence (as core_exact) on dual numbers: every input x carries the tangent
    tangents[name] (same nesting as the input; names alpha, beta, kn, qn, v, S0).  Returns
    (out, S) as nested lists of Dual; the .b parts are the exact directional derivatives."""
    def lift(x, dx):
        if isinstance(x, list):
            return [lift(a, b) for a, b in zip(x, dx)]
        return Dual(x, dx)

    A = lift(alpha, tangents["alpha"])
    Bt = lift(beta, tangents["beta"])
    Kn = lift(kn, tangents["kn"])
    Qn = lift(qn, tangents["qn"])
    Vv = lift(v, tangents["v"])
    S = lift(S0, tangents["S0"])
    T, Vd, K = len(alpha), len(S0), len(S0[0])
    out = []
    for t in range(T):
        for i in range(Vd):
            for c in range(K):
                S[i][c] = S[i][c] * A[t][c]
        for i in range(Vd):
            pred = Dual(0)
            for c in range(K):
                pred = pred + S[i][c] * Kn[t][c]
            r = Vv[t][i] - pred
            for c in range(K):
                S[i][c] = S[i][c] + Bt[t] * r * Kn[t][c]
        row = []
        for i in range(Vd):
            acc = Dual(0)
            for c in range(K):
                acc = acc + S[i][c] * Qn[t][c]
            row.append(acc * scale)
        out.append(row)
    return out, S
