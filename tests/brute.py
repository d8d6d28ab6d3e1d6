"""Exact brute force for tiny heads, in rational arithmetic.

Uses the matrix form of one token of the gated delta rule with per-channel decay,
    S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T ,   o_t = S_t^T q ,
which is algebraically equal to the column-wise update the oracle performs
(decay, u = S^T k, S += beta k (v - u)^T) but reaches it by a different route:
an explicit dk x dk projector applied to the decayed state. Every binary float
is a dyadic rational, so ``Fraction(x)`` is exact and the result carries no
rounding at all.
"""

from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence, Tuple


def _F(x) -> Fraction:
    return Fraction(float(x)) if not isinstance(x, Fraction) else x


def brute_run(S0, tokens: Sequence[Tuple]) -> Tuple[List, List]:
    """S0: dk x dv nested sequence (row i = key channel). tokens: (q, k, v, alpha, beta)
    per token, q may be None. Returns (states after each token, outputs after each token)
    as nested lists of Fractions."""
    S = [[_F(x) for x in row] for row in S0]
    dk = len(S)
    dv = len(S[0]) if dk else 0
    states, outs = [], []
    for (q, k, v, alpha, beta) in tokens:
        k = [_F(x) for x in k]
        v = [_F(x) for x in v]
        a = [_F(x) for x in alpha]
        b = _F(beta)
        D = [[a[i] * S[i][j] for j in range(dv)] for i in range(dk)]
        P = [[(Fraction(1) if i == l else Fraction(0)) - b * k[i] * k[l] for l in range(dk)]
             for i in range(dk)]
        S = [[sum((P[i][l] * D[l][j] for l in range(dk)), Fraction(0)) + b * k[i] * v[j]
              for j in range(dv)] for i in range(dk)]
        states.append([row[:] for row in S])
        if q is not None:
            qq = [_F(x) for x in q]
            outs.append([sum((S[i][j] * qq[i] for i in range(dk)), Fraction(0)) for j in range(dv)])
        else:
            outs.append(None)
    return states, outs


def to_float(m):
    """Nested Fractions -> nested floats (correctly rounded to double)."""
    if isinstance(m, Fraction):
        return float(m)
    return [to_float(x) for x in m]
