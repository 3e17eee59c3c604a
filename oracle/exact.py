"""Exact rational evaluation of the literal dense gated delta rule (oracle; test infrastructure only).

Evaluates, with ``fractions.Fraction``, the key-to-value orientation exactly as the rule
is usually written:

    S_t = S_{t-1} . A_t . (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = scale S_t q_t,

S_t of shape [dv, dk], A_t = alpha_t I (GDN) or diag(alpha_t) (KDA).  It forms the dense
dk x dk matrix (I - beta k k^T) and multiplies full matrices, so it shares no
rearrangement with ``delta_rule`` (which never builds that matrix and works on the
transposed, stored [dk, dv] layout).  Used only on tiny shapes by the pin tests.
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence

Matrix = List[List[Fraction]]


def _zeros(r, c) -> Matrix:
    return [[Fraction(0)] * c for _ in range(r)]


def _eye(n) -> Matrix:
    m = _zeros(n, n)
    for i in range(n):
        m[i][i] = Fraction(1)
    return m


def _matmul(a: Matrix, b: Matrix) -> Matrix:
    n, k, m = len(a), len(b), len(b[0])
    return [[sum((a[i][x] * b[x][j] for x in range(k)), Fraction(0)) for j in range(m)]
            for i in range(n)]


def _add(a: Matrix, b: Matrix) -> Matrix:
    return [[a[i][j] + b[i][j] for j in range(len(a[0]))] for i in range(len(a))]


def _scale(a: Matrix, s) -> Matrix:
    return [[x * s for x in row] for row in a]


def _outer(u: Sequence[Fraction], w: Sequence[Fraction]) -> Matrix:
    return [[x * y for y in w] for x in u]


def dense_step(S: Matrix, k, v, beta, alpha, kda: bool) -> Matrix:
    """One token on S [dv][dk] (key-to-value orientation), dense literal form."""
    dk = len(k)
    if kda:
        A = _zeros(dk, dk)
        for i in range(dk):
            A[i][i] = Fraction(alpha[i])
    else:
        A = _scale(_eye(dk), Fraction(alpha))
    P = _add(_eye(dk), _scale(_outer(k, k), -Fraction(beta)))
    return _add(_matmul(_matmul(S, A), P), _scale(_outer(v, k), Fraction(beta)))


def dense_output(S: Matrix, q, scale=Fraction(1)) -> List[Fraction]:
    return [Fraction(scale) * sum((S[i][j] * q[j] for j in range(len(q))), Fraction(0))
            for i in range(len(S))]


def run(S0: Matrix, tokens, kda: bool, scale=Fraction(1)):
    """tokens: list of (q, k, v, beta, alpha) with Fraction entries.  Returns (final S,
    outputs per token, each scaled by the query scale)."""
    S, outs = S0, []
    for (q, k, v, beta, alpha) in tokens:
        S = dense_step(S, k, v, beta, alpha, kda)
        outs.append(dense_output(S, q, scale))
    return S, outs
