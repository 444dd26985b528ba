"""Exact rational brute force for tiny decode problems (an oracle pin).

It evaluates the recurrence in its product form with explicit matrices, in
``fractions.Fraction`` arithmetic, so no rounding enters. For the gated delta
rule and KDA, one token is

    S_t = S_{t-1} D_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t,

with D_t = alpha_t I (GDN) or diag(e_t) (KDA), and S the V x K storage tile.
This is the matrix form of "decay by exp(g_t), then add
beta_t k_t (x) (v_t - S^T k_t); output S^T q_t" in the aiter KDA decode page
(advisory review, summary paragraph), written with the state as stored
(V rows, K contiguous). For Lightning, S_t = lambda S_{t-1} + v_t k_t^T.

It shares no code with the fp64 oracle: different formulation (matrix
products instead of row loops), different arithmetic (exact rationals).
"""
from __future__ import annotations

from fractions import Fraction as F


def _zeros(r, c):
    return [[F(0)] * c for _ in range(r)]


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    assert len(A[0]) == m
    return [[sum((A[i][l] * B[l][j] for l in range(m)), F(0))
             for j in range(p)] for i in range(n)]


def _add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def _scale(A, s):
    return [[a * s for a in row] for row in A]


def _outer(x, y):
    return [[a * b for b in y] for a in x]


def _identity(n):
    return [[F(int(i == j)) for j in range(n)] for i in range(n)]


def _matvec(A, x):
    return [sum((a * b for a, b in zip(row, x)), F(0)) for row in A]


def run(variant, S0, tokens):
    """variant: 'lightning' | 'gdn' | 'kda'.

    S0: V x K list of Fractions. tokens: list of dicts with q, k (length K),
    v (length V) and, for gdn, 'alpha' (Fraction) and 'beta'; for kda,
    'e' (length K) and 'beta'; for lightning, 'lam'.
    Returns (outputs per token, states per token)."""
    S = [row[:] for row in S0]
    K = len(S0[0])
    outs, states = [], []
    for tok in tokens:
        q, k, v = tok["q"], tok["k"], tok["v"]
        if variant == "lightning":
            S = _add(_scale(S, tok["lam"]), _outer(v, k))
        else:
            if variant == "gdn":
                D = _scale(_identity(K), tok["alpha"])
            else:
                D = _zeros(K, K)
                for j in range(K):
                    D[j][j] = tok["e"][j]
            b = tok["beta"]
            P = _add(_identity(K), _scale(_outer(k, k), -b))
            S = _add(_matmul(_matmul(S, D), P), _scale(_outer(v, k), b))
        outs.append(_matvec(S, q))
        states.append([row[:] for row in S])
    return outs, states
