"""Exact rational brute force of the gated delta rule (tiny inputs; test infrastructure).

This evaluates the matrix-product form of the recurrence as written for the
Gated DeltaNet layer that the FlashQLA pages accelerate (section on optimising
GDN chunked prefill):
    S_t = a_t * S_{t-1} @ (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t,
with S_t a d_v x d_k matrix (the "recurrent" orientation, not the transposed one
the other oracle forms use), explicit identity and outer-product matrices, and
Python ``Fraction`` arithmetic, so the result is exact when every input
(including the gate a_t itself, given directly rather than as log a_t) is
rational.
"""
from __future__ import annotations

from fractions import Fraction


def _mat(r, c):
    return [[Fraction(0)] * c for _ in range(r)]


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def gdn_exact_fraction(q, k, v, alpha, beta, scale, S0=None):
    """One sequence, one head, exact arithmetic.

    q, k: T lists of d_k rationals; v: T lists of d_v rationals; alpha, beta: T
    rationals (alpha is the gate itself, not its log); scale: rational;
    S0: None or a d_v x d_k nested list (recurrent orientation).
    Returns (o: T lists of d_v Fractions, S_T: d_v x d_k Fractions).
    """
    T = len(q)
    d_k = len(k[0]) if T else (len(S0[0]) if S0 else 0)
    d_v = len(v[0]) if T else (len(S0) if S0 else 0)
    S = _mat(d_v, d_k) if S0 is None else [[Fraction(x) for x in row] for row in S0]
    I = [[Fraction(int(i == j)) for j in range(d_k)] for i in range(d_k)]
    out = []
    for t in range(T):
        kt = [Fraction(x) for x in k[t]]
        a, b = Fraction(alpha[t]), Fraction(beta[t])
        kkT = [[kt[i] * kt[j] for j in range(d_k)] for i in range(d_k)]
        P = [[I[i][j] - b * kkT[i][j] for j in range(d_k)] for i in range(d_k)]
        SP = _matmul(S, P)
        vkT = [[Fraction(v[t][i]) * kt[j] for j in range(d_k)] for i in range(d_v)]
        S = [[a * SP[i][j] + b * vkT[i][j] for j in range(d_k)] for i in range(d_v)]
        qt = [[Fraction(x)] for x in q[t]]
        o = _matmul(S, qt)
        out.append([Fraction(scale) * o[i][0] for i in range(d_v)])
    return out, S
