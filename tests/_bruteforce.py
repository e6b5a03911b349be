"""Exact rational recurrence for tiny cases (test helper, pins the oracle).

It evaluates the gated delta rule in its literal matrix form with Python
fractions:  M_t = a_t (I - beta_t k_t k_t^T)  (a dk x dk transition matrix),
S_t = S_{t-1} M_t + beta_t v_t k_t^T,  o_t = S_t q_t.  This association
differs from the oracle's row-wise expansion, and every product is exact.
"""
from fractions import Fraction


def frac(x):
    return Fraction(x)


def matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][j] * B[j][c] for j in range(m)), Fraction(0)) for c in range(p)]
            for i in range(n)]


def recurrence(S0, a, beta, k, v, q):
    """S0: dv x dk; a, beta: [T]; k, q: [T][dk]; v: [T][dv].
    Returns (list of states S_1..S_T, list of outputs o_1..o_T)."""
    dv, dk = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    states, outs = [], []
    for t in range(len(a)):
        M = [[a[t] * ((1 if i == j else 0) - beta[t] * k[t][i] * k[t][j]) for j in range(dk)]
             for i in range(dk)]
        SM = matmul(S, M)
        S = [[SM[i][j] + beta[t] * v[t][i] * k[t][j] for j in range(dk)] for i in range(dv)]
        o = [sum((S[i][j] * q[t][j] for j in range(dk)), Fraction(0)) for i in range(dv)]
        states.append([r[:] for r in S])
        outs.append(o)
    return states, outs
