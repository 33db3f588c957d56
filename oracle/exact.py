"""Exact rational evaluation of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

The recurrence (pages "Optimizing on-device inference for Apple Silicon",
section "Qwen creates three distinct workload shapes": a gate keeps part of the
state, a delta update writes the current token, tokens are processed in order):

    S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,    o_t = S_t q_t

Here the retention a_t is given directly as a rational number (the floating
point oracle receives g_t = log a_t).  Every quantity is a ``fractions.Fraction``,
so the result has no rounding at all; it is used to write the golden fixtures
under tests/golden/ that pin the floating point oracle.  Plain nested lists,
explicit loops, the formula exactly as written above (matrix products spelled
out).  Tiny sizes only.
"""
from fractions import Fraction


def _matmul(X, Y):
    n, m, p = len(X), len(Y), len(Y[0])
    return [[sum((X[i][l] * Y[l][j] for l in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def _outer(x, y):
    return [[xi * yj for yj in y] for xi in x]


def scan(q, k, v, a, beta, S0=None):
    """q, k: T lists of dk Fractions; v: T lists of dv Fractions; a, beta: T
    Fractions; S0: dv x dk Fractions or None.  Returns (o: T lists of dv, S_T)."""
    T = len(q)
    dk = len(k[0])
    dv = len(v[0])
    S = [[Fraction(0)] * dk for _ in range(dv)] if S0 is None else [list(r) for r in S0]
    outs = []
    for t in range(T):
        kk = _outer(k[t], k[t])
        M = [[(Fraction(1) if i == j else Fraction(0)) - beta[t] * kk[i][j] for j in range(dk)]
             for i in range(dk)]
        SM = _matmul(S, M)
        vk = _outer(v[t], k[t])
        S = [[a[t] * SM[i][j] + beta[t] * vk[i][j] for j in range(dk)] for i in range(dv)]
        outs.append([sum((S[i][j] * q[t][j] for j in range(dk)), Fraction(0)) for i in range(dv)])
    return outs, S
