"""Exact-rational brute force of the KDA recurrence (tiny inputs only).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Builds each token's transition matrix explicitly,

    M_t = (I - beta_t k_t k_t^T) Diag(alpha_t),

and evaluates the state as the closed product/sum

    S_t = M_t ... M_1 S_0 + sum_{s<=t} M_t ... M_{s+1} beta_s k_s v_s^T,
    o_t = S_t^T q_t,

with Python Fractions, so there is no rounding at all. This is the gated
delta rule with per-channel diagonal decay written as matrices (the pages
describe the delta rule as a correction of the value-retrieval error and KDA's
forgetting factor as a diagonal matrix: Kimi K3 report, "Methodology notes").
It shares no code with the fp64 recurrence and uses a different association
(products of explicit matrices instead of a rank-1 update).
"""

from __future__ import annotations

from fractions import Fraction


def _mat(rows, cols, val=Fraction(0)):
    return [[val for _ in range(cols)] for _ in range(rows)]


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def _add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def transition(alpha, beta, k):
    """M = (I - beta k k^T) Diag(alpha) as an explicit Dk x Dk matrix."""
    D = len(k)
    M = _mat(D, D)
    for i in range(D):
        for j in range(D):
            ident = Fraction(1) if i == j else Fraction(0)
            M[i][j] = (ident - beta * k[i] * k[j]) * alpha[j]
    return M


def run(q, k, v, alpha, beta, S0):
    """All arguments are nested lists of Fractions:
    q, k [T][Dk], v [T][Dv], alpha [T][Dk], beta [T], S0 [Dk][Dv].
    Returns (o [T][Dv], states [T][Dk][Dv]) where states[t] = S_t."""
    T = len(k)
    Dk, Dv = len(S0), len(S0[0])
    Ms = [transition(alpha[t], beta[t], k[t]) for t in range(T)]
    outs, states = [], []
    for t in range(T):
        # prod = M_t ... M_1
        prod = [[Fraction(int(i == j)) for j in range(Dk)] for i in range(Dk)]
        for s in range(t + 1):
            prod = _matmul(Ms[s], prod)
        S = _matmul(prod, S0)
        for s in range(t + 1):
            tail = [[Fraction(int(i == j)) for j in range(Dk)] for i in range(Dk)]
            for r in range(s + 1, t + 1):
                tail = _matmul(Ms[r], tail)
            kv = [[beta[s] * k[s][i] * v[s][j] for j in range(Dv)] for i in range(Dk)]
            S = _add(S, _matmul(tail, kv))
        o = [sum((S[i][j] * q[t][i] for i in range(Dk)), Fraction(0)) for j in range(Dv)]
        outs.append(o)
        states.append(S)
    return outs, states
