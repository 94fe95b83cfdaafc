"""Exact-rational brute force of the KDA recurrence on tiny inputs.

TEST INFRASTRUCTURE ONLY (same rule as ``kda_oracle``): used to pin the fp64
oracle and to write the golden fixtures under ``tests/golden/``.

This is a different formulation of the same method, written from the matrix
form of the KDA update (miniKimiK3 card, "Architecture" section, the Kimi
Delta Attention bullet; matrix form S_t = M_t S_{t-1} + beta_t k_t v_t^T with
M_t = (I - beta_t k_t k_t^T) Diag(alpha_t)).  Instead of stepping a state, the
state after every token t is recomputed from scratch by unrolling:

    S_t = Phi(t, 0) S_0 + sum_{i <= t} Phi(t, i) beta_i k_i v_i^T,
    Phi(t, i) = M_t M_{t-1} ... M_{i+1}   (Phi(t, t) = I)

and o_t = S_t^T q_t.  Everything is Python ``fractions.Fraction``: no
rounding anywhere, so the result is the exact value of the recurrence for
rational alpha, beta, q, k, v, S_0.
"""

from fractions import Fraction

__all__ = ["brute_force"]


def _zeros(r, c):
    return [[Fraction(0)] * c for _ in range(r)]


def _eye(n):
    m = _zeros(n, n)
    for i in range(n):
        m[i][i] = Fraction(1)
    return m


def _matmul(a, b):
    r, n, c = len(a), len(b), len(b[0])
    out = _zeros(r, c)
    for i in range(r):
        for j in range(c):
            s = Fraction(0)
            for t in range(n):
                s += a[i][t] * b[t][j]
            out[i][j] = s
    return out


def _add(a, b):
    return [[x + y for x, y in zip(ra, rb)] for ra, rb in zip(a, b)]


def _transition(alpha, beta, k):
    """M = (I - beta k k^T) Diag(alpha) as an exact d_k x d_k matrix."""
    dk = len(k)
    m = _zeros(dk, dk)
    for i in range(dk):
        for j in range(dk):
            eye = Fraction(1) if i == j else Fraction(0)
            m[i][j] = (eye - beta * k[i] * k[j]) * alpha[j]
    return m


def brute_force(q, k, v, alpha, beta, S0):
    """Exact outputs and states of the KDA recurrence.

    q, k: lists of T vectors of length dk; v: T vectors of length dv;
    alpha: T vectors of length dk (decay per key channel, alpha = exp(g));
    beta: T scalars; S0: dk x dv matrix.  All entries Fractions (or ints).
    Returns (o: T vectors of length dv, states: T matrices dk x dv).
    """
    T = len(q)
    dk = len(k[0])
    dv = len(v[0])
    conv = lambda x: Fraction(x)
    q = [[conv(x) for x in row] for row in q]
    k = [[conv(x) for x in row] for row in k]
    v = [[conv(x) for x in row] for row in v]
    alpha = [[conv(x) for x in row] for row in alpha]
    beta = [conv(x) for x in beta]
    S0 = [[conv(x) for x in row] for row in S0]
    M = [_transition(alpha[t], beta[t], k[t]) for t in range(T)]

    def phi(t, i):
        # product M_t M_{t-1} ... M_{i+1}, recomputed from scratch
        p = _eye(dk)
        for j in range(i + 1, t + 1):
            p = _matmul(M[j], p)
        return p

    outs, states = [], []
    for t in range(T):
        # the "-1" index means the initial state S_0: Phi(t, -1) applies M_0..M_t
        S = _matmul(phi(t, -1), S0)
        for i in range(t + 1):
            write = _zeros(dk, dv)
            for a in range(dk):
                for b in range(dv):
                    write[a][b] = beta[i] * k[i][a] * v[i][b]
            S = _add(S, _matmul(phi(t, i), write))
        o = [sum((S[a][b] * q[t][a] for a in range(dk)), Fraction(0)) for b in range(dv)]
        outs.append(o)
        states.append(S)
    return outs, states
