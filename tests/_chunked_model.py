"""CPU float64 model of the chunked parallel form of KDA (test utility).

Not the oracle.  This is the block algebra the GPU path evaluates, derived
from the recurrence (miniKimiK3 card, "Architecture", KDA bullet: the method
"trains through a chunked parallel form"), written out with numpy in float64
so that the oracle can be pinned against an independent formulation and so
that the algebra itself is checked before any kernel uses it.

Per head and chunk of c tokens, with S0 the state entering the chunk,
G_r = sum_{j<=r} g_j (per key channel, inclusive, chunk-local):

    Kt = K * exp(G)        Qt = Q * exp(G)        Kh = K * exp(-G)
    Kb = K * exp(G_c - G)  (G_c = last row of G)
    A  = strictly_lower(Diag(beta) Kt Kh^T)
    P  = lower_including_diagonal(Qt Kh^T)
    T  = (I + A)^-1 Diag(beta)                    (UT transform)
    U  = T (V - Kt S0)
    O  = Qt S0 + P U
    S  = Diag(exp(G_c)) S0 + Kb^T U
"""

import numpy as np


def chunked_forward(q, k, v, g, beta, S0, C):
    """q, k [L, dk]; v [L, dv]; g [L, dk] (expanded); beta [L]; S0 [dk, dv].
    Returns (o [L, dv], S_L)."""
    L, dk = q.shape
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((L, v.shape[1]))
    for s in range(0, L, C):
        e = min(L, s + C)
        c = e - s
        G = np.cumsum(g[s:e], axis=0)
        Kt = k[s:e] * np.exp(G)
        Qt = q[s:e] * np.exp(G)
        Kh = k[s:e] * np.exp(-G)
        Kb = k[s:e] * np.exp(G[-1] - G)
        b = beta[s:e]
        A = np.tril(b[:, None] * (Kt @ Kh.T), -1)
        P = np.tril(Qt @ Kh.T, 0)
        T = np.linalg.solve(np.eye(c) + A, np.diag(b))
        U = T @ (v[s:e] - Kt @ S)
        o[s:e] = Qt @ S + P @ U
        S = np.exp(G[-1])[:, None] * S + Kb.T @ U
    return o, S
