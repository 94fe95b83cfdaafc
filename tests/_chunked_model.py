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


def chunked_backward(q, k, v, g, beta, S0, do, dST, C):
    """Gradients of <do, o> + <dST, S_L> through the chunked form, for one
    head: q, k [L, dk]; v, do [L, dv]; g [L, dk] (expanded); beta [L];
    S0, dST [dk, dv].  Returns a dict of dq, dk, dv, dg, dbeta, dh0.

    The decomposition the GPU backward uses:

    1. forward, keeping the state S_c entering every chunk;
    2. per chunk, independently: the transfer of the state cotangent
       F^T = (I - W^T Kh) Diag(gam) with W = T Kt, and the offset
       b = Z^T dO with Z = Qt - P W, so that the reverse state pass is
       dS_c = F^T dS_{c+1} + b  (F = Diag(gam)(I - Kh^T W) is the chunk's
       forward transfer S -> Diag(gam) S + Kb^T U restricted to S);
    3. the reverse state pass over chunks, keeping dS_{c+1} for every chunk;
    4. per chunk, independently, with dSt = Diag(gam) dS_{c+1}:
         R = V - Kt S;  U = T R;  dU = Kh dSt + P^T dO;  dR = T^T dU  (= dv)
         dP = lower_incl(dO U^T);  dT = lower_incl(dU R^T)
         dbeta_j = sum_i dT_ij X_ij;  dA = -strict(X^T dT Diag(beta) X^T)
         dbeta_r += sum_i dA_ri B_ri  (B = Kt Kh^T);  dB = Diag(beta) dA
         dQt = dO S^T + dP Kh;  dKt = -dR S^T + dB Kh
         dKH = dB^T Kt + dP^T Qt + U dSt^T
         dq = dQt e^G;  dk = dKt e^G + dKH e^-G
         dG = q dq + k (dKt e^G - dKH e^-G), and on the chunk's last row
              + sum_r (U dSt^T * Kh)_r + rowsum(S * dSt)
         dg = reverse cumulative sum of dG over the chunk.
    """
    L, dk = q.shape
    starts = list(range(0, L, C))
    S_in = []
    S = np.array(S0, dtype=np.float64, copy=True)
    blocks = []
    for s in starts:
        e = min(L, s + C)
        c = e - s
        G = np.cumsum(g[s:e], axis=0)
        eG, emG = np.exp(G), np.exp(-G)
        gam = eG[-1]
        Kt, Qt, Kh = k[s:e] * eG, q[s:e] * eG, k[s:e] * emG
        b = beta[s:e]
        Bm = np.tril(Kt @ Kh.T, -1)
        A = b[:, None] * Bm
        P = np.tril(Qt @ Kh.T, 0)
        X = np.linalg.inv(np.eye(c) + A)
        T = X * b[None, :]
        blocks.append(dict(s=s, e=e, G=G, eG=eG, emG=emG, gam=gam, Kt=Kt, Qt=Qt, Kh=Kh, B=Bm, P=P, X=X, T=T))
        S_in.append(S.copy())
        U = T @ (v[s:e] - Kt @ S)
        S = gam[:, None] * S + (Kh * gam[None, :]).T @ U
    # 2. per-chunk transfer and offset of the state cotangent
    Ft, off = [], []
    for bl in blocks:
        W = bl["T"] @ bl["Kt"]
        Z = bl["Qt"] - bl["P"] @ W
        Ft.append((np.eye(dk) - W.T @ bl["Kh"]) * bl["gam"][None, :])
        off.append(Z.T @ do[bl["s"]:bl["e"]])
    # 3. reverse state pass
    dS = np.array(dST, dtype=np.float64, copy=True)
    dS_out = [None] * len(blocks)
    for i in range(len(blocks) - 1, -1, -1):
        dS_out[i] = dS.copy()
        dS = Ft[i] @ dS + off[i]
    res = {n: np.zeros(x.shape) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    res["dh0"] = dS
    # 4. chunk-local gradients
    for i, bl in enumerate(blocks):
        s, e = bl["s"], bl["e"]
        Sc, dSt = S_in[i], bl["gam"][:, None] * dS_out[i]
        dO = do[s:e]
        T, X, P, Kh, Kt, Qt = bl["T"], bl["X"], bl["P"], bl["Kh"], bl["Kt"], bl["Qt"]
        bb = beta[s:e]
        R = v[s:e] - Kt @ Sc
        U = T @ R
        dU = Kh @ dSt + P.T @ dO
        dR = T.T @ dU
        dP = np.tril(dO @ U.T, 0)
        dT = np.tril(dU @ R.T, 0)
        db = np.sum(dT * X, axis=0)
        dA = -np.tril(X.T @ (dT * bb[None, :]) @ X.T, -1)
        db += np.sum(dA * bl["B"], axis=1)
        dB = bb[:, None] * dA
        dQt = dO @ Sc.T + dP @ Kh
        dKt = -dR @ Sc.T + dB @ Kh
        dKb = U @ dSt.T
        dKH = dB.T @ Kt + dP.T @ Qt + dKb
        dq = dQt * bl["eG"]
        dkk = dKt * bl["eG"] + dKH * bl["emG"]
        dG = q[s:e] * dq + k[s:e] * (dKt * bl["eG"] - dKH * bl["emG"])
        dG[-1] += np.sum(dKb * Kh, axis=0) + np.sum(Sc * dSt, axis=1)
        res["dq"][s:e] = dq
        res["dk"][s:e] = dkk
        res["dv"][s:e] = dR
        res["dg"][s:e] = np.cumsum(dG[::-1], axis=0)[::-1]
        res["dbeta"][s:e] = db
    return res


def _block_refs(g, B):
    """Chunk-local cumulative decay G and, per row, the reference m of its
    B-row block: the midpoint of the block's decay, so that the factors
    e^{+-(G - m)} of its rows stay within e^{|block sum| / 2}."""
    G = np.cumsum(g, axis=0)
    m = np.zeros_like(G)
    for a in range(0, G.shape[0], B):
        e = min(G.shape[0], a + B)
        prev = G[a - 1] if a > 0 else np.zeros(G.shape[1])
        m[a:e] = prev + 0.5 * (G[e - 1] - prev)
    return G, m


def chunked_backward_blockref(q, k, v, g, beta, S0, do, dST, C=64, B=16, rnd=None):
    """The same gradients as chunked_backward, with every factor of the block
    algebra referenced so that none exceeds 1 beyond one B-row block: the
    operand rows qt = Q e^{G - m}, kt = K e^{G - m}, kh = K e^{m - G} use
    their block's reference m; a pair of blocks (I, J), I >= J, of the k-k
    and q-k products carries the shift e^{m_I - m_J} <= 1; the state side
    uses Kt = kt e^{m}, Qt = qt e^{m} and Kb = kh e^{G_c - m} (all <= 1).
    Each product is the chunk-start one exactly (the references cancel), so
    the gradients follow with the references held constant.  rnd, if given,
    is applied where the GPU path stores a bf16 operand (the referenced rows
    and their scaled forms, T, S, dS and the per-chunk transfer), to model its
    roundings."""
    r = rnd if rnd is not None else (lambda x: x)
    L, dk = q.shape
    S = np.array(S0, dtype=np.float64, copy=True)
    chunks, S_in = [], []
    for s in range(0, L, C):
        e = min(L, s + C)
        c = e - s
        G, m = _block_refs(g[s:e], B)
        qt, kt, kh = r(q[s:e] * np.exp(G - m)), r(k[s:e] * np.exp(G - m)), r(k[s:e] * np.exp(m - G))
        blk = np.arange(c) // B
        mb = m[np.minimum(np.arange(0, c, B), c - 1)]           # [blocks, dk]
        shift = np.where((blk[:, None] >= blk[None, :])[:, :, None], mb[blk][:, None, :] - mb[blk][None, :, :], -np.inf)
        D = np.exp(shift)                                        # e^{m_I - m_J} for I >= J, else 0
        Bm = np.tril(np.einsum("ic,jc,ijc->ij", kt, kh, D), -1)
        P = np.tril(np.einsum("ic,jc,ijc->ij", qt, kh, D), 0)
        b = beta[s:e]
        X = np.linalg.inv(np.eye(c) + b[:, None] * Bm)
        T = r(X * b[None, :])
        Kt, Qt, Kb = r(kt * np.exp(m)), r(qt * np.exp(m)), r(kh * np.exp(G[-1] - m))
        gam = np.exp(G[-1])
        chunks.append(dict(s=s, e=e, G=G, m=m, qt=qt, kt=kt, kh=kh, D=D, B=Bm, P=P, X=X, T=T, Kt=Kt, Qt=Qt,
                           Kb=Kb, gam=gam))
        S_in.append(r(S.copy()))
        U = T @ (v[s:e] - Kt @ S)
        S = gam[:, None] * S + Kb.T @ U
    # per-chunk transfer F = Diag(gam) - Kb^T W (the decay part kept apart) and offset
    Mt, off = [], []
    for ch in chunks:
        W = ch["T"] @ ch["Kt"]
        Z = ch["Qt"] - ch["P"] @ W
        Mt.append(r(W.T @ ch["Kb"]))                             # M^T
        off.append(r(Z.T @ do[ch["s"]:ch["e"]]))
    dS = np.array(dST, dtype=np.float64, copy=True)
    dS_out = [None] * len(chunks)
    for i in range(len(chunks) - 1, -1, -1):
        dS_out[i] = r(dS.copy())
        dS = chunks[i]["gam"][:, None] * dS - Mt[i] @ dS + off[i]
    res = {n: np.zeros(x.shape) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    res["dh0"] = dS
    for i, ch in enumerate(chunks):
        s, e = ch["s"], ch["e"]
        Sc, dSo, dO, bb = S_in[i], dS_out[i], do[s:e], beta[s:e]
        T, X, P, D = ch["T"], ch["X"], ch["P"], ch["D"]
        R = v[s:e] - ch["Kt"] @ Sc
        U = T @ R
        dU = ch["Kb"] @ dSo + P.T @ dO
        dR = T.T @ dU
        dP = np.tril(dO @ U.T, 0)
        dT = np.tril(dU @ R.T, 0)
        dA = -np.tril(X.T @ (dT * bb[None, :]) @ X.T, -1)
        dB = bb[:, None] * dA
        db = np.sum(dT * X, axis=0) + np.sum(dA * ch["B"], axis=1)
        em = np.exp(ch["m"])
        dqt = em * (dO @ Sc.T) + np.einsum("ij,jc,ijc->ic", dP, ch["kh"], D)
        dkt = -em * (dR @ Sc.T) + np.einsum("ij,jc,ijc->ic", dB, ch["kh"], D)
        dkh = np.einsum("ij,ic,ijc->jc", dB, ch["kt"], D) + np.einsum("ij,ic,ijc->jc", dP, ch["qt"], D)
        dkb = U @ dSo.T
        G, m = ch["G"], ch["m"]
        up, dn, tail = np.exp(G - m), np.exp(m - G), np.exp(G[-1][None, :] - G)
        dq = dqt * up
        a = dkt * up
        bt = dkh * dn + dkb * tail
        dG = q[s:e] * dq + k[s:e] * (a - bt)
        dG[-1] += np.sum(dkb * tail * k[s:e], axis=0) + ch["gam"] * np.sum(Sc * dSo, axis=1)
        res["dq"][s:e] = dq
        res["dk"][s:e] = a + bt
        res["dv"][s:e] = dR
        res["dg"][s:e] = np.cumsum(dG[::-1], axis=0)[::-1]
        res["dbeta"][s:e] = db
    return res
