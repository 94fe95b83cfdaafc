"""CPU fp64 oracle for the KDA backward pass (reverse mode of the recurrence).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
use it.  It shares no code with the HIP path.

What it computes
----------------
The miniKimiK3 card ("Architecture", Kimi Delta Attention bullet) says KDA
trains through a chunked parallel form.  Training needs the gradients of a
scalar loss with respect to every input of the forward pass.  Here the loss
is the one whose output cotangents are given:

    L = sum_t <do_t, o_t> + sum_n <dht_n, ht_n>

and this module returns dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta and dL/dh0.
They are exact (up to float64 rounding) derivatives of the plain sequential
recurrence of ``kda_oracle``, taken by reverse mode one token at a time.  The
forward states are recomputed and kept, then each step is undone in reverse
order.

One token of the forward (the matrix form of the bullet, decay first):

    a = exp(g);  S' = Diag(a) S;  e = S'^T k;  u = beta (v - e)
    S_new = S' + k u^T;  o = S_new^T q

Its reverse, for the cotangent dS of S_new and do of o (a step's only
consumers are o and the next token):

    dS += q do^T                 dq  = S_new do
    dk  = dS u + S' de           du  = dS^T k
    dbeta = du . (v - e)         dv  = beta du        de = -beta du
    dS' = dS + k de^T
    dg  = a * rowsum(dS' * S)    dS_prev = Diag(a) dS'

With g_group > 1 a stored log-decay value feeds g_group channels, so its
gradient is the sum over them.  Under cu_seqlens every document is
independent.  So a document's gradients depend only on its own inputs and
cotangents, and a cross-document gradient is exactly zero.  This is the
gradient side of the packed-document isolation in the Mini-K3-1H-mamba2
README.
"""

import sys

import numpy as np

from .kda_oracle import expand_decay

_this = sys.modules[__name__]

__all__ = ["reverse_step", "kda_backward_sequence", "kda_backward"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def reverse_step(Sp, q, k, v, g, beta, do, dS):
    """Reverse mode of one token, vectorised over leading heads.

    Sp: [..., dk, dv] state entering the token; q, k, g: [..., dk];
    v, do: [..., dv]; beta: [...]; dS: cotangent of the token's output
    state.  Recomputes the token's forward quantities and returns
    (dq, dk, dv, dg, dbeta, dS_prev).
    """
    a = np.exp(g)
    Sd = a[..., :, None] * Sp
    e = np.matmul(k[..., None, :], Sd)[..., 0, :]
    r = v - e
    u = beta[..., None] * r
    S_new = Sd + k[..., :, None] * u[..., None, :]
    # o = S_new^T q
    dq = np.matmul(S_new, do[..., :, None])[..., 0]
    dS = dS + q[..., :, None] * do[..., None, :]
    # S_new = S' + k u^T
    du = np.matmul(k[..., None, :], dS)[..., 0, :]
    dk = np.matmul(dS, u[..., :, None])[..., 0]
    # u = beta (v - e)
    db = np.sum(du * r, axis=-1)
    dv = beta[..., None] * du
    de = -beta[..., None] * du
    # e = S'^T k
    dk = dk + np.matmul(Sd, de[..., :, None])[..., 0]
    dSd = dS + k[..., :, None] * de[..., None, :]
    # S' = Diag(a) S
    dg = a * np.sum(dSd * Sp, axis=-1)
    return dq, dk, dv, dg, db, a[..., :, None] * dSd


def kda_backward_sequence(q, k, v, g, beta, S0, do, dST):
    """Reverse mode over one time axis, vectorised over leading heads.

    q, k: [L, ..., dk]; v, do: [L, ..., dv]; g: [L, ..., dk] (expanded);
    beta: [L, ...]; S0, dST: [..., dk, dv] (dST = cotangent of the final
    state).  Returns (dq, dk, dv, dg, dbeta, dS0) with the shapes of
    (q, k, v, g, beta, S0).
    """
    L = q.shape[0]
    # forward, keeping the state entering every token
    S_in = np.empty((L,) + S0.shape)
    S = np.array(S0, dtype=np.float64, copy=True)
    for t in range(L):
        S_in[t] = S
        a = np.exp(g[t])
        Sd = a[..., :, None] * S
        e = np.matmul(k[t][..., None, :], Sd)[..., 0, :]
        u = beta[t][..., None] * (v[t] - e)
        S = Sd + k[t][..., :, None] * u[..., None, :]

    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    dg = np.zeros(g.shape)
    db = np.zeros(beta.shape)
    dS = np.array(dST, dtype=np.float64, copy=True)
    for t in range(L - 1, -1, -1):
        dq[t], dk[t], dv[t], dg[t], db[t], dS = _this.reverse_step(S_in[t], q[t], k[t], v[t], g[t], beta[t], do[t], dS)
    return dq, dk, dv, dg, db, dS


def _group_sum(dg, g_group):
    if g_group == 1:
        return dg
    sh = dg.shape
    return dg.reshape(sh[:-1] + (sh[-1] // g_group, g_group)).sum(axis=-1)


def kda_backward(q, k, v, g, beta, do, h0=None, dht=None, cu_seqlens=None, g_group=1):
    """Gradients of L = <do, o> + <dht, ht> for ``kda_oracle.kda_forward``.

    Shapes and conventions follow the forward: q, k [B, T, H, dk];
    v, do [B, T, H, dv]; g [B, T, H, dk // g_group]; beta [B, T, H];
    h0, dht [N, H, dk, dv] or None (zeros).  Returns a dict with dq, dk, dv,
    dg (compact, the shape of g), dbeta and dh0 ([N, H, dk, dv]).
    """
    q, k, v, g, beta, do = map(_f64, (q, k, v, g, beta, do))
    B, T, H, dk = q.shape
    dv_ = v.shape[-1]
    ge = expand_decay(g, dk, g_group)
    dq = np.zeros(q.shape)
    dkk = np.zeros(k.shape)
    dvv = np.zeros(v.shape)
    dge = np.zeros(ge.shape)
    db = np.zeros(beta.shape)
    if cu_seqlens is None:
        N = B
        spans = [(b, 0, T) for b in range(B)]
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        N = len(cu) - 1
        spans = [(0, int(cu[n]), int(cu[n + 1])) for n in range(N)]
    S0s = np.zeros((N, H, dk, dv_)) if h0 is None else _f64(h0)
    dTs = np.zeros((N, H, dk, dv_)) if dht is None else _f64(dht)
    dh0 = np.zeros((N, H, dk, dv_))
    for n, (b, s, e) in enumerate(spans):
        if e == s:
            dh0[n] = dTs[n]  # ht = h0 for an empty document
            continue
        sl = (b, slice(s, e))
        res = kda_backward_sequence(q[sl], k[sl], v[sl], ge[sl], beta[sl], S0s[n], do[sl], dTs[n])
        dq[sl], dkk[sl], dvv[sl], dge[sl], db[sl], dh0[n] = res
    return {"dq": dq, "dk": dkk, "dv": dvv, "dg": _group_sum(dge, g_group), "dbeta": db, "dh0": dh0}
