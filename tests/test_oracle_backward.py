"""The backward oracle against what the mathematics fixes (CPU only).

The oracle's gradients are the reverse mode of the sequential recurrence.
They are pinned to things other than themselves:

* central finite differences of the forward oracle's loss
  L = <do, o> + <dht, ht>, along random directions, for every input;
* exact per-element finite differences on a tiny case;
* closed forms: with alpha = 1 and beta = 0 the state is frozen, so
  o_t = S0^T q_t and every gradient has a short formula; with alpha = 1 and
  orthonormal keys the method is causal linear attention, whose gradients
  with respect to v, q and beta have a textbook form;
* packed-document isolation: a cotangent on one document gives exactly
  zero gradient on every other document (the page's gate for training on
  packed documents);
* split equivalence: chaining the backward of two halves through
  dh0 -> dht equals the backward of the whole;
* decay groups: the compact g's gradient is the group sum of the expanded one.
"""

import numpy as np
import pytest

import oracle.kda_oracle as orc
from oracle.kda_backward import kda_backward
from tests._chunked_model import chunked_backward, chunked_backward_blockref


def _unit(rng, *shape):
    z = rng.standard_normal(shape)
    return z / np.linalg.norm(z, axis=-1, keepdims=True)


def _case(rng, B, T, H, dk, dv, g_group=1, scale_g=1.0):
    q = _unit(rng, B, T, H, dk)
    k = _unit(rng, B, T, H, dk)
    v = rng.standard_normal((B, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    g = -np.log1p(np.exp(rng.standard_normal((B, T, H, dk // g_group)) - 2.0)) * scale_g
    return q, k, v, g, beta


def _loss(do, dht, q, k, v, g, beta, h0, cu=None, g_group=1):
    o, ht = orc.kda_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu, g_group=g_group)
    return float(np.sum(do * o) + np.sum(dht * ht))


@pytest.mark.parametrize("g_group", [1, 2])
def test_directional_finite_differences(g_group):
    rng = np.random.default_rng(100 + g_group)
    B, T, H, dk, dv = 2, 7, 2, 4, 3
    q, k, v, g, beta = _case(rng, B, T, H, dk, dv, g_group)
    h0 = 0.3 * rng.standard_normal((B, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dht = rng.standard_normal((B, H, dk, dv))
    gr = kda_backward(q, k, v, g, beta, do, h0=h0, dht=dht, g_group=g_group)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", h0="dh0")
    eps = 1e-6
    for name, x in args.items():
        for trial in range(3):
            d = rng.standard_normal(x.shape)
            plus = dict(args)
            minus = dict(args)
            plus[name] = x + eps * d
            minus[name] = x - eps * d
            fd = (_loss(do, dht, g_group=g_group, **plus) - _loss(do, dht, g_group=g_group, **minus)) / (2 * eps)
            an = float(np.sum(gr[names[name]] * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_elementwise_finite_differences_tiny():
    rng = np.random.default_rng(7)
    B, T, H, dk, dv = 1, 3, 1, 2, 2
    q, k, v, g, beta = _case(rng, B, T, H, dk, dv)
    h0 = rng.standard_normal((B, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dht = rng.standard_normal((B, H, dk, dv))
    gr = kda_backward(q, k, v, g, beta, do, h0=h0, dht=dht)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", h0="dh0")
    eps = 1e-6
    for name, x in args.items():
        for idx in np.ndindex(x.shape):
            plus = dict(args)
            minus = dict(args)
            xp = x.copy()
            xm = x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            plus[name] = xp
            minus[name] = xm
            fd = (_loss(do, dht, **plus) - _loss(do, dht, **minus)) / (2 * eps)
            assert abs(fd - gr[names[name]][idx]) <= 1e-8 * max(1.0, abs(fd)), (name, idx)


def test_frozen_state_closed_forms():
    """alpha = 1, beta = 0: S_t = S0, o_t = S0^T q_t.  With
    D_t = dht + sum_{s >= t} q_s do_s^T (the cotangent reaching token t):
    dq_t = S0 do_t, dk = dv = 0, dbeta_t = (D_t^T k_t) . (v_t - S0^T k_t),
    dg_t[c] = sum_j D_t[c, j] S0[c, j], dh0 = D_1."""
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 1, 6, 1, 4, 3
    q, k, v, _, _ = _case(rng, B, T, H, dk, dv)
    g = np.zeros((B, T, H, dk))
    beta = np.zeros((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dht = rng.standard_normal((B, H, dk, dv))
    gr = kda_backward(q, k, v, g, beta, do, h0=S0, dht=dht)
    S = S0[0, 0]
    D = dht[0, 0].copy()
    Ds = [None] * T
    for t in range(T - 1, -1, -1):
        D = D + np.outer(q[0, t, 0], do[0, t, 0])
        Ds[t] = D.copy()
    for t in range(T):
        assert np.allclose(gr["dq"][0, t, 0], S @ do[0, t, 0], atol=1e-13)
        db = (Ds[t].T @ k[0, t, 0]) @ (v[0, t, 0] - S.T @ k[0, t, 0])
        assert abs(gr["dbeta"][0, t, 0] - db) < 1e-12
        assert np.allclose(gr["dg"][0, t, 0], np.sum(Ds[t] * S, axis=1), atol=1e-12)
    assert np.max(np.abs(gr["dk"])) == 0.0 and np.max(np.abs(gr["dv"])) == 0.0
    assert np.allclose(gr["dh0"][0, 0], Ds[0], atol=1e-13)


def test_linear_attention_closed_forms():
    """alpha = 1, orthonormal keys, S0 = 0: o_t = sum_{i<=t} beta_i (q_t . k_i) v_i.
    Then dv_i = beta_i sum_{t>=i} (q_t . k_i) do_t,
    dq_t = sum_{i<=t} beta_i (v_i . do_t) k_i,
    dbeta_i = sum_{t>=i} (q_t . k_i)(v_i . do_t)."""
    rng = np.random.default_rng(12)
    T, dk, dv = 5, 6, 3
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][None, :, None, :]
    q = _unit(rng, 1, T, 1, dk)
    v = rng.standard_normal((1, T, 1, dv))
    beta = rng.uniform(0.1, 0.9, (1, T, 1))
    g = np.zeros((1, T, 1, dk))
    do = rng.standard_normal((1, T, 1, dv))
    gr = kda_backward(q, k, v, g, beta, do)
    qk = q[0, :, 0] @ k[0, :, 0].T  # [t, i]
    mask = np.tril(np.ones((T, T)))
    W = qk * mask  # W[t, i] = q_t . k_i for i <= t
    b = beta[0, :, 0]
    dv_ref = b[:, None] * (W.T @ do[0, :, 0])
    vd = v[0, :, 0] @ do[0, :, 0].T  # [i, t] = v_i . do_t
    dq_ref = (mask * (vd.T * b[None, :])) @ k[0, :, 0]
    db_ref = np.sum(W.T * vd, axis=1)
    assert np.allclose(gr["dv"][0, :, 0], dv_ref, atol=1e-13)
    assert np.allclose(gr["dq"][0, :, 0], dq_ref, atol=1e-13)
    assert np.allclose(gr["dbeta"][0, :, 0], db_ref, atol=1e-13)


def test_packed_documents_have_zero_cross_gradient():
    rng = np.random.default_rng(13)
    cu = np.array([0, 5, 5, 12, 20])
    T, H, dk, dv = 20, 2, 4, 3
    q, k, v, g, beta = _case(rng, 1, T, H, dk, dv)
    N = len(cu) - 1
    h0 = rng.standard_normal((N, H, dk, dv))
    for doc in range(N):
        do = np.zeros((1, T, H, dv))
        do[0, cu[doc]:cu[doc + 1]] = rng.standard_normal((cu[doc + 1] - cu[doc], H, dv))
        dht = np.zeros((N, H, dk, dv))
        dht[doc] = rng.standard_normal((H, dk, dv))
        gr = kda_backward(q, k, v, g, beta, do, h0=h0, dht=dht, cu_seqlens=cu)
        outside = np.ones(T, dtype=bool)
        outside[cu[doc]:cu[doc + 1]] = False
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            assert np.all(gr[name][0, outside] == 0.0), (doc, name)
        others = [n for n in range(N) if n != doc]
        assert np.all(gr["dh0"][others] == 0.0)
        if cu[doc + 1] == cu[doc]:
            assert np.array_equal(gr["dh0"][doc], dht[doc])  # ht = h0 for an empty document


def test_split_equivalence_of_gradients():
    """Backward over [0, T) equals the backward of [t, T) (from h0 = ht of
    [0, t)) chained into the backward of [0, t) through dht = dh0."""
    rng = np.random.default_rng(14)
    T, t, H, dk, dv = 11, 4, 2, 4, 3
    q, k, v, g, beta = _case(rng, 1, T, H, dk, dv)
    h0 = rng.standard_normal((1, H, dk, dv))
    do = rng.standard_normal((1, T, H, dv))
    dht = rng.standard_normal((1, H, dk, dv))
    full = kda_backward(q, k, v, g, beta, do, h0=h0, dht=dht)
    sl1, sl2 = slice(0, t), slice(t, T)
    _, hmid = orc.kda_forward(q[:, sl1], k[:, sl1], v[:, sl1], g[:, sl1], beta[:, sl1], h0=h0)
    second = kda_backward(q[:, sl2], k[:, sl2], v[:, sl2], g[:, sl2], beta[:, sl2], do[:, sl2], h0=hmid, dht=dht)
    first = kda_backward(q[:, sl1], k[:, sl1], v[:, sl1], g[:, sl1], beta[:, sl1], do[:, sl1], h0=h0,
                         dht=second["dh0"])
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        joined = np.concatenate([first[name], second[name]], axis=1)
        assert np.allclose(joined, full[name], atol=1e-12), name
    assert np.allclose(first["dh0"], full["dh0"], atol=1e-12)


def test_decay_group_gradient_is_group_sum():
    rng = np.random.default_rng(15)
    T, H, dk, dv, gg = 9, 2, 8, 3, 4
    q, k, v, g, beta = _case(rng, 1, T, H, dk, dv, g_group=gg)
    do = rng.standard_normal((1, T, H, dv))
    compact = kda_backward(q, k, v, g, beta, do, g_group=gg)
    expanded = kda_backward(q, k, v, np.repeat(g, gg, axis=-1), beta, do, g_group=1)
    assert np.allclose(compact["dg"], expanded["dg"].reshape(1, T, H, dk // gg, gg).sum(-1), atol=1e-13)
    for name in ("dq", "dk", "dv", "dbeta"):
        assert np.allclose(compact[name], expanded[name], atol=1e-13)


@pytest.mark.parametrize("C", [1, 5, 16, 64])
def test_chunked_backward_model_matches_oracle(C):
    """The block algebra the GPU backward evaluates (per-chunk transfer
    F^T, offset b, the reverse state pass, the chunk-local gradients), in
    float64, against the oracle's reverse mode."""
    rng = np.random.default_rng(200 + C)
    T, dk, dv = 70, 8, 5
    q, k, v, g, beta = _case(rng, 1, T, 1, dk, dv, scale_g=3.0)
    h0 = rng.standard_normal((1, 1, dk, dv))
    do = rng.standard_normal((1, T, 1, dv))
    dht = rng.standard_normal((1, 1, dk, dv))
    ref = kda_backward(q, k, v, g, beta, do, h0=h0, dht=dht)
    got = chunked_backward(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], h0[0, 0], do[0, :, 0],
                           dht[0, 0], C)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        r = ref[name][0, :, 0]
        assert np.max(np.abs(got[name] - r)) <= 1e-10 * max(1.0, np.max(np.abs(r))), name
    assert np.max(np.abs(got["dh0"] - ref["dh0"][0, 0])) <= 1e-10 * max(1.0, np.max(np.abs(ref["dh0"])))


@pytest.mark.parametrize("C,B", [(64, 16), (16, 4), (20, 16)])
def test_block_referenced_backward_model_matches_oracle(C, B):
    """The block-referenced algebra (factors of at most one block's decay;
    pairs of blocks through e^{m_I - m_J}), in float64, against the oracle's
    reverse mode on decays of about -1,000 per 64 tokens on some channels:
    there the chunk-start factors e^{+-G} exceed float64's range, the block
    ones (at most e^{125} for B = 16) do not."""
    rng = np.random.default_rng(300 + C + B)
    T, dk, dv = 90, 6, 5
    q, k, v, g, beta = _case(rng, 1, T, 1, dk, dv)
    g[..., ::3] = -(1000.0 / 64.0) * (1.0 + 0.2 * np.tanh(rng.standard_normal(g[..., ::3].shape)))
    h0 = rng.standard_normal((1, 1, dk, dv))
    do = rng.standard_normal((1, T, 1, dv))
    dht = rng.standard_normal((1, 1, dk, dv))
    ref = kda_backward(q, k, v, g, beta, do, h0=h0, dht=dht)
    sl = lambda x: x[0, :, 0]
    with np.errstate(over="ignore", invalid="ignore"):
        plain = chunked_backward(sl(q), sl(k), sl(v), sl(g), sl(beta), h0[0, 0], sl(do), dht[0, 0], 64)
    assert not all(np.all(np.isfinite(plain[n])) for n in ("dq", "dk", "dg")), "chunk-start factors stayed finite"
    got = chunked_backward_blockref(sl(q), sl(k), sl(v), sl(g), sl(beta), h0[0, 0], sl(do), dht[0, 0], C, B)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        r = ref[name][0, :, 0]
        assert np.max(np.abs(got[name] - r)) <= 1e-10 * max(1.0, np.max(np.abs(r))), name
    assert np.max(np.abs(got["dh0"] - ref["dh0"][0, 0])) <= 1e-10 * max(1.0, np.max(np.abs(ref["dh0"])))
