"""Pins of the CPU oracle: checks against facts the pages and the mathematics
fix, independent of the oracle's own arithmetic.

Each ``pin_*`` function runs one check through the oracle module passed in
(``oracle.kda_oracle`` or a planted-mistake variant of it) and raises
AssertionError when the check fails.  ``tests/test_oracle_pins.py`` runs them
on the real oracle; ``tests/test_oracle_mutants.py`` runs them on oracles with
a planted mistake and requires every mistake to fail at least one pin.
"""

from fractions import Fraction

import numpy as np

from oracle.brute import brute_force
from tests._chunked_model import chunked_forward


def _unit(rng, *shape):
    z = rng.standard_normal(shape)
    return z / np.linalg.norm(z, axis=-1, keepdims=True)


def _case(rng, T, H, dk, dv, decay_shift=2.0):
    q = _unit(rng, 1, T, H, dk)
    k = _unit(rng, 1, T, H, dk)
    v = rng.standard_normal((1, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, H))))
    g = -np.logaddexp(0.0, rng.standard_normal((1, T, H, dk)) - decay_shift)
    return q, k, v, g, beta


def pin_fd_gradient_step(orc, seed=0):
    """The write is one gradient-descent step on 1/2 ||S^T k - v||^2 taken from
    the decayed state (miniKimiK3 card, KDA bullet).  The gradient is taken by
    central differences, not by formula."""
    rng = np.random.default_rng(seed)
    dk, dv = 5, 3
    S = rng.standard_normal((dk, dv))
    q, k = rng.standard_normal(dk), rng.standard_normal(dk)
    v = rng.standard_normal(dv)
    g = -np.abs(rng.standard_normal(dk)) * 0.5
    beta = 0.37
    S_dec = np.exp(g)[:, None] * S

    def loss(M):
        r = M.T @ k - v
        return 0.5 * float(r @ r)

    h = 1e-6
    grad = np.zeros_like(S_dec)
    for i in range(dk):
        for j in range(dv):
            E = np.zeros_like(S_dec)
            E[i, j] = h
            grad[i, j] = (loss(S_dec + E) - loss(S_dec - E)) / (2 * h)
    expect = S_dec - beta * grad
    S_new, o = orc.kda_step(S, q, k, v, g, np.float64(beta))
    assert np.max(np.abs(S_new - expect)) < 1e-8, "state update is not the gradient step"
    assert np.max(np.abs(o - expect.T @ q)) < 1e-8, "output does not read the post-update state"


def pin_exact_replacement(orc, seed=1):
    """||k|| = 1 and beta = 1: the write replaces what the state stores for k,
    S_t^T k_t = v_t, whatever alpha and the previous state are.  For general
    beta: S_t^T k = (1 - beta||k||^2) S'^T k + beta||k||^2 v (closed form)."""
    rng = np.random.default_rng(seed)
    for dk, dv in ((4, 4), (6, 3), (64, 64)):
        S = rng.standard_normal((dk, dv))
        k = _unit(rng, dk)
        q = rng.standard_normal(dk)
        v = rng.standard_normal(dv)
        g = -np.abs(rng.standard_normal(dk))
        S_new, _ = orc.kda_step(S, q, k, v, g, np.float64(1.0))
        assert np.max(np.abs(S_new.T @ k - v)) < 1e-12, "beta=1, |k|=1 write is not an exact replacement"
        beta = 0.3
        kk = rng.standard_normal(dk)
        S_new, _ = orc.kda_step(S, q, kk, v, g, np.float64(beta))
        Sd = np.exp(g)[:, None] * S
        n2 = kk @ kk
        expect = (1 - beta * n2) * (Sd.T @ kk) + beta * n2 * v
        assert np.max(np.abs(S_new.T @ kk - expect)) < 1e-10, "closed form of the read-back fails"


def pin_frozen_state(orc, seed=2):
    """alpha = 1 and beta = 0: the update is the identity, o_t = S_0^T q_t."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 9, 2, 5, 4
    q, k, v, _, _ = _case(rng, T, H, dk, dv)
    g = np.zeros((1, T, H, dk))
    beta = np.zeros((1, T, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    o, ht = orc.kda_forward(q, k, v, g, beta, h0=S0)
    expect = np.einsum("bthk,bhkv->bthv", q, S0)
    assert np.max(np.abs(o - expect)) < 1e-13
    assert np.max(np.abs(ht - S0)) < 1e-13


def pin_linear_attention(orc, seed=3):
    """alpha = 1, orthonormal keys, S_0 = 0: the erase term vanishes and KDA is
    causal linear attention, o = tril(Q K^T) Diag(beta) V (a masked GEMM)."""
    rng = np.random.default_rng(seed)
    T, dk, dv = 7, 8, 5
    Kmat, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Kmat[:, :T].T.copy()                      # T orthonormal rows
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 0.9, T)
    expect = np.tril(q @ k.T) @ (beta[:, None] * v)
    o, _ = orc.kda_forward(q[None, :, None], k[None, :, None], v[None, :, None],
                           np.zeros((1, T, 1, dk)), beta[None, :, None])
    assert np.max(np.abs(o[0, :, 0] - expect)) < 1e-13


def pin_pure_decay(orc, seed=4):
    """beta = 0: S_t = Diag(exp(sum_{j<=t} g_j)) S_0 -- the decay acts on the key
    channels (rows of S) and compounds."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 6, 1, 4, 3
    q, k, v, g, _ = _case(rng, T, H, dk, dv)
    beta = np.zeros((1, T, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    o, ht = orc.kda_forward(q, k, v, g, beta, h0=S0)
    cum = np.cumsum(g[0, :, 0], axis=0)            # [T, dk]
    for t in range(T):
        St = np.exp(cum[t])[:, None] * S0[0, 0]
        assert np.max(np.abs(o[0, t, 0] - St.T @ q[0, t, 0])) < 1e-13
    assert np.max(np.abs(ht[0, 0] - np.exp(cum[-1])[:, None] * S0[0, 0])) < 1e-13


def rational_case(seed, T=4, dk=3, dv=2):
    """A tiny exact case: rational alpha, beta, q, k, v, S_0."""
    r = np.random.default_rng(seed)
    fr = lambda lo, hi, den: Fraction(int(r.integers(lo, hi)), den)
    q = [[fr(-4, 5, 4) for _ in range(dk)] for _ in range(T)]
    k = [[fr(-5, 6, 5) for _ in range(dk)] for _ in range(T)]
    v = [[fr(-6, 7, 3) for _ in range(dv)] for _ in range(T)]
    alpha = [[fr(1, 9, 8) for _ in range(dk)] for _ in range(T)]
    beta = [fr(0, 5, 4) for _ in range(T)]
    S0 = [[fr(-3, 4, 2) for _ in range(dv)] for _ in range(dk)]
    return q, k, v, alpha, beta, S0


def oracle_on_rational(orc, q, k, v, alpha, beta, S0):
    f = lambda x: np.array([[float(y) for y in row] for row in x])
    qa, ka, va, al = f(q), f(k), f(v), f(alpha)
    ba = np.array([float(b) for b in beta])
    g = np.log(al)
    o, ht = orc.kda_forward(qa[None, :, None], ka[None, :, None], va[None, :, None], g[None, :, None],
                            ba[None, :, None], h0=f(S0)[None, None])
    return o[0, :, 0], ht[0, 0]


def pin_brute_force(orc, seeds=(10, 11, 12)):
    """Exact rational brute force (per-token recomputation of the unrolled
    products of transition matrices) on tiny inputs."""
    for s in seeds:
        case = rational_case(s)
        o_ex, S_ex = brute_force(*case)
        o, ht = oracle_on_rational(orc, *case)
        o_ref = np.array([[float(x) for x in row] for row in o_ex])
        S_ref = np.array([[float(x) for x in row] for row in S_ex[-1]])
        scale = 1.0 + np.max(np.abs(o_ref))
        assert np.max(np.abs(o - o_ref)) < 1e-13 * scale, "oracle differs from exact brute force"
        assert np.max(np.abs(ht - S_ref)) < 1e-13 * (1.0 + np.max(np.abs(S_ref)))


def pin_chunked_equals_sequential(orc, seed=5):
    """The chunked parallel form (derived block algebra) reaches the sequential
    result for several chunk sizes, including a ragged last chunk."""
    rng = np.random.default_rng(seed)
    T, dk, dv = 200, 8, 6
    q, k, v, g, beta = _case(rng, T, 1, dk, dv)
    S0 = rng.standard_normal((1, 1, dk, dv)) * 0.1
    o, ht = orc.kda_forward(q, k, v, g, beta, h0=S0)
    for C in (1, 16, 37, 64):
        oc, Sc = chunked_forward(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0[0, 0], C)
        assert np.max(np.abs(oc - o[0, :, 0])) < 1e-12
        assert np.max(np.abs(Sc - ht[0, 0])) < 1e-12


def pin_superposition(orc, seed=6):
    """With q, k, g, beta fixed, the map (V, S_0) -> (o, S_T) is linear."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 12, 2, 4, 3
    q, k, v1, g, beta = _case(rng, T, H, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    S1 = rng.standard_normal((1, H, dk, dv))
    S2 = rng.standard_normal((1, H, dk, dv))
    o1, h1 = orc.kda_forward(q, k, v1, g, beta, h0=S1)
    o2, h2 = orc.kda_forward(q, k, v2, g, beta, h0=S2)
    o3, h3 = orc.kda_forward(q, k, v1 + 2.0 * v2, g, beta, h0=S1 + 2.0 * S2)
    assert np.max(np.abs(o3 - (o1 + 2.0 * o2))) < 1e-12
    assert np.max(np.abs(h3 - (h1 + 2.0 * h2))) < 1e-12


def pin_split_equivalence(orc, seed=7):
    """Running tokens [0, t) then [t, T) from the carried state equals one run."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 20, 2, 4, 4
    q, k, v, g, beta = _case(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, ht = orc.kda_forward(q, k, v, g, beta, h0=S0)
    for t in (1, 7, 13):
        sl = lambda x, a, b: x[:, a:b]
        oa, ha = orc.kda_forward(sl(q, 0, t), sl(k, 0, t), sl(v, 0, t), sl(g, 0, t), sl(beta, 0, t), h0=S0)
        ob, hb = orc.kda_forward(sl(q, t, T), sl(k, t, T), sl(v, t, T), sl(g, t, T), sl(beta, t, T), h0=ha)
        assert np.max(np.abs(np.concatenate([oa, ob], axis=1) - o)) < 1e-13
        assert np.max(np.abs(hb - ht)) < 1e-13


def pin_varlen_isolation(orc, seed=8):
    """Packed documents: the packed run equals separate runs, and a change (or a
    NaN) in one document leaves every other document exactly unchanged
    (Mini-K3-1H-mamba2 README: state flow reset at every document boundary)."""
    rng = np.random.default_rng(seed)
    lens = [5, 1, 9, 0, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = int(cu[-1]), 2, 4, 3
    q, k, v, g, beta = _case(rng, T, H, dk, dv)
    N = len(lens)
    h0 = rng.standard_normal((N, H, dk, dv))
    o, ht = orc.kda_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        if a == b:
            assert np.array_equal(ht[n], h0[n]), "an empty document must return its initial state"
            continue
        on, hn = orc.kda_forward(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], h0=h0[n:n + 1])
        assert np.array_equal(on, o[:, a:b]), "packed output differs from the separate run"
        assert np.array_equal(hn[0], ht[n])
    j = 2
    a, b = cu[j], cu[j + 1]
    v2 = v.copy()
    v2[:, a:b] += 1.0
    q2 = q.copy()
    q2[:, a + 1] = np.nan
    o2, ht2 = orc.kda_forward(q2, k, v2, g, beta, h0=h0, cu_seqlens=cu)
    mask = np.ones(T, bool)
    mask[a:b] = False
    assert np.array_equal(o2[:, mask], o[:, mask]), "a perturbed document leaked into another"
    others = [n for n in range(N) if n != j]
    assert np.array_equal(ht2[others], ht[others])


def pin_boundedness(orc, seed=9):
    """|k| = 1, beta in [0, 1], alpha in (0, 1]: ||S_t||_F <= ||S_0||_F +
    sum_i beta_i ||v_i|| (each transition is a contraction)."""
    rng = np.random.default_rng(seed)
    T, dk, dv = 300, 6, 4
    q, k, v, g, beta = _case(rng, T, 1, dk, dv, decay_shift=8.0)
    S0 = rng.standard_normal((1, 1, dk, dv))
    bound = np.linalg.norm(S0)
    for t in range(1, T + 1):
        _, ht = orc.kda_forward(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], h0=S0)
        bound_t = bound + np.sum(beta[0, :t, 0] * np.linalg.norm(v[0, :t, 0], axis=-1))
        assert np.linalg.norm(ht) <= bound_t + 1e-12
        if t > 40:
            break


def pin_decay_groups(orc, seed=13):
    """decay-g64: compact g (one value per 64-channel group) equals the same
    values repeated over their 64 channels with g_group = 1, and each value
    acts on its own 64 channels; with dk = 64 it is a scalar (head-wise) decay."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 10, 2, 128, 8
    q, k, v, _, beta = _case(rng, T, H, dk, dv)
    gc = -np.logaddexp(0.0, rng.standard_normal((1, T, H, dk // 64)) - 2.0)
    ge = np.concatenate([np.broadcast_to(gc[..., i:i + 1], (1, T, H, 64)) for i in range(dk // 64)], axis=-1)
    oc, hc = orc.kda_forward(q, k, v, gc, beta, g_group=64)
    oe, he = orc.kda_forward(q, k, v, ge, beta, g_group=1)
    assert np.array_equal(oc, oe) and np.array_equal(hc, he)
    # beta = 0 from a known state: channel block i decays by exp(sum of group i)
    S0 = rng.standard_normal((1, H, dk, dv))
    _, ht = orc.kda_forward(q, k, v, gc, np.zeros_like(beta), h0=S0, g_group=64)
    tot = gc[0].sum(axis=0)                          # [H, groups]
    for h in range(H):
        for i in range(dk // 64):
            blk = slice(64 * i, 64 * (i + 1))
            assert np.max(np.abs(ht[0, h, blk] - np.exp(tot[h, i]) * S0[0, h, blk])) < 1e-13


def pin_decode_is_one_step(orc, seed=14):
    """The decode step equals a length-1 forward from the same state."""
    rng = np.random.default_rng(seed)
    N, H, dk, dv = 3, 2, 8, 4
    q, k, v, g, beta = _case(rng, N, H, dk, dv)          # use the T axis as N
    S0 = rng.standard_normal((N, H, dk, dv))
    Sn, o = orc.kda_decode_step(S0, q[0], k[0], v[0], g[0], beta[0])
    tm = lambda x: x[0][:, None]
    of, hf = orc.kda_forward(tm(q), tm(k), tm(v), tm(g), tm(beta), h0=S0)
    assert np.max(np.abs(o - of[:, 0])) < 1e-14
    assert np.max(np.abs(Sn - hf)) < 1e-14


ALL_PINS = [
    pin_fd_gradient_step,
    pin_exact_replacement,
    pin_frozen_state,
    pin_linear_attention,
    pin_pure_decay,
    pin_brute_force,
    pin_chunked_equals_sequential,
    pin_superposition,
    pin_split_equivalence,
    pin_varlen_isolation,
    pin_boundedness,
    pin_decay_groups,
    pin_decode_is_one_step,
]
