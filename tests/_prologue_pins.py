"""Pins of the prologue oracle (closed forms and invariants), as callable
checks: each raises AssertionError when the oracle breaks it.  Used by
test_oracle_prologue.py, and by test_oracle_prologue_mutants.py to show
that planted mistakes fail them."""

import numpy as np

import oracle.kda_oracle as orc
import oracle.prologue as pro


def pin_activations():
    """softplus and sigmoid at values fixed by their definitions."""
    assert abs(pro.softplus(0.0) - np.log(2.0)) < 1e-15
    assert abs(pro.softplus(50.0) - 50.0) < 1e-15  # log(1 + e^50) = 50 + log(1 + e^-50)
    assert abs(pro.softplus(-50.0) - np.exp(-50.0)) < 1e-30
    assert pro.sigmoid(0.0) == 0.5
    x = np.linspace(-5, 5, 11)
    assert np.allclose(pro.sigmoid(x) + pro.sigmoid(-x), 1.0, atol=1e-15)
    assert np.allclose(pro.softplus(x) - pro.softplus(-x), x, atol=1e-14)  # softplus(x) - softplus(-x) = x


def pin_normalisation():
    """Rows come out with unit norm along the channel axis, invariant to a
    positive rescaling of each row; an all-zero row stays zero (the guard)."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 3, 16)) * rng.uniform(0.5, 20, (7, 3, 1))
    n = pro.l2_normalize(x)
    assert np.allclose(np.linalg.norm(n, axis=-1), 1.0, atol=1e-8)
    assert np.allclose(pro.l2_normalize(3.5 * x), n, atol=1e-9)
    z = pro.l2_normalize(np.zeros((2, 16)))
    assert np.all(np.isfinite(z)) and np.all(z == 0.0)


def pin_gate_inversion():
    """The gate is <= 0 and reproduces a chosen log-decay through the
    inverse softplus: softplus(y) = s <=> y = log(expm1(s))."""
    rng = np.random.default_rng(1)
    H, dk = 2, 8
    A_log = rng.normal(0, 0.3, (H, dk))
    dt_bias = rng.normal(-2, 0.3, (H, dk))
    g_want = -rng.uniform(0.01, 2.0, (5, H, dk))
    f = np.log(np.expm1(-g_want / np.exp(A_log))) - dt_bias
    g = pro.gate(f, A_log, dt_bias)
    assert np.all(g <= 0)
    assert np.allclose(g, g_want, rtol=1e-12, atol=1e-14)


def _prepared(seed=2, gg=4):
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 40, 2, 8, 4
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)  # not the oracle's own normalisation
    q = unit(rng.standard_normal((B, T, H, dk)))
    k = unit(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    g = -rng.uniform(0.01, 1.0, (B, T, H, dk // gg))
    A_log = rng.normal(0, 0.3, (H, dk // gg))
    dt_bias = rng.normal(-2, 0.3, (H, dk // gg))
    f = np.log(np.expm1(-g / np.exp(A_log))) - dt_bias
    b_raw = np.log(beta / (1 - beta))
    return q, k, v, beta, g, A_log, dt_bias, f, b_raw, rng


def pin_forward_on_prepared_inputs():
    """Raw inputs built from a known (q, k, g, beta) (rows rescaled, gate and
    beta inverted) give the plain forward's result on those values."""
    gg = 4
    q, k, v, beta, g, A_log, dt_bias, f, b_raw, rng = _prepared(gg=gg)
    scale = rng.uniform(0.3, 5.0, q.shape[:-1] + (1,))
    o1, h1 = pro.kda_forward_prologue(q * scale, k * scale, v, f, b_raw, A_log, dt_bias, g_group=gg)
    o2, h2 = orc.kda_forward(q, k, v, g, beta, g_group=gg)
    # the eps guard moves a row of norm s by eps / (2 s^2) relative (<= 6e-6 here)
    assert np.max(np.abs(o1 - o2)) < 1e-4 and np.max(np.abs(h1 - h2)) < 1e-4
    o3, h3 = pro.kda_forward_prologue(q, k, v, f, b_raw, A_log, dt_bias, g_group=gg)
    assert np.max(np.abs(o3 - o2)) < 1e-5 and np.max(np.abs(h3 - h2)) < 1e-5


def pin_decode_on_prepared_inputs():
    """The same for one decode step from a random state."""
    gg = 4
    q, k, v, beta, g, A_log, dt_bias, f, b_raw, rng = _prepared(seed=3, gg=gg)
    sl = lambda t: t[0, :5]  # five "sequences" = the first five tokens
    S0 = 0.1 * rng.standard_normal((5, q.shape[2], q.shape[3], v.shape[3]))
    S1, o1 = pro.kda_decode_step_prologue(S0, sl(q) * 2.0, sl(k) * 0.5, sl(v), sl(f), sl(b_raw), A_log, dt_bias,
                                          g_group=gg)
    S2, o2 = orc.kda_decode_step(S0, sl(q), sl(k), sl(v), sl(g), sl(beta), g_group=gg)
    assert np.max(np.abs(o1 - o2)) < 1e-5 and np.max(np.abs(S1 - S2)) < 1e-5


ALL = [pin_activations, pin_normalisation, pin_gate_inversion, pin_forward_on_prepared_inputs,
       pin_decode_on_prepared_inputs]
