"""The prologue oracle against closed forms and invariants (CPU only).

Pins:
* softplus and sigmoid at points where their values are known exactly or
  to textbook limits;
* normalised rows have unit norm, and the prologue is invariant to a
  positive rescaling of the raw q and k;
* the gate is <= 0 and reproduces a chosen log-decay through the inverse
  softplus;
* with prepared inputs built from a known (q, k, g, beta), the prologue
  forward equals the plain forward on those values.
"""

import numpy as np

import oracle.kda_oracle as orc
import oracle.prologue as pro


def test_softplus_sigmoid_closed_forms():
    assert abs(pro.softplus(0.0) - np.log(2.0)) < 1e-15
    assert abs(pro.softplus(50.0) - 50.0) < 1e-15  # log(1 + e^50) = 50 + log(1 + e^-50)
    assert abs(pro.softplus(-50.0) - np.exp(-50.0)) < 1e-30
    assert pro.sigmoid(0.0) == 0.5
    x = np.linspace(-5, 5, 11)
    assert np.allclose(pro.sigmoid(x) + pro.sigmoid(-x), 1.0, atol=1e-15)
    # softplus(x) - softplus(-x) = x
    assert np.allclose(pro.softplus(x) - pro.softplus(-x), x, atol=1e-14)


def test_normalisation_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 3, 16)) * rng.uniform(0.5, 20, (7, 3, 1))
    n = pro.l2_normalize(x)
    assert np.allclose(np.linalg.norm(n, axis=-1), 1.0, atol=1e-8)
    assert np.allclose(pro.l2_normalize(3.5 * x), n, atol=1e-9)


def test_gate_inverts_to_a_chosen_decay():
    rng = np.random.default_rng(1)
    H, dk = 2, 8
    A_log = rng.normal(0, 0.3, (H, dk))
    dt_bias = rng.normal(-2, 0.3, (H, dk))
    g_want = -rng.uniform(0.01, 2.0, (5, H, dk))
    # softplus(y) = s  <=>  y = log(expm1(s))
    f = np.log(np.expm1(-g_want / np.exp(A_log))) - dt_bias
    g = pro.gate(f, A_log, dt_bias)
    assert np.all(g <= 0)
    assert np.allclose(g, g_want, rtol=1e-12, atol=1e-14)


def test_prologue_forward_equals_plain_forward_on_prepared_inputs():
    rng = np.random.default_rng(2)
    B, T, H, dk, dv, gg = 1, 40, 2, 8, 4, 4
    q = pro.l2_normalize(rng.standard_normal((B, T, H, dk)))
    k = pro.l2_normalize(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    g = -rng.uniform(0.01, 1.0, (B, T, H, dk // gg))
    A_log = rng.normal(0, 0.3, (H, dk // gg))
    dt_bias = rng.normal(-2, 0.3, (H, dk // gg))
    f = np.log(np.expm1(-g / np.exp(A_log))) - dt_bias
    b_raw = np.log(beta / (1 - beta))
    scale = rng.uniform(0.3, 5.0, (B, T, H, 1))
    o1, h1 = pro.kda_forward_prologue(q * scale, k * scale, v, f, b_raw, A_log, dt_bias, g_group=gg)
    o2, h2 = orc.kda_forward(q, k, v, g, beta, g_group=gg)
    # the eps guard moves a row of norm s by eps / (2 s^2) relative (<= 6e-6 here)
    assert np.max(np.abs(o1 - o2)) < 1e-4 and np.max(np.abs(h1 - h2)) < 1e-4
    o3, h3 = pro.kda_forward_prologue(q, k, v, f, b_raw, A_log, dt_bias, g_group=gg)
    assert np.max(np.abs(o3 - o2)) < 1e-5 and np.max(np.abs(h3 - h2)) < 1e-5
