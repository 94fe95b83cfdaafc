"""Pins of the prologue's backward in the oracle (CPU only), and planted
mistakes that each fail one of them.

* directional finite differences of L = <do, o> + <dht, ht> through the
  prologue and the recurrence, for every input and parameter (q_raw, k_raw,
  v, f, b_raw, A_log, dt_bias, h0), per channel and with decay groups;
* the gradient of an L2-normalised row is orthogonal to the raw row and
  scales as 1/c when the raw row is scaled by c;
* the gate's derivative at f + dt_bias = 0 (sigmoid 1/2, softplus ln 2) and
  its vanishing for a strongly negative argument;
* the write gate's derivative at b = 0 and b = ln 3 (beta = 1/2 and 3/4).
"""

import numpy as np
import pytest

import oracle.prologue as pro


def _case(rng, B=2, T=9, H=2, dk=4, dv=3, gg=1):
    scale = np.exp(rng.uniform(np.log(0.5), np.log(4.0), (B, T, H, 1)))
    return dict(
        q_raw=rng.standard_normal((B, T, H, dk)) * scale,
        k_raw=rng.standard_normal((B, T, H, dk)) * scale,
        v=rng.standard_normal((B, T, H, dv)),
        f=rng.standard_normal((B, T, H, dk // gg)),
        b_raw=rng.standard_normal((B, T, H)),
        A_log=0.5 + 0.3 * rng.standard_normal((H, dk // gg)),
        dt_bias=-1.0 + 0.3 * rng.standard_normal((H, dk // gg)),
        h0=0.3 * rng.standard_normal((B, H, dk, dv)),
    )


def _loss(c, do, dht, gg):
    o, ht = pro.kda_forward_prologue(c["q_raw"], c["k_raw"], c["v"], c["f"], c["b_raw"], c["A_log"], c["dt_bias"],
                                     h0=c["h0"], g_group=gg)
    return float(np.sum(do * o) + np.sum(dht * ht))


GRAD = dict(q_raw="dq_raw", k_raw="dk_raw", v="dv", f="df", b_raw="db_raw", A_log="dA_log", dt_bias="ddt_bias",
            h0="dh0")


def pin_finite_differences():
    for gg in (1, 2):
        rng = np.random.default_rng(500 + gg)
        c = _case(rng, gg=gg)
        do = rng.standard_normal(c["v"].shape)
        dht = rng.standard_normal(c["h0"].shape)
        gr = pro.kda_backward_prologue(c["q_raw"], c["k_raw"], c["v"], c["f"], c["b_raw"], c["A_log"],
                                       c["dt_bias"], do, h0=c["h0"], dht=dht, g_group=gg)
        eps = 1e-6
        for name, gname in GRAD.items():
            for _ in range(2):
                d = rng.standard_normal(c[name].shape)
                plus, minus = dict(c), dict(c)
                plus[name] = c[name] + eps * d
                minus[name] = c[name] - eps * d
                fd = (_loss(plus, do, dht, gg) - _loss(minus, do, dht, gg)) / (2 * eps)
                an = float(np.sum(gr[gname] * d))
                assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (gg, name, fd, an)


def pin_normalisation_gradient():
    rng = np.random.default_rng(510)
    x = rng.standard_normal((7, 5)) * 3.0
    dy = rng.standard_normal((7, 5))
    dx = pro.l2_normalize_backward(x, dy)
    cosine = np.sum(x * dx, axis=-1) / (np.linalg.norm(x, axis=-1) * np.linalg.norm(dx, axis=-1))
    assert np.max(np.abs(cosine)) <= 1e-6
    for c in (0.5, 8.0):
        assert np.allclose(pro.l2_normalize_backward(c * x, dy), dx / c, rtol=1e-5, atol=0)


def pin_gate_derivative():
    A = np.array([[0.0, np.log(16.0)]])
    bias = np.array([[0.7, -2.0]])
    f = -bias[None].repeat(3, 0)                      # f + dt_bias = 0: sigmoid 1/2, softplus ln 2
    dg = np.array([[[1.0, 2.0]], [[-1.0, 0.5]], [[3.0, 1.0]]])
    z = np.zeros((3, 1, 2))
    out = pro.prologue_backward(z, z, f, np.zeros((3, 1)), A, bias, z, z, dg, np.zeros((3, 1)))
    assert np.allclose(out["df"], -np.exp(A) * 0.5 * dg, rtol=1e-14, atol=0)
    assert np.allclose(out["ddt_bias"], np.sum(-np.exp(A) * 0.5 * dg, axis=0), rtol=1e-14, atol=0)
    assert np.allclose(out["dA_log"], np.sum(dg, axis=0) * (-np.exp(A) * np.log(2.0)), rtol=1e-14, atol=0)
    far = pro.prologue_backward(z, z, f - 80.0, np.zeros((3, 1)), A, bias, z, z, dg, np.zeros((3, 1)))
    assert np.max(np.abs(far["df"])) <= 16.0 * 3.0 * np.exp(-79.0)


def pin_write_gate_derivative():
    b = np.array([[0.0, np.log(3.0)]])
    dbeta = np.array([[2.0, 16.0]])
    z = np.zeros((1, 2, 1))
    out = pro.prologue_backward(z, z, z, b, np.zeros((2, 1)), np.zeros((2, 1)), z, z, z, dbeta)
    assert np.allclose(out["db_raw"], [[0.5, 3.0]], rtol=1e-14, atol=0)


PINS = [pin_finite_differences, pin_normalisation_gradient, pin_gate_derivative, pin_write_gate_derivative]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_prologue_backward_pin(pin):
    pin()


# ---------------------------------------------------------------- planted mistakes
_real = pro.prologue_backward


def _mutant(change):
    def fn(q_raw, k_raw, f, b_raw, A_log, dt_bias, dq, dk, dg, dbeta):
        out = _real(q_raw, k_raw, f, b_raw, A_log, dt_bias, dq, dk, dg, dbeta)
        return change(out, locals())
    return fn


def _sum_lead(x):
    x = np.asarray(x, dtype=np.float64)
    return np.sum(x, axis=tuple(range(x.ndim - 2)))


MUTANTS = {
    "norm_grad_without_projection": ("l2_normalize_backward",
                                     lambda x, dy, eps=pro.EPS: np.asarray(dy) / np.sqrt(
                                         np.sum(np.asarray(x) ** 2, axis=-1, keepdims=True) + eps)),
    "norm_grad_cubed_scale": ("l2_normalize_backward",
                              lambda x, dy, eps=pro.EPS: (lambda r: r ** 3 * (np.asarray(dy) - np.asarray(x) * r * np.sum(
                                  np.asarray(x) * r * np.asarray(dy), axis=-1, keepdims=True)))(
                                  1.0 / np.sqrt(np.sum(np.asarray(x) ** 2, axis=-1, keepdims=True) + eps))),
    "gate_grad_sign": ("prologue_backward", _mutant(lambda o, a: dict(o, df=-o["df"], ddt_bias=-o["ddt_bias"]))),
    "A_log_grad_without_g": ("prologue_backward", _mutant(lambda o, a: dict(o, dA_log=_sum_lead(a["dg"])))),
    "dt_bias_grad_unchained": ("prologue_backward", _mutant(lambda o, a: dict(o, ddt_bias=_sum_lead(a["dg"])))),
    "write_gate_grad_unchained": ("prologue_backward", _mutant(lambda o, a: dict(o, db_raw=np.asarray(a["dbeta"])))),
}


def _failing_pins():
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(pro, attr, fn)
    failed = _failing_pins()
    print("mutant %s fails: %s" % (name, ", ".join(failed)))
    assert failed, name
