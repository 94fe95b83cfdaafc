"""Planted mistakes in the prologue oracle (on the CPU): each plausible slip
in the gate, the activations or the normalisation must make at least one
prologue pin fail, so the pins constrain every step of the prologue."""

import numpy as np
import pytest

import oracle.prologue as pro
from tests import _prologue_pins as pins

f64 = lambda x: np.asarray(x, dtype=np.float64)

MUTANTS = {
    # the gate
    "gate_positive": ("gate", lambda f, A, d: np.exp(f64(A)) * pro.softplus(f64(f) + f64(d))),
    "gate_without_exp": ("gate", lambda f, A, d: -f64(A) * pro.softplus(f64(f) + f64(d))),
    "gate_bias_outside_softplus": ("gate", lambda f, A, d: -np.exp(f64(A)) * (pro.softplus(f64(f)) + f64(d))),
    "gate_without_softplus": ("gate", lambda f, A, d: -np.exp(f64(A)) * (f64(f) + f64(d))),
    # the activations
    "softplus_as_relu": ("softplus", lambda x: np.maximum(f64(x), 0.0)),
    "softplus_as_exp": ("softplus", lambda x: np.exp(f64(x))),
    "sigmoid_as_tanh": ("sigmoid", lambda x: np.tanh(f64(x))),
    "beta_unsquashed": ("sigmoid", lambda x: f64(x)),
    # the normalisation
    "norm_over_tokens": ("l2_normalize",
                         lambda x, eps=pro.EPS: f64(x) / np.sqrt(np.sum(f64(x) ** 2, axis=0, keepdims=True) + eps)),
    "norm_without_sqrt": ("l2_normalize",
                          lambda x, eps=pro.EPS: f64(x) / (np.sum(f64(x) ** 2, axis=-1, keepdims=True) + eps)),
    "norm_without_guard": ("l2_normalize",
                           lambda x, eps=pro.EPS: f64(x) / np.sqrt(np.sum(f64(x) ** 2, axis=-1, keepdims=True))),
    "norm_l1": ("l2_normalize", lambda x, eps=pro.EPS: f64(x) / (np.sum(np.abs(f64(x)), axis=-1, keepdims=True) + eps)),
}


def _fails_a_pin():
    failed = []
    for pin in pins.ALL:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            failed.append(pin.__name__)
    return failed


def test_pins_pass_on_the_oracle():
    assert _fails_a_pin() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(pro, attr, fn)
    failed = _fails_a_pin()
    print("mutant %s fails: %s" % (name, ", ".join(failed)))
    assert failed, name
