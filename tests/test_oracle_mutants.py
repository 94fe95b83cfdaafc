"""Planted mistakes in the oracle (on the CPU): every plausible mistake --
a dropped term, a wrong sign, a wrong axis or order, a transposed operand --
must make at least one pin fail.  This shows the pins constrain the oracle."""

import numpy as np
import pytest

import oracle.kda_oracle as orc
from tests import _oracle_pins as pins

_real_step = orc.kda_step
_real_forward = orc.kda_forward


def _step(decay_axis="rows", decay_sign=1.0, order="decay_first", erase_from="decayed",
          beta_scale=1.0, beta_on_erase=True, sign=1.0, read="post", transpose_read=False, erase=True):
    def step(S, q, k, v, g, beta):
        alpha = np.exp(decay_sign * g)
        dec = (lambda M: alpha[..., :, None] * M) if decay_axis == "rows" else (lambda M: alpha[..., None, :] * M)
        S_in = dec(S) if order == "decay_first" else S
        src = S_in if erase_from == "decayed" else S
        e = np.matmul(k[..., None, :], src)[..., 0, :] if erase else 0.0 * v
        b = beta_scale * beta
        if beta_on_erase:
            upd = b[..., None, None] * (k[..., :, None] * (v - e)[..., None, :])
        else:
            upd = k[..., :, None] * (b[..., None] * v - e)[..., None, :]
        S_new = S_in + sign * upd
        if order == "write_first":
            S_new = dec(S_new)
        R = S_in if read == "pre" else S_new
        if transpose_read:
            o = np.matmul(R, q[..., :, None])[..., :, 0]
        else:
            o = np.matmul(q[..., None, :], R)[..., 0, :]
        return S_new, o
    return step


STEP_MUTANTS = {
    "write_then_decay": _step(order="write_first"),
    "decay_on_value_axis": _step(decay_axis="cols"),
    "inverse_decay": _step(decay_sign=-1.0),
    "erase_from_undecayed_state": _step(erase_from="raw"),
    "literal_squared_norm_step": _step(beta_scale=2.0),
    "beta_only_on_value": _step(beta_on_erase=False),
    "wrong_sign_of_write": _step(sign=-1.0),
    "read_before_write": _step(read="pre"),
    "transposed_read": _step(transpose_read=True),
    "no_erase_term": _step(erase=False),
}


def _any_pin_fails():
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except Exception:  # an assertion, or a shape error from a wrong axis
            failed.append(pin.__name__)
    return failed


def test_real_oracle_passes_all():
    assert _any_pin_fails() == []


@pytest.mark.parametrize("name", sorted(STEP_MUTANTS))
def test_step_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(orc, "kda_step", STEP_MUTANTS[name])
    assert _any_pin_fails(), "planted mistake %r passed every pin" % name


def test_group_expansion_mutant_is_caught(monkeypatch):
    def tiled(g, dk, g_group):
        g = np.asarray(g, dtype=np.float64)
        return g if g_group == 1 else np.tile(g, (1,) * (g.ndim - 1) + (g_group,))
    monkeypatch.setattr(orc, "expand_decay", tiled)
    assert _any_pin_fails()


def test_no_document_reset_mutant_is_caught(monkeypatch):
    def carry(q, k, v, g, beta, h0=None, cu_seqlens=None, g_group=1):
        if cu_seqlens is None:
            return _real_forward(q, k, v, g, beta, h0=h0, g_group=g_group)
        cu = np.asarray(cu_seqlens)
        o, _ = _real_forward(q, k, v, g, beta, h0=None if h0 is None else h0[:1], g_group=g_group)
        N = len(cu) - 1
        ht = np.repeat(_real_forward(q, k, v, g, beta, h0=None if h0 is None else h0[:1],
                                     g_group=g_group)[1], N, axis=0)
        return o, ht
    monkeypatch.setattr(orc, "kda_forward", carry)
    assert _any_pin_fails()
