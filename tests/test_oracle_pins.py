"""The CPU oracle against what the pages and the mathematics fix (CPU only)."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.kda_oracle as orc
from oracle.brute import brute_force
from tests import _oracle_pins as pins
from tests._oracle_pins import oracle_on_rational

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(orc)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        d = json.load(f)
    dec = lambda m: [[Fraction(x) for x in row] for row in m]
    return d, dec


@pytest.mark.parametrize("name", ["worked_d2_t3.json", "rational_d3_t5.json"])
def test_golden_fixture(name):
    """Exact-rational fixtures written by tests/golden/make_golden.py.
    worked_d2_t3.json was also checked by hand, token by token, against the
    matrix form of the KDA update (decay, erase-and-write, read-out)."""
    d, dec = _load(name)
    case = [dec(d["q"]), dec(d["k"]), dec(d["v"]), dec(d["alpha"]), [Fraction(b) for b in d["beta"]], dec(d["S0"])]
    o, ht = oracle_on_rational(orc, *case)
    o_ref = np.array([[float(x) for x in row] for row in dec(d["o"])])
    S_ref = np.array([[float(x) for x in row] for row in dec(d["S_final"])])
    assert np.max(np.abs(o - o_ref)) < 1e-13
    assert np.max(np.abs(ht - S_ref)) < 1e-13
    # and the fixture is still what the exact brute force gives
    o_ex, S_ex = brute_force(*case)
    assert [[str(x) for x in r] for r in o_ex] == d["o"]


def test_worked_example_values():
    """The worked example's exact values (hand-derived): token 0 is an exact
    replacement under key e_1, so o_0 = v_0."""
    d, dec = _load("worked_d2_t3.json")
    assert d["o"][0] == ["2", "-1"]
    assert d["o"][1] == ["11/10", "0"]
    assert d["S_final"] == [["291/200", "-3/10"], ["37/100", "363/160"]]
