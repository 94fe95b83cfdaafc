"""The prologue oracle against closed forms and invariants (CPU only).

Pins (tests/_prologue_pins.py):
* softplus and sigmoid at points where their values are known exactly or
  to textbook limits;
* normalised rows have unit norm, the prologue is invariant to a positive
  rescaling of the raw q and k, and an all-zero row stays zero;
* the gate is <= 0 and reproduces a chosen log-decay through the inverse
  softplus;
* with prepared inputs built from a known (q, k, g, beta), the prologue
  forward and decode step equal the plain ones on those values.
"""

import pytest

from tests import _prologue_pins as pins


@pytest.mark.parametrize("pin", pins.ALL, ids=lambda p: p.__name__)
def test_prologue_pin(pin):
    pin()
