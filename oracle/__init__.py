"""CPU oracle for KDA -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""

from .kda_oracle import expand_decay, kda_step, kda_sequence, kda_forward, kda_decode_step  # noqa: F401
