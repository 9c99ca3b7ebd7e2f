"""CPU oracle for the W4A8 linear / MoE-expert path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
"""
from .w4a8_oracle import *  # noqa: F401,F403
