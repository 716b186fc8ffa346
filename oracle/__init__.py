"""CPU oracle for the ConvRot W8A8 INT8 linear -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``w8a8_int8_rotated_amd`` and neither imports the other.
"""
from .oracle import *  # noqa: F401,F403
