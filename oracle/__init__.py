"""CPU oracle for the packed audio-video DiT block -- TEST INFRASTRUCTURE ONLY.

Plain, slow float64 numpy code written from the definitions of each step.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the GPU path and imports
nothing from it; the only module both sides use is ``workloads`` (seeded input
draws, no arithmetic of the method).
"""
from .h3_oracle import *  # noqa: F401,F403
