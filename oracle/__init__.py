"""CPU oracle for WavePrune attention -- test infrastructure only.

Importable by tests/, ``__graft_entry__.smoke()`` and bench.py's cpu_baseline
leg; never by the library.  See oracle/waveprune.py.
"""
from .waveprune import *  # noqa: F401,F403
from .waveprune import INT32_MAX, NEVER, SKIP, PARTIAL, FULL  # noqa: F401
