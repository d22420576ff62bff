"""Plain CPU oracle for the CubicQuant dequant-GEMM path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
HIP library never links, imports or calls it, and shares no code with it.
"""
from .cubic_oracle import *  # noqa: F401,F403
