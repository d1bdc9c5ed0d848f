"""CPU oracle for the OSCAR INT2-history decode path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package; the HIP library neither imports it nor shares code with it.
"""
from .oscar_oracle import *  # noqa: F401,F403
from .oscar_oracle import Geometry  # noqa: F401
