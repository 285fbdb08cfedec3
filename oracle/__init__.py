"""CPU oracle for the SparsePR per-call sparse attention operator.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never calls it and shares no code with it.
"""
from .sparsepr_ref import *  # noqa: F401,F403
