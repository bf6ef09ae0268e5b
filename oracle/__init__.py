"""CPU oracle for the CSA/HCA attention forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never calls it.
"""
from .lcs_oracle import *  # noqa: F401,F403
