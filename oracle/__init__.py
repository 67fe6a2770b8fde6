"""CPU oracle (test infrastructure only; never imported by the library).

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.
"""
from .kv_oracle import *  # noqa: F401,F403
