"""CPU oracle (test infrastructure only): see ``oracle/paged_oracle.py``.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package. The product path never does.
"""
from .paged_oracle import *  # noqa: F401,F403
