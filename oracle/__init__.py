"""CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The HIP path never imports or calls it.
"""
from .sp_oracle import *  # noqa: F401,F403
from .sp_oracle import __all__  # noqa: F401
