"""CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package. The library and its binding
never do.
"""
from .mcsparse_ref import *  # noqa: F401,F403
from .mcsparse_ref import __all__  # noqa: F401
