"""fp64 CPU oracle for exact attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  The product path (the HIP library and its
Python binding) never imports it and shares no code with it.
"""
from .attention import *  # noqa: F401,F403
from .attention import __all__  # noqa: F401
