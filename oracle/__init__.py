"""CPU oracle for OSCAR-style 2-bit KV demotion and tiered decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The product path (the HIP library and its Python binding) never does, and
this package imports nothing from the product package.
"""
from .oscar_oracle import *  # noqa: F401,F403
