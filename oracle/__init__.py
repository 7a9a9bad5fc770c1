"""Test infrastructure: the fp64 CPU oracle for batched speculative-sampling verification.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import anything from this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it.
"""
from .spec_oracle import *  # noqa: F401,F403
