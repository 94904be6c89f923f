"""CPU oracle for Sliding Tile Attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does.
"""
from .sta_oracle import *  # noqa: F401,F403
