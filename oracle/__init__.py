"""fp64 CPU oracle of the PACK3D operator.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py``, never by
the product path.  See ``pack3d_oracle.py``.
"""
from .pack3d_oracle import *  # noqa: F401,F403
