"""Plain fp64 CPU oracle for the Locks decode path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.
"""

from .locks_oracle import *  # noqa: F401,F403
