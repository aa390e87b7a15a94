"""The CPU oracle: test infrastructure, not part of the library.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP path.
"""

from .qmm_oracle import *  # noqa: F401,F403
