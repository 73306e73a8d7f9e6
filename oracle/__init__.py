"""CPU oracle for the DiT block forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The HIP library never calls it and shares no code with it.
"""

from .dit_oracle import *  # noqa: F401,F403
