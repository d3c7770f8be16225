"""CPU oracle for Monodratic routed sparse causal attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the HIP library or its
Python binding.  Every function states the passage of the method it follows.
"""

from .mdr_oracle import *  # noqa: F401,F403
