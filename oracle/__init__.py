"""CPU oracle for the int4 routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run anything here.  The
GPU library never calls it, and it shares no code with the GPU library.
"""
from .moe_oracle import *  # noqa: F401,F403
