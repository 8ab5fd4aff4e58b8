"""Float64 CPU oracle for the KATA causal linear-attention forward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
HIP product path never imports it, and this package imports nothing from the
HIP path.
"""
from .kata_oracle import *  # noqa: F401,F403
