"""CPU float64 oracle of the MoE layer hot path -- test infrastructure, never the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
import this package. It shares no code with the HIP library.
"""
from . import moe_oracle  # noqa: F401
from .moe_oracle import *  # noqa: F401,F403
