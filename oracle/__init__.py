"""CPU oracle of the sparse MoE layer (test infrastructure only).

Importable by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` -- never by the product path.
"""
from . import moe_oracle  # noqa: F401
from .moe_oracle import *  # noqa: F401,F403
