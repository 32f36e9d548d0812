"""fp64 CPU oracle of the MLA decode step -- test infrastructure only.

Importable by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``; never by the GPU library or its binding.
"""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import gather_rows  # noqa: F401
