"""fp64 CPU oracle of the top-k MoE layer forward.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library never
imports or calls it, and it shares no code with the GPU library.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision); this module
builds it with gcc, loads it with ctypes and converts numpy/torch-CPU arrays.
"""
from .oracle import (  # noqa: F401
    Oracle,
    build_oracle,
    default_oracle,
    ORACLE_SOURCE,
)
