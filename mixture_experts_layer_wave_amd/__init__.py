"""MI355X (gfx950) top-k Mixture-of-Experts layer forward.

The compute path is the HIP library ``libmoe_mi355x.so`` built from ``csrc/`` with the C
ABI declared in ``include/moe.h``; ``binding`` is a thin ctypes layer over it with the
same function names. ``configs`` and ``inputs`` describe and draw the synthetic
workloads. Importing this package loads nothing native; the library is loaded on first
use of ``binding`` and a missing library is an error, never a fallback.
"""

__all__ = ["binding", "configs", "inputs"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
